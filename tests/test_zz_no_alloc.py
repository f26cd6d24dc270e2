"""k2_block_forward_static_ws (the block forward that allocates nothing, its scratch a static device
array) against k2_block_forward on the same inputs, through the C ABI: two calls in a row, the second
smaller than the first, each bit-identical to the workspace entry point (same kernels, same order),
and the first also within the bf16 parity bounds of the oracle. The static scratch keeps the first
call's contents when the second runs."""
import numpy as np
import pytest

from flow_matching_diffusion_amd import synth as S
from oracle import k2_oracle as O
from tests.k2_testutil import device, gpu_block, parity, temb_for, workload

pytestmark = pytest.mark.gpu


def _static(wl, inp, temb, dev):
    import torch
    import flow_matching_diffusion_amd as k2
    cfg = k2.block_cfg(wl.dims, wl.dtype)
    w = k2.upload(inp["weights"], wl.dtype, dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = k2.block_forward_static_ws(cfg, w, t(inp["h"]), t(temb.astype(np.float32)), t(inp["position_ids"]),
                                     None if inp["mask"] is None else t(inp["mask"]), wl.T)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_static_scratch_matches_workspace_entry_point_twice():
    dev = device()
    big = workload("block512")                                    # 123.3 MiB of the 128 MiB scratch
    dims = S.BlockDims(hidden=512, num_heads=4, num_kv_heads=1, head_dim=128, intermediate=1024,
                       axes_dims=(32, 48, 48))
    small = S.Workload("static_small", 160, "bf16", 2, 12, (11, 9), (12, 3), dims=dims)
    for i, wl in enumerate((big, small)):
        inp = S.block_inputs(wl)
        temb = temb_for(wl, inp)
        got = _static(wl, inp, temb, dev)
        ref = gpu_block(wl, inp, temb)
        print(f"static-scratch call {i + 1} ({wl.name}, B={wl.B}, L={wl.L}): "
              f"max |static - workspace| = {np.abs(got - ref).max():.3e}", flush=True)
        np.testing.assert_array_equal(got, ref)
        if i == 1:
            fn = lambda rnd: O.block_forward(inp["h"], temb, inp["position_ids"], inp["mask"], inp["weights"],
                                             wl.dims, wl.T, rnd=rnd)
            parity(f"static-scratch {wl.name}", wl.dtype, got, fn)
