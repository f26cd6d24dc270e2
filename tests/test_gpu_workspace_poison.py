"""Workspace poisoning: every entry point that takes a workspace must write each scratch byte it reads
before reading it. The same call runs with the workspace filled with 0x00 bytes and with 0xFF bytes
(NaN in float32 and bf16); the outputs must be bit-identical and finite. A read of unwritten scratch
would carry the fill value into the output."""
import ctypes

import numpy as np
import pytest

from flow_matching_diffusion_amd import synth as S
from oracle import k2_oracle as O
from tests.k2_testutil import device, temb_for

pytestmark = pytest.mark.gpu

DIMS = S.BlockDims(hidden=512, num_heads=4, num_kv_heads=1, head_dim=128, intermediate=1024, axes_dims=(32, 48, 48))


def _filled(nbytes, byte, dev):
    import torch
    return torch.full((max(nbytes, 1),), byte, dtype=torch.uint8, device=dev)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_block_forward_and_backward_ignore_workspace_contents(dt):
    import torch
    import flow_matching_diffusion_amd as k2
    dev = device()
    wl = S.Workload("poison", 150, dt, 2, 12, (11, 9), (12, 3), dims=DIMS)
    inp = S.block_inputs(wl)
    temb = temb_for(wl, inp)
    cfg = k2.block_cfg(wl.dims, dt)
    w = k2.upload(inp["weights"], dt, dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h, tb, pos, mask = t(inp["h"]), t(temb.astype(np.float32)), t(inp["position_ids"]), t(inp["mask"])
    gout = t(np.random.default_rng(3).standard_normal(inp["h"].shape).astype(np.float32))
    nf = k2.load().k2_block_workspace_bytes(ctypes.byref(cfg), wl.B, wl.T, wl.N)
    nb = k2.block_backward_workspace_bytes(cfg, wl.B, wl.T, wl.N)
    ids = t(np.concatenate([np.full(wl.T, -1), np.zeros(40), np.ones(wl.N - 40)]).astype(np.int32))
    res = []
    for byte in (0x00, 0xFF):
        fw = k2.block_forward(cfg, w, h, tb, pos, mask, wl.T, workspace=_filled(nf, byte, dev))
        bc = k2.block_forward(cfg, w, h, tb, pos, mask, wl.T, workspace=_filled(nf, byte, dev), image_ids=ids)
        gi, gt, gw = k2.block_backward(cfg, w, h, tb, pos, mask, wl.T, gout, workspace=_filled(nb, byte, dev))
        torch.cuda.synchronize()
        res.append([fw.cpu().numpy(), bc.cpu().numpy(), gi.cpu().numpy(), gt.cpu().numpy()] +
                   [gw[k].cpu().numpy() for k in sorted(gw)])
    for a, b in zip(*res):
        assert np.all(np.isfinite(a))
        np.testing.assert_array_equal(a, b)


def test_backbone_ignores_workspace_contents():
    import torch
    import flow_matching_diffusion_amd as k2
    dev = device()
    td = S.TextDims(hidden=256, num_heads=2, num_kv_heads=2, head_dim=128, intermediate=320, num_layers=3)
    d = S.BlockDims(hidden=256, num_heads=4, num_kv_heads=2, head_dim=64, intermediate=200, axes_dims=(16, 24, 24))
    wl = S.Workload("poisonbb", 151, "bf16", 2, 9, (6, 5), (9, 4), t=(0.7, 0.3), dims=d, text=td, num_layers=2,
                    in_channels=64)
    mw = k2.upload(S.model_weights(wl.seed, wl), "bf16", dev)
    inp = S.backbone_inputs(wl)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    cfg = k2.model_cfg(wl.dims, td, wl.num_layers, wl.in_channels, wl.timestep_embed_dim, "bf16")
    x = t(S.as_dtype(inp["x"], "bf16")).to(torch.bfloat16)
    enc = t(inp["enc"]).to(torch.bfloat16)
    n = k2.backbone_workspace_bytes(cfg, wl.B, wl.T, wl.N)
    outs = []
    for byte in (0x00, 0xFF):
        v = k2.backbone_forward(cfg, mw, x, enc, t(inp["timestep"]), t(inp["position_ids"]), t(inp["mask"]),
                                workspace=_filled(n, byte, dev))
        torch.cuda.synchronize()
        outs.append(v.float().cpu().numpy())
    assert np.all(np.isfinite(outs[0]))
    np.testing.assert_array_equal(outs[0], outs[1])
