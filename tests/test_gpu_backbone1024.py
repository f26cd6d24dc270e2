"""GPU parity of k2_backbone_forward at its own configuration: the 28-block model at 1024^2, B = 2 as a
CFG pair (text 512 tokens with 300 / 16 valid, 64 x 64 latent grid), text fusion over the
(2, 512, 12, 2560) stack, t = 0.7, random-init weights ~N(0, 0.02) in bf16. The expected velocities
(2, 4096, 64) come from tests/golden/backbone1024_velocity.npz, written by
tests/golden/backbone1024_oracle.py from oracle/ alone on the same seeded inputs: the exact function
and the three bf16 realisations that tests/k2_testutil.parity derives its bounds from."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

from flow_matching_diffusion_amd import synth as S
from tests.k2_testutil import device, parity

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
FIXTURE = os.path.join(HERE, "golden", "backbone1024_velocity.npz")


def _fixture_key(wl):
    import importlib.util
    spec = importlib.util.spec_from_file_location("bb_fixture", os.path.join(HERE, "golden", "backbone1024_oracle.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.fixture_key(wl)


def test_backbone1024_against_oracle_fixture():
    import torch
    import flow_matching_diffusion_amd as k2
    wl = S.WORKLOADS["backbone1024"]
    if not os.path.exists(FIXTURE):
        pytest.skip("fixture not written: run tests/golden/backbone1024_oracle.py (about an hour on the host)")
    fx = np.load(FIXTURE, allow_pickle=False)
    assert str(fx["key"]) == _fixture_key(wl), \
        "the oracle or the generators changed since the fixture was written: run tests/golden/backbone1024_oracle.py"
    dev = device()
    mw = k2.upload(S.model_weights(wl.seed, wl, blocks=False), "bf16", dev)

    def one(i):  # draw and round one block's weights on the host (the generators release the GIL)
        return S.block_weights(wl.seed, f"blocks{i}.", wl.dims, wl.dtype)

    mw["blocks"] = []
    with ThreadPoolExecutor(8) as ex:
        for i, w in enumerate(ex.map(one, range(wl.num_layers))):
            mw["blocks"].append(k2.upload(w, "bf16", dev))
            del w
            print(f"backbone1024: block {i + 1}/{wl.num_layers} weights on the device", flush=True)
    inp = S.backbone_inputs(wl)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    x = t(S.as_dtype(inp["x"], "bf16")).to(torch.bfloat16)
    enc = t(inp["enc"]).to(torch.bfloat16)
    cfg = k2.model_cfg(wl.dims, wl.text, wl.num_layers, wl.in_channels, wl.timestep_embed_dim, "bf16")
    got = k2.backbone_forward(cfg, mw, x, enc, t(inp["timestep"]), t(inp["position_ids"]), t(inp["mask"]))
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert got.shape == (2, 4096, 64)
    forms = {None: "exact", (False, False): "A", (True, False): "B", (True, True): "C"}
    fn = lambda rnd: fx[forms[None if rnd is None else (rnd.flash, rnd.f32_products)]].astype(np.float64)
    parity("backbone1024 (28 blocks, text fusion 2x512x12x2560)", "bf16", got, fn)
