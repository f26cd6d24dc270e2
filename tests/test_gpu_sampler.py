"""GPU parity of the sampler entry points against the CPU oracle: the fused guidance + Euler update
(element by element, ragged tail, aliasing) and the denoise step of one image (transformer on the
prompt / negative-prompt pair, then the update), in float32 and bfloat16, guided and unguided, and a
three-step loop."""
import numpy as np
import pytest

import flow_matching_diffusion_amd as k2
import oracle.k2_oracle as O
from flow_matching_diffusion_amd import synth as S
from tests.k2_testutil import device, parity, rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,g", [(4096 * 64 + 3, 4.5), (1000, 0.0), (7, 1.0)])
def test_cfg_euler_update(n, g):
    import torch
    dev = device()
    rng = np.random.default_rng(n)
    x, vc, vu = (rng.standard_normal(n).astype(np.float32) for _ in range(3))
    sig, sig_next = 0.71223218, 0.59758782
    tx, tc, tu = (torch.from_numpy(a).to(dev) for a in (x, vc, vu))
    got = k2.cfg_euler_update(tx, tc, tu if g > 0 else None, g, sig, sig_next)
    inplace = tx.clone()
    k2.cfg_euler_update(inplace, tc, tu if g > 0 else None, g, sig, sig_next, out=inplace)
    torch.cuda.synchronize()
    ref = O.euler_step(x, O.cfg_velocity(vc, vu, g), sig, sig_next)
    err, _ = rel_err(got.cpu().numpy(), ref)
    print(f"cfg_euler n={n} g={g}: {err:.2e}")
    assert err <= 1e-6
    np.testing.assert_array_equal(inplace.cpu().numpy(), got.cpu().numpy())


TEXT_SMALL = S.TextDims(hidden=256, num_heads=2, num_kv_heads=2, head_dim=128, intermediate=200, num_layers=5,
                        num_layerwise_blocks=2, num_refiner_blocks=2)
DIMS = S.BlockDims(hidden=256, num_heads=4, num_kv_heads=1, head_dim=64, intermediate=384, axes_dims=(16, 24, 24))


def _case(dt, seed=401, T=12, grid=(6, 5), valid=(9, 3), layers=2, in_ch=64):
    import torch
    dev = device()
    wl = S.Workload("smp", seed, dt, 2, T, grid, valid, dims=DIMS, text=TEXT_SMALL, num_layers=layers,
                    in_channels=in_ch, timestep_embed_dim=256)
    mw = S.model_weights(seed, wl)
    inp = S.backbone_inputs(wl)
    td = torch.bfloat16 if dt == "bf16" else torch.float32
    cfg = k2.model_cfg(DIMS, TEXT_SMALL, layers, in_ch, 256, dt)
    return wl, mw, inp, cfg, k2.upload(mw, dt, dev), td, dev


@pytest.mark.parametrize("dt,g", [("f32", 4.5), ("f32", 0.0), ("bf16", 4.5), ("bf16", 0.0)])
def test_denoise_step(dt, g):
    import torch
    wl, mw, inp, cfg, wdev, td, dev = _case(dt)
    x = inp["x"][:1].astype(np.float32)
    G = 2 if g > 0 else 1
    enc = inp["enc"][:G]
    mask = inp["mask"][:G]
    sig, sig_next = 0.80487956, 0.71223218
    lat = torch.from_numpy(x.copy()).to(dev)
    k2.denoise_step(cfg, wdev, lat, torch.from_numpy(S.as_dtype(enc, dt)).to(dev).to(td),
                    torch.from_numpy(inp["position_ids"]).to(dev), torch.from_numpy(mask).to(dev), sig, sig_next, g)
    torch.cuda.synchronize()
    enc_o = S.as_dtype(enc, dt)
    fn = lambda rnd: O.denoise_step(x, enc_o[:1], enc_o[1:] if g > 0 else None, mask[:1], mask[1:] if g > 0 else None,
                                    inp["position_ids"], mw, DIMS, S.text_block_dims(TEXT_SMALL), wl.T, sig, sig_next,
                                    g, time_dim=256, rnd=rnd)
    # compare the update (latents move by (sigma_next - sigma) v, small against x): judge it on the
    # change, the part the step computes
    got = lat.cpu().numpy() - x
    parity(f"denoise step {dt} g={g} (update)", dt, got, lambda rnd: fn(rnd) - x)


def test_three_step_loop_f32():
    import torch
    wl, mw, inp, cfg, wdev, td, dev = _case("f32", seed=402)
    x0 = inp["x"][:1].astype(np.float32)
    enc, mask = inp["enc"], inp["mask"]
    sig = O.flow_sigmas(3, wl.N)
    lat = torch.from_numpy(x0.copy()).to(dev)
    encd, maskd, posd = (torch.from_numpy(a).to(dev) for a in (enc, mask, inp["position_ids"]))
    for i in range(3):
        k2.denoise_step(cfg, wdev, lat, encd, posd, maskd, float(sig[i]), float(sig[i + 1]), 4.5)
    torch.cuda.synchronize()
    x = x0.astype(np.float64)
    for i in range(3):
        x = O.denoise_step(x, enc[:1], enc[1:], mask[:1], mask[1:], inp["position_ids"], mw, DIMS,
                           S.text_block_dims(TEXT_SMALL), wl.T, sig[i], sig[i + 1], 4.5, time_dim=256)
    err, _ = rel_err(lat.cpu().numpy() - x0, x - x0)
    print(f"3-step loop f32: {err:.2e}")
    assert err <= 1e-4


@pytest.mark.parametrize("dt,g", [("bf16", 4.5), ("f32", 0.0)])
def test_cached_denoise_steps_bit_identical(dt, g):
    """Three sampler steps through k2_denoise_step_cached with the text rows computed once equal three
    steps of k2_denoise_step bit for bit."""
    import torch
    wl, mw, inp, cfg, wdev, td, dev = _case(dt, seed=403)
    G = 2 if g > 0 else 1
    enc = torch.from_numpy(S.as_dtype(inp["enc"][:G], dt)).to(dev).to(td)
    mask = torch.from_numpy(inp["mask"][:G]).to(dev)
    pos = torch.from_numpy(inp["position_ids"]).to(dev)
    x0 = torch.from_numpy(inp["x"][:1].astype(np.float32)).to(dev)
    sig = O.flow_sigmas(3, wl.N)
    a, b = x0.clone(), x0.clone()
    txt_h = k2.text_embed(cfg, wdev, enc, mask)
    for i in range(3):
        k2.denoise_step(cfg, wdev, a, enc, pos, mask, float(sig[i]), float(sig[i + 1]), g)
        k2.denoise_step_cached(cfg, wdev, b, txt_h, pos, mask, float(sig[i]), float(sig[i + 1]), g)
    torch.cuda.synchronize()
    assert torch.equal(a, b), f"max diff {(a - b).abs().max().item()}"
    assert bool(torch.isfinite(a).all())
