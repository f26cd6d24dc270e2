"""GPU parity of k2_block_backward (the block's backward pass, forward recomputed from its input)
against the CPU oracle's chain-rule gradients, which are pinned to torch autograd and to finite
differences on the CPU. Every output is compared: the input gradient, the temb gradient and each
weight gradient, as max |gpu - oracle| / rms(oracle). float32: <= 1e-4 against the exact oracle.
bf16: tests/k2_testutil.parity's bounds for gradients, derived from legitimate realisations of the
bf16 model that the oracle computes (its rounding points include the backward's matrix-product
operands, reading R20)."""
import json

import numpy as np
import pytest

from flow_matching_diffusion_amd import synth as S
from oracle import k2_oracle as O
from tests.k2_testutil import device, err_stats, parity, spread_bound, temb_for

pytestmark = pytest.mark.gpu

G4 = S.BlockDims(hidden=512, num_heads=4, num_kv_heads=1, head_dim=128, intermediate=256, axes_dims=(32, 48, 48))
G2 = S.BlockDims(hidden=256, num_heads=4, num_kv_heads=2, head_dim=64, intermediate=200, axes_dims=(16, 24, 24))
G1 = S.BlockDims(hidden=256, num_heads=2, num_kv_heads=2, head_dim=128, intermediate=320, axes_dims=(32, 48, 48))

CASES = {
    # several 32-key tiles, ragged tails, a text mask with a nearly empty row
    "g4_hd128_f32": (G4, "f32", 2, 12, (6, 5), (12, 3), True),
    "g4_hd128_bf16": (G4, "bf16", 2, 12, (6, 5), (12, 3), True),
    # G = 2, head_dim 64, intermediate not a multiple of 64
    "g2_hd64_f32": (G2, "f32", 1, 7, (5, 3), (5,), True),
    "g2_hd64_bf16": (G2, "bf16", 2, 7, (9, 8), (5, 0), True),
    # MHA over 70 tokens, no mask
    "g1_hd128_bf16": (G1, "bf16", 1, 6, (8, 8), None, True),
    # text-fusion style: no modulation, no RoPE
    "unmodulated_f32": (G2, "f32", 2, 0, (4, 5), None, False),
}


def _case(name):
    dims, dt, B, T, grid, valid, modulated = CASES[name]
    wl = S.Workload(name, 500 + sorted(CASES).index(name), dt, B, T, grid, valid, dims=dims)
    inp = S.block_inputs(wl)
    temb = temb_for(wl, inp)
    if not modulated:
        inp["weights"].pop("scale_shift_table")
        inp["position_ids"] = None
        temb = None
    g = np.random.default_rng(wl.seed)
    dh_out = g.standard_normal(inp["h"].shape).astype(np.float32)
    return wl, inp, temb, dh_out


@pytest.mark.parametrize("name", sorted(CASES))
def test_block_backward(name):
    import torch
    import flow_matching_diffusion_amd as k2
    wl, inp, temb, dh_out = _case(name)
    dev = device()
    cfg = k2.block_cfg(wl.dims, wl.dtype)
    wdev = k2.upload(inp["weights"], wl.dtype, dev)
    ht = torch.from_numpy(np.ascontiguousarray(inp["h"])).to(dev)
    tt = None if temb is None else torch.from_numpy(np.ascontiguousarray(temb, dtype=np.float32)).to(dev)
    pt = None if inp["position_ids"] is None else torch.from_numpy(inp["position_ids"]).to(dev)
    mt = None if inp["mask"] is None else torch.from_numpy(inp["mask"]).to(dev)
    gi, gtemb, grads = k2.block_backward(cfg, wdev, ht, tt, pt, mt, wl.T, torch.from_numpy(dh_out).to(dev))
    torch.cuda.synchronize()
    got = {"h": gi.cpu().numpy()}
    if gtemb is not None:
        got["temb"] = gtemb.cpu().numpy()
    got.update({k: v.cpu().numpy() for k, v in grads.items()})
    cache = {}

    def oracle(rnd):
        key = None if rnd is None else (rnd.flash, rnd.f32_products)
        if key not in cache:
            dh, dtemb, gr = O.block_backward(inp["h"], temb, inp["position_ids"], inp["mask"], inp["weights"], wl.dims,
                                             wl.T, dh_out, rnd=rnd)
            cache[key] = dict(gr, h=dh, temb=dtemb)
        return cache[key]

    assert set(got) == {k for k, v in oracle(None).items() if v is not None}
    for k in sorted(got):
        parity(f"{name} d{k}", wl.dtype, got[k], lambda rnd, k=k: oracle(rnd)[k], kind="backward")


def test_block512_backward_full_width():
    """The full-size block (hidden 6144, 48/12 heads, intermediate 16384) on the 512^2 shape
    (1280 tokens, 192 of 256 text tokens valid), every gradient compared in full."""
    import torch
    import flow_matching_diffusion_amd as k2
    from tests.k2_testutil import workload
    wl = workload("block512")
    inp = S.block_inputs(wl)
    temb = temb_for(wl, inp)
    dh_out = np.random.default_rng(wl.seed + 1).standard_normal(inp["h"].shape).astype(np.float32)
    dev = device()
    cfg = k2.block_cfg(wl.dims, wl.dtype)
    wdev = k2.upload(inp["weights"], wl.dtype, dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    gi, gtemb, grads = k2.block_backward(cfg, wdev, t(inp["h"]), t(temb.astype(np.float32)), t(inp["position_ids"]),
                                         t(inp["mask"]), wl.T, t(dh_out))
    torch.cuda.synchronize()
    got = dict({k: v.cpu().numpy() for k, v in grads.items()}, h=gi.cpu().numpy(), temb=gtemb.cpu().numpy())
    del grads, gi, gtemb, wdev
    cache = {}

    def oracle(rnd):
        key = None if rnd is None else (rnd.flash, rnd.f32_products)
        if key not in cache:
            dh, dtemb, gr = O.block_backward(inp["h"], temb, inp["position_ids"], inp["mask"], inp["weights"], wl.dims,
                                             wl.T, dh_out, rnd=rnd)
            cache[key] = dict(gr, h=dh, temb=dtemb)
        return cache[key]

    # one oracle pass per form (exact and the three bf16 realisations), each kept for every tensor
    for k in sorted(got):
        parity(f"block512 d{k}", wl.dtype, got[k], lambda rnd, k=k: oracle(rnd)[k], kind="backward")


def test_block1024_backward_properties():
    """The benchmarked shape (block1024: 9216 tokens, hidden 6144), where the oracle's backward is out
    of reach on the host, checked through properties that hold at any size:
    - float32: directional derivatives of L = <g, block(h)> from k2_block_backward (along a random
      direction of h, of temb and of the down-projection weight) against central differences of
      two k2_block_forward runs;
    - bf16: its input, temb and down-projection gradients against the float32 ones (which sit within
      1e-4 of the exact function), each statistic (max, p99.9, rms) within the bf16 model's own
      deviation for that gradient at the full-size 512^2 block: the largest of the oracle's three bf16
      realisations against its exact gradients there (tests/golden/block512_backward_bf16_stats.json,
      written from oracle/ alone), times the backward spread factor. Same hidden and intermediate
      sizes, so the same products and reductions; block1024 only has the longer sequence."""
    import torch
    import flow_matching_diffusion_amd as k2
    from tests.k2_testutil import workload
    wl = workload("block1024")
    inp = S.block_inputs(wl)
    temb = temb_for(wl, inp).astype(np.float32)
    rng = np.random.default_rng(wl.seed + 7)
    dev = device()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    h, tb, pos, mask = t(inp["h"]), t(temb), t(inp["position_ids"]), t(inp["mask"])
    g = t(rng.standard_normal(inp["h"].shape).astype(np.float32))

    cfg32 = k2.block_cfg(wl.dims, "f32")
    w32 = k2.upload(inp["weights"], "f32", dev)
    gi, gtemb, grads = k2.block_backward(cfg32, w32, h, tb, pos, mask, wl.T, g, want=["ff_down"])
    torch.cuda.synchronize()

    def loss(hh, tt):
        out = k2.block_forward(cfg32, w32, hh, tt, pos, mask, wl.T)
        return float((g.double() * out.double()).sum())

    eps = 1e-2
    v = t(rng.standard_normal(inp["h"].shape).astype(np.float32))
    u = t(rng.standard_normal(temb.shape).astype(np.float32))
    wd = w32["ff_down"]
    V = torch.randn(wd.shape, device=dev, generator=torch.Generator(device=dev).manual_seed(11)) * 0.02
    checks = []
    checks.append(("h", float((gi.double() * v.double()).sum()),
                   (loss(h + eps * v, tb) - loss(h - eps * v, tb)) / (2 * eps)))
    checks.append(("temb", float((gtemb.double() * u.double()).sum()),
                   (loss(h, tb + eps * u) - loss(h, tb - eps * u)) / (2 * eps)))
    wd.add_(eps * V)
    lp = loss(h, tb)
    wd.sub_(2 * eps * V)
    lm = loss(h, tb)
    wd.add_(eps * V)
    checks.append(("ff_down", float((grads["ff_down"].double() * V.double()).sum()), (lp - lm) / (2 * eps)))
    for name, an, fd in checks:
        rel = abs(an - fd) / abs(fd)
        print(f"block1024 f32 <d{name}, dir>: backward {an:.6e}, central difference {fd:.6e}, rel {rel:.2e}", flush=True)
        assert rel <= 2e-3, f"d{name}: {rel:.2e}"
    ref = {"h": gi.cpu().numpy(), "temb": gtemb.cpu().numpy(), "ff_down": grads["ff_down"].cpu().numpy()}
    del grads, gi, gtemb, w32, wd, V
    torch.cuda.empty_cache()

    cfg16 = k2.block_cfg(wl.dims, "bf16")
    w16 = k2.upload(inp["weights"], "bf16", dev)
    gi, gtemb, grads = k2.block_backward(cfg16, w16, h, tb, pos, mask, wl.T, g, want=["ff_down", "to_q", "norm2_w"])
    torch.cuda.synchronize()
    got = {"h": gi.cpu().numpy(), "temb": gtemb.cpu().numpy(), "ff_down": grads["ff_down"].cpu().numpy()}
    from tests.golden.block512_backward_stats import OUT as STATS, stats_key
    model = json.load(open(STATS))
    assert model["key"] == stats_key(workload("block512")), \
        "the oracle or the generators changed since the statistics were written: run tests/golden/block512_backward_stats.py"
    bad = []
    for k in got:
        assert np.all(np.isfinite(got[k])), k
        st = err_stats(got[k], ref[k], float(np.sqrt(np.mean(np.square(ref[k], dtype=np.float64)))))
        for stat in ("max", "p999", "rms"):
            bound = spread_bound("backward", stat, [model["stats"][k][f] for f in ("A", "B", "C")])
            print(f"block1024 bf16 vs f32 d{k}: {stat} {st[stat]:.3e} (bound {bound:.3e})", flush=True)
            if st[stat] > bound:
                bad.append(f"d{k}: {stat} {st[stat]:.3e} > {bound:.3e}")
    assert not bad, "; ".join(bad)
    for k in ("to_q", "norm2_w"):
        assert np.all(np.isfinite(grads[k].cpu().numpy())), k
