"""GPU parity of k2_block_forward against the CPU oracle (needs an MI355X and libk2.so).

Sizes: the tiny fp32 block and micro shapes with ragged tails are compared element by element;
the full-size 512^2 block in full; the 1024^2 pair and the 2048^2 long block on seeded row samples
(keys and values of every row enter each sampled row's attention, so the sample still checks the
whole key range). Tolerances on max|gpu - oracle| / rms(oracle): fp32 <= 1e-4 against the exact
oracle; bf16 <= 2e-2 against the oracle with bf16 operands, and against the exact oracle no worse
than that oracle's own bf16-vs-exact deviation (tests/k2_testutil.parity).
"""
import numpy as np
import pytest

from flow_matching_diffusion_amd import synth as S
from oracle import k2_oracle as O
from tests.k2_testutil import gpu_block, parity, rel_err, temb_for, workload

pytestmark = pytest.mark.gpu


def _check(wl, inp, rows=None, tag=""):
    temb = temb_for(wl, inp)
    got = gpu_block(wl, inp, temb)
    if rows is not None:
        got = got[:, rows]
    fn = lambda rnd: O.block_forward(inp["h"], temb, inp["position_ids"], inp["mask"], inp["weights"], wl.dims, wl.T,
                                     rows=rows, rnd=rnd)
    parity(tag or wl.name, wl.dtype, got, fn)
    return got


def test_tiny_fp32_block():
    wl = workload("tiny")
    _check(wl, S.block_inputs(wl))


MICRO = {
    # G = 2, head_dim 64, ragged text / grid / intermediate, second batch row with no valid text
    "g2_hd64_f32": (S.BlockDims(hidden=256, num_heads=4, num_kv_heads=2, head_dim=64, intermediate=200,
                                axes_dims=(16, 24, 24)), "f32", 2, 7, (5, 3), (5, 0)),
    "g2_hd64_bf16": (S.BlockDims(hidden=256, num_heads=4, num_kv_heads=2, head_dim=64, intermediate=200,
                                 axes_dims=(16, 24, 24)), "bf16", 2, 7, (5, 3), (5, 0)),
    # MHA, head_dim 128, one batch row
    "g1_hd128_bf16": (S.BlockDims(hidden=256, num_heads=2, num_kv_heads=2, head_dim=128, intermediate=320,
                                  axes_dims=(32, 48, 48)), "bf16", 1, 33, (9, 7), (20,)),
    # G = 4 over two M tiles with a ragged tail, several key tiles, one fully padded text tile
    "g4_hd128_bf16": (S.BlockDims(hidden=512, num_heads=4, num_kv_heads=1, head_dim=128, intermediate=1024,
                                  axes_dims=(32, 48, 48)), "bf16", 2, 140, (12, 11), (70, 3)),
    "g4_hd128_f32": (S.BlockDims(hidden=512, num_heads=4, num_kv_heads=1, head_dim=128, intermediate=1024,
                                 axes_dims=(32, 48, 48)), "f32", 2, 140, (12, 11), (70, 3)),
    # short sequences (L <= 32, the layerwise text-fusion shape): many batch rows, one key chunk
    # (L = 12, no text, no mask), masked text with one row all padding (L = 16), two key chunks at
    # the limit (L = 32), and L = 5 where half the lanes hold no key
    "short12_g1_hd128_bf16": (S.BlockDims(hidden=256, num_heads=2, num_kv_heads=2, head_dim=128, intermediate=320,
                                          axes_dims=(32, 48, 48)), "bf16", 40, 0, (3, 4), None),
    "short16_g4_hd64_bf16": (S.BlockDims(hidden=256, num_heads=4, num_kv_heads=1, head_dim=64, intermediate=200,
                                         axes_dims=(16, 24, 24)), "bf16", 5, 6, (2, 5), (4, 0, 6, 1, 3)),
    "short32_g2_hd128_bf16": (S.BlockDims(hidden=512, num_heads=4, num_kv_heads=2, head_dim=128, intermediate=256,
                                          axes_dims=(32, 48, 48)), "bf16", 3, 7, (5, 5), (7, 2, 0)),
    "short5_g4_hd128_bf16": (S.BlockDims(hidden=512, num_heads=4, num_kv_heads=1, head_dim=128, intermediate=256,
                                         axes_dims=(32, 48, 48)), "bf16", 7, 2, (1, 3), (1, 2, 0, 2, 1, 1, 2)),
}


@pytest.mark.parametrize("name", sorted(MICRO))
def test_micro_block(name):
    dims, dt, B, T, grid, valid = MICRO[name]
    wl = S.Workload(name, 100 + sorted(MICRO).index(name), dt, B, T, grid, valid, dims=dims)
    _check(wl, S.block_inputs(wl), tag=name)


def test_micro_block_no_text_and_no_mask():
    dims = S.BlockDims(hidden=256, num_heads=4, num_kv_heads=1, head_dim=64, intermediate=256, axes_dims=(16, 24, 24))
    wl = S.Workload("notext", 120, "bf16", 2, 0, (8, 9), None, dims=dims)
    _check(wl, S.block_inputs(wl), tag="no text tokens")


def test_block_stages_micro():
    """Intermediates left in the workspace against the oracle's, to localise a mismatch."""
    import torch
    import flow_matching_diffusion_amd as k2
    dims, dt, B, T, grid, valid = MICRO["g4_hd128_f32"]
    wl = S.Workload("stages", 130, dt, B, T, grid, valid, dims=dims)
    inp = S.block_inputs(wl)
    temb = temb_for(wl, inp)
    _, ws, cfg = gpu_block(wl, inp, temb, keep_ws=True)
    _, st = O.block_forward(inp["h"], temb, inp["position_ids"], inp["mask"], inp["weights"], dims, T,
                            intermediates=True)
    lay = k2.block_workspace_layout(cfg, B, T, wl.N)
    L, M, nq, nk, hd = wl.L, wl.M, dims.num_heads * dims.head_dim, dims.num_kv_heads * dims.head_dim, dims.head_dim
    td = torch.float32

    def view(off, n, shape):
        return ws[off:off + 4 * n].view(td).reshape(shape).cpu().numpy()

    checks = {
        "x1": (view(lay.x1, M * dims.hidden, (B, L, dims.hidden)), st["x1"]),
        "q": (view(lay.q, M * nq, (B, L, nq)), st["q"].transpose(0, 2, 1, 3).reshape(B, L, nq)),
        "k": (view(lay.k, M * nk, (B, L, nk)), st["k"].transpose(0, 2, 1, 3).reshape(B, L, nk)),
        "vt": (view(lay.vt, B * nk * lay.ldvt, (B, dims.num_kv_heads, hd, lay.ldvt))[..., :L],
               st["v"].transpose(0, 1, 3, 2)),
        "g": (view(lay.g, M * nq, (B, L, nq)), st["g"]),
        "og": (view(lay.og, M * nq, (B, L, nq)), st["og"]),
        "x2": (view(lay.x2, M * dims.hidden, (B, L, dims.hidden)), st["x2"]),
        "a": (view(lay.a, M * dims.intermediate, (B, L, dims.intermediate)), st["a"]),
    }
    bad = []
    for name, (g, r) in checks.items():
        err, _ = rel_err(g, r)
        print(f"stage {name}: {err:.3e}", flush=True)
        if not err <= 1e-4:
            bad.append(f"{name}={err:.2e}")
    assert not bad, "stages off: " + ", ".join(bad)


def test_padded_text_rows_cannot_change_valid_rows_gpu():
    dims, dt, B, T, grid, valid = MICRO["g4_hd128_bf16"]
    wl = S.Workload("maskinv", 140, dt, B, T, grid, valid, dims=dims)
    inp = S.block_inputs(wl)
    temb = temb_for(wl, inp)
    a = gpu_block(wl, inp, temb)
    h2 = inp["h"].copy()
    g = np.random.default_rng(1)
    for b, v in enumerate(valid):
        h2[b, v:T] = 7.0 * g.standard_normal(h2[b, v:T].shape)
    c = gpu_block(wl, inp, temb, h=h2)
    for b, v in enumerate(valid):
        keep = np.r_[0:v, T:wl.L]
        np.testing.assert_array_equal(a[b, keep], c[b, keep])


def test_null_mask_equals_all_true_mask_gpu():
    dims, dt, B, T, grid, valid = MICRO["g4_hd128_bf16"]
    wl = S.Workload("nullmask", 141, dt, B, T, grid, None, dims=dims)
    inp = S.block_inputs(wl)
    temb = temb_for(wl, inp)
    a = gpu_block(wl, inp, temb, mask=None)
    b = gpu_block(wl, inp, temb, mask=np.ones((B, T), np.uint8))
    np.testing.assert_array_equal(a, b)


def test_block512_full():
    wl = workload("block512")
    _check(wl, S.block_inputs(wl))


def test_block1024_sampled_rows():
    wl = workload("block1024")
    _check(wl, S.block_inputs(wl), rows=S.sample_rows(wl, 96))


def test_block2048_sampled_rows():
    wl = workload("block2048")
    inp = S.block_inputs(wl)
    rows = S.sample_rows(wl, 256)
    assert {0, 511, 512, 16895} <= set(rows.tolist())
    _check(wl, inp, rows=rows)
