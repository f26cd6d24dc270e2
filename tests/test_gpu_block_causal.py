"""GPU parity of k2_block_forward_block_causal (QwenImage 2.1 model page, block-causal attention item)
against the CPU oracle: query i attends key j iff j <= i or both lie in the same image block, on top
of the key-padding mask. Cases cover every attention kernel (64-key bf16 tiles, 32-key fp32 tiles,
the short-sequence kernel), workgroups whose queries straddle block boundaries, adjacent blocks,
pure causal attention, and text queries left with no key; the 1024^2 shape with a condition block
and a target block is compared on sampled rows. Same tolerances as the block tests."""
import numpy as np
import pytest

from flow_matching_diffusion_amd import synth as S
from oracle import k2_oracle as O
from tests.k2_testutil import gpu_block, parity, temb_for, workload

pytestmark = pytest.mark.gpu

G4_128 = S.BlockDims(hidden=512, num_heads=4, num_kv_heads=1, head_dim=128, intermediate=1024, axes_dims=(32, 48, 48))
G2_64 = S.BlockDims(hidden=256, num_heads=4, num_kv_heads=2, head_dim=64, intermediate=200, axes_dims=(16, 24, 24))
G1_128 = S.BlockDims(hidden=256, num_heads=2, num_kv_heads=2, head_dim=128, intermediate=320, axes_dims=(32, 48, 48))


def _ids(T, spans, N):
    """-1 for the T text tokens, then image runs: spans is a list of (length, id), the last run fills N."""
    ids = [-1] * T
    used = 0
    for n, i in spans:
        ids += [i] * n
        used += n
    assert used == N, (used, N)
    return np.array(ids, np.int32)


CASES = {
    # text | condition block | target block; query workgroups straddle both boundaries
    "cond_target_g4_bf16": (G4_128, "bf16", 2, 12, (12, 11), (12, 3), [(40, 0), (92, 1)]),
    "cond_target_g4_f32": (G4_128, "f32", 2, 12, (12, 11), (12, 3), [(40, 0), (92, 1)]),
    # text only but for one closing image token: plain causal attention over the text
    "causal_g2_bf16": (G2_64, "bf16", 2, 100, (1, 1), (70, 100), [(1, 7)]),
    "causal_g2_f32": (G2_64, "f32", 1, 40, (1, 1), (33,), [(1, 7)]),
    # adjacent blocks with different ids, then text between blocks (text as -1 runs inside the image rows)
    "adjacent_g1_bf16": (G1_128, "bf16", 2, 5, (7, 10), (5, 2), [(20, 0), (20, 1), (3, -1), (27, 2)]),
    # short sequences (L <= 32): the short kernel
    "short_g4_bf16": (G4_128, "bf16", 3, 6, (2, 7), (6, 1, 0), [(5, 0), (9, 1)]),
    # a batch row with no valid text: its text queries have no key (zero attention output)
    "empty_text_g2_f32": (G2_64, "f32", 2, 9, (4, 5), (9, 0), [(6, 0), (14, 1)]),
}


def _run(name, dims, dt, B, T, grid, valid, spans, seed, rows=None):
    wl = S.Workload(name, seed, dt, B, T, grid, valid, dims=dims)
    ids = _ids(T, spans, wl.N)
    inp = S.block_inputs(wl)
    temb = temb_for(wl, inp)
    got = gpu_block(wl, inp, temb, image_ids=ids)
    if rows is not None:
        got = got[:, rows]
    fn = lambda rnd: O.block_forward(inp["h"], temb, inp["position_ids"], inp["mask"], inp["weights"], wl.dims, wl.T,
                                     rows=rows, rnd=rnd, image_ids=ids)
    parity(name, dt, got, fn)
    return wl, inp, temb, ids


@pytest.mark.parametrize("name", sorted(CASES))
def test_block_causal_micro(name):
    dims, dt, B, T, grid, valid, spans = CASES[name]
    _run(name, dims, dt, B, T, grid, valid, spans, 400 + sorted(CASES).index(name))


def test_single_block_equals_plain_block():
    """One image block over the whole sequence lets every query see every key: bit-identical to
    k2_block_forward (the restriction then changes no tile)."""
    dims, dt, B, T, grid, valid, _ = CASES["cond_target_g4_bf16"]
    wl = S.Workload("oneblock", 420, dt, B, T, grid, valid, dims=dims)
    inp = S.block_inputs(wl)
    temb = temb_for(wl, inp)
    a = gpu_block(wl, inp, temb)
    b = gpu_block(wl, inp, temb, image_ids=np.zeros(wl.L, np.int32))
    np.testing.assert_array_equal(a, b)


def test_reach_across_chunks():
    """The per-token reach the kernels use (workspace field reach): the end of each image run, the
    token itself for text, over a sequence longer than three 1024-position chunks with runs that
    cross chunk boundaries."""
    import torch
    import flow_matching_diffusion_amd as k2
    dims = S.BlockDims(hidden=256, num_heads=2, num_kv_heads=2, head_dim=128, intermediate=64, axes_dims=(32, 48, 48))
    g = np.random.default_rng(3)
    T, N = 100, 3300
    spans, left, nid = [], N, 0
    while left:
        n = int(min(left, g.integers(1, 900)))
        spans.append((n, -1 if g.random() < 0.3 else nid))
        nid += 1
        left -= n
    ids = _ids(T, spans, N)
    wl = S.Workload("reach", 421, "bf16", 1, T, (N, 1), None, dims=dims)
    inp = S.block_inputs(wl)
    _, ws, cfg = gpu_block(wl, inp, temb_for(wl, inp), keep_ws=True, image_ids=ids)
    lay = k2.block_workspace_layout(cfg, 1, T, N)
    got = ws[lay.reach:lay.reach + 4 * wl.L].view(torch.int32).cpu().numpy()
    want = np.arange(wl.L)
    for i in range(wl.L - 2, -1, -1):
        if ids[i] >= 0 and ids[i + 1] == ids[i]:
            want[i] = want[i + 1]
    np.testing.assert_array_equal(got, want)


def test_block1024_cond_target_sampled_rows():
    """The 1024^2 CFG pair with the last 4096 tokens split into a 1024-token condition block and a
    3072-token target block; sampled rows from every part."""
    wl = workload("block1024")
    ids = _ids(wl.T, [(1024, 0), (3072, 1)], wl.N)
    rows = np.unique(np.concatenate([S.sample_rows(wl, 64), [0, 299, 300, 511, 512, 1535, 1536, wl.L - 1]]))
    inp = S.block_inputs(wl)
    temb = temb_for(wl, inp)
    got = gpu_block(wl, inp, temb, image_ids=ids)[:, rows]
    fn = lambda rnd: O.block_forward(inp["h"], temb, inp["position_ids"], inp["mask"], inp["weights"], wl.dims, wl.T,
                                     rows=rows, rnd=rnd, image_ids=ids)
    parity("block1024 block-causal", wl.dtype, got, fn)
