"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one part of the oracle to a closed form, an invariant the pages fix, a library
routine that computes the same definition (torch CPU float64), or a brute-force evaluation on
tiny inputs written as explicit scalar loops. Sources are cited by page title and section:
[API] the 'Krea2Transformer2DModel' model page, [ARTICLE] the architecture article
'Diffusers 中的 Krea2Transformer2DModel' (sections 一..八), [PIPELINE] the 'Krea 2' pipeline page.
"""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.k2_oracle as O
from flow_matching_diffusion_amd import synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

MICRO = S.BlockDims(hidden=32, num_heads=4, num_kv_heads=2, head_dim=8, intermediate=16,
                    axes_dims=(2, 2, 4), rope_theta=1000.0, eps=1e-5)


def micro_inputs(seed=11, B=2, T=4, grid=(2, 2), valid=(3, 2), dims=MICRO, modulated=True):
    wl = S.Workload("micro", seed, "f32", B, T, grid, valid, dims=dims)
    inp = S.block_inputs(wl)
    inp["temb"] = S.normal(seed, "temb", (B, 6 * dims.hidden))
    if not modulated:
        inp["weights"].pop("scale_shift_table")
    return wl, inp


# ----------------------------------------------------------------------------------------------
# Elementwise pieces
# ----------------------------------------------------------------------------------------------
def test_rmsnorm_matches_library():
    # [ARTICLE] §四.4: multiplier (1 + weight); torch's rms_norm puts eps inside the root.
    g = np.random.default_rng(0)
    x = g.standard_normal((7, 33))
    w = 0.1 * g.standard_normal(33)
    ref = F.rms_norm(torch.from_numpy(x), (33,), weight=1 + torch.from_numpy(w), eps=1e-5).numpy()
    np.testing.assert_allclose(O.rms_norm(x, w, 1e-5), ref, rtol=1e-13, atol=1e-13)


def test_rmsnorm_constant_vector_closed_form():
    # RMSNorm of a constant vector c: sign(c) * (1 + w) / sqrt(1 + eps / c^2).
    for c in (-3.0, 0.25, 7.5):
        w = np.linspace(-0.1, 0.1, 16)
        y = O.rms_norm(np.full(16, c), w, 1e-5)
        np.testing.assert_allclose(y, np.sign(c) * (1 + w) / math.sqrt(1 + 1e-5 / c ** 2), rtol=1e-14)
    # zero-centred weight: w = 0 is the identity multiplier
    x = np.arange(1.0, 9.0)
    np.testing.assert_array_equal(O.rms_norm(x, np.zeros(8), 0.0), O.rms_norm(x, None, 0.0))


def test_elementwise_library():
    x = np.linspace(-8, 8, 101)
    t = torch.from_numpy(x)
    np.testing.assert_allclose(O.sigmoid(x), torch.sigmoid(t).numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.silu(x), F.silu(t).numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.gelu_tanh(x), F.gelu(t, approximate="tanh").numpy(), rtol=1e-13, atol=1e-15)
    assert O.sigmoid(np.float64(0.0)) == 0.5


# ----------------------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------------------
@pytest.mark.parametrize("nh,nkv", [(4, 1), (4, 2), (6, 3), (4, 4)])
def test_attention_matches_sdpa(nh, nkv):
    # [ARTICLE] §四.3: GQA by repeating K/V heads, SDPA with the key-padding mask.
    g = np.random.default_rng(nh * 10 + nkv)
    B, L, hd = 2, 9, 16
    q = g.standard_normal((B, nh, L, hd))
    k = g.standard_normal((B, nkv, L, hd))
    v = g.standard_normal((B, nkv, L, hd))
    valid = np.ones((B, L), bool)
    valid[0, 2:4] = False
    valid[1, 0] = False
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
                                         attn_mask=torch.from_numpy(valid)[:, None, None, :],
                                         enable_gqa=True).numpy()
    np.testing.assert_allclose(O.attention(q, k, v, valid), ref, rtol=1e-12, atol=1e-13)


def test_gqa_head_map_is_repeat_interleave():
    # repeat_interleave (head hq -> kv hq // G) is what the article names; plain tiling differs.
    g = np.random.default_rng(5)
    B, nh, nkv, L, hd = 1, 4, 2, 6, 8
    q = g.standard_normal((B, nh, L, hd))
    k = g.standard_normal((B, nkv, L, hd))
    v = g.standard_normal((B, nkv, L, hd))
    o = O.attention(q, k, v, None)
    mha_interleave = O.attention(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1), None)
    mha_tile = O.attention(q, np.tile(k, (1, 2, 1, 1)), np.tile(v, (1, 2, 1, 1)), None)
    np.testing.assert_array_equal(o, mha_interleave)
    assert np.abs(o - mha_tile).max() > 1e-3


def test_attention_softmax_rows_and_single_key():
    g = np.random.default_rng(9)
    q = g.standard_normal((1, 2, 5, 4))
    k = g.standard_normal((1, 2, 5, 4))
    v = g.standard_normal((1, 2, 5, 4))
    # with one valid key the output is that key's value row
    valid = np.zeros((1, 5), bool)
    valid[0, 3] = True
    o = O.attention(q, k, v, valid)
    np.testing.assert_allclose(o, np.broadcast_to(v[:, :, 3:4, :], o.shape), rtol=0, atol=1e-15)
    # constant values: any softmax average gives the constant back
    o = O.attention(q, k, np.ones_like(v), None)
    np.testing.assert_allclose(o, 1.0, rtol=1e-14)


# ----------------------------------------------------------------------------------------------
# Block-causal attention (QwenImage 2.1 page: block-causal attention item; build_token_metadata)
# ----------------------------------------------------------------------------------------------
def test_block_causal_visibility_by_hand():
    # text(3) | image block 0 (3) | image block 1 right after it (2) | text(1) | image block 2 (3):
    # the rule "j <= i, or same image block" written out row by row
    ids = np.array([-1, -1, -1, 0, 0, 0, 1, 1, -1, 2, 2, 2])
    L = ids.size
    want = np.zeros((L, L), bool)
    for i in range(L):
        want[i, :i + 1] = True
    want[3:6, 3:6] = True      # block 0 sees itself in full, not block 1 although it follows
    want[6:8, 6:8] = True
    want[9:12, 9:12] = True
    np.testing.assert_array_equal(O.block_causal_visible(ids), want)
    np.testing.assert_array_equal(O.block_causal_visible(ids, rows=[1, 4, 11]), want[[1, 4, 11]])


def test_block_causal_special_cases_reduce_to_library():
    g = np.random.default_rng(21)
    B, nh, nkv, L, hd = 2, 4, 2, 7, 8
    q = g.standard_normal((B, nh, L, hd))
    k = g.standard_normal((B, nkv, L, hd))
    v = g.standard_normal((B, nkv, L, hd))
    tq, tk, tv = (torch.from_numpy(a) for a in (q, k, v))
    # no image block at all: plain causal attention
    causal = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True).numpy()
    got = O.attention(q, k, v, None, O.block_causal_visible(np.full(L, -1)))
    np.testing.assert_allclose(got, causal, rtol=1e-12, atol=1e-13)
    # one block over the whole sequence: every key visible, the same numbers as no restriction
    full = O.attention(q, k, v, None)
    np.testing.assert_array_equal(O.attention(q, k, v, None, O.block_causal_visible(np.zeros(L, int))), full)
    # text prefix + one target block (the usual layout): the block's rows see every key
    ids = np.array([-1, -1, -1, 5, 5, 5, 5])
    got = O.attention(q, k, v, None, O.block_causal_visible(ids))
    np.testing.assert_array_equal(got[:, :, 3:], full[:, :, 3:])
    np.testing.assert_allclose(got[:, :, :3], causal[:, :, :3], rtol=1e-12, atol=1e-13)


def test_block_causal_bruteforce_with_padding():
    # explicit loops over allowed keys (padding and block-causal together) against the vectorised form
    g = np.random.default_rng(22)
    B, nh, nkv, L, hd = 2, 2, 1, 9, 4
    q = g.standard_normal((B, nh, L, hd))
    k = g.standard_normal((B, nkv, L, hd))
    v = g.standard_normal((B, nkv, L, hd))
    ids = np.array([-1, -1, -1, -1, 3, 3, 3, -1, -1])
    valid = np.ones((B, L), bool)
    valid[0, 2] = False
    valid[1, 0:4] = False          # row 1: the first text queries have no key left
    got = O.attention(q, k, v, valid, O.block_causal_visible(ids))
    for b in range(B):
        for h in range(nh):
            for i in range(L):
                keys = [j for j in range(L) if valid[b, j] and (j <= i or (ids[i] >= 0 and ids[i] == ids[j]))]
                if not keys:
                    np.testing.assert_array_equal(got[b, h, i], 0.0)
                    continue
                sc = [float(np.dot(q[b, h, i], k[b, h // (nh // nkv), j])) / math.sqrt(hd) for j in keys]
                mx = max(sc)
                wts = [math.exp(x - mx) for x in sc]
                ref = sum(w * v[b, h // (nh // nkv), j] for w, j in zip(wts, keys)) / sum(wts)
                np.testing.assert_allclose(got[b, h, i], ref, rtol=1e-12, atol=1e-13)


def test_block_causal_block_ignores_invisible_tokens():
    # block level: a row's output cannot depend on tokens it may not attend (their h rows are
    # randomised); rows that may attend them change
    wl, inp = micro_inputs(seed=38, B=2, T=4, grid=(2, 3), valid=(3, 4))
    ids = np.array([-1, -1, -1, -1, 0, 0, 0, 1, 1, 1])   # text, condition block, target block
    args = (inp["temb"], inp["position_ids"], inp["mask"], inp["weights"], MICRO, wl.T)
    a = O.block_forward(inp["h"], *args, image_ids=ids)
    h2 = inp["h"].copy()
    h2[:, 7:] = 5 * np.random.default_rng(8).standard_normal(h2[:, 7:].shape)   # the target block
    c = O.block_forward(h2, *args, image_ids=ids)
    np.testing.assert_array_equal(a[:, :7], c[:, :7])
    assert np.abs(a[:, 7:] - c[:, 7:]).max() > 1e-3
    h3 = inp["h"].copy()
    h3[:, 2] += 3.0                                          # a text token: later rows see it
    d = O.block_forward(h3, *args, image_ids=ids)
    np.testing.assert_array_equal(a[:, :2], d[:, :2])
    assert np.abs(a[:, 3:] - d[:, 3:]).max() > 1e-6
    # one block over everything equals the unrestricted block
    np.testing.assert_array_equal(O.block_forward(inp["h"], *args, image_ids=np.zeros(wl.L, int)),
                                  O.block_forward(inp["h"], *args))


# ----------------------------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------------------------
def test_rope_matches_complex_rotation():
    # A rotation of pair (x0, x1) by phi is complex multiplication (x0 + i x1) * exp(i phi).
    g = np.random.default_rng(3)
    x = g.standard_normal((2, 3, 5, 16))
    ang = g.standard_normal((5, 8)) * 3
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * np.exp(1j * ang)
    ref = np.stack([z.real, z.imag], axis=-1).reshape(x.shape)
    np.testing.assert_allclose(O.apply_rope(x, ang), ref, rtol=1e-13, atol=1e-14)


def test_rope_text_rows_identity_and_norm():
    # [API] position_ids: text rows all zero -> identity rotation; rotations keep norms.
    pos = S.position_ids(4, 3, 3)
    ang = O.rope_angles(pos, (32, 48, 48), 1000.0)
    assert ang.shape == (13, 64)
    assert np.all(ang[:4] == 0)
    x = np.random.default_rng(1).standard_normal((13, 128))
    y = O.apply_rope(x, ang)
    np.testing.assert_array_equal(y[:4], x[:4])
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


def test_rope_axis_split_and_first_frequency():
    # [API] axes_dims_rope splits the head dim among (t, h, w) in that order: a unit step on one
    # axis turns only that axis' pairs, and the first pair of each axis turns by the position.
    axes = (32, 48, 48)
    for a, (lo, hi) in enumerate([(0, 16), (16, 40), (40, 64)]):
        pos = np.zeros((1, 3))
        pos[0, a] = 2.0
        ang = O.rope_angles(pos, axes, 1000.0)[0]
        assert np.all(ang[:lo] == 0) and np.all(ang[hi:] == 0)
        assert ang[lo] == 2.0
        # frequencies fall geometrically to theta^(-(d-2)/d) at the last pair of the axis
        d = axes[a]
        np.testing.assert_allclose(ang[hi - 1], 2.0 * 1000.0 ** (-(d - 2) / d), rtol=1e-14)
        np.testing.assert_allclose(ang[lo + 1:hi] / ang[lo:hi - 1], 1000.0 ** (-2.0 / d), rtol=1e-13)


def test_rope_relative_position():
    # After rotation, q.k depends on the position difference only.
    g = np.random.default_rng(4)
    q = g.standard_normal((1, 16))
    k = g.standard_normal((1, 16))
    axes = (4, 6, 6)
    p1, p2 = np.array([[0.0, 3, 5]]), np.array([[0.0, 1, 2]])
    shift = np.array([[2.0, -7, 11]])
    d0 = O.apply_rope(q, O.rope_angles(p1, axes, 1000.0)) @ O.apply_rope(k, O.rope_angles(p2, axes, 1000.0)).T
    d1 = O.apply_rope(q, O.rope_angles(p1 + shift, axes, 1000.0)) @ O.apply_rope(k, O.rope_angles(p2 + shift, axes, 1000.0)).T
    np.testing.assert_allclose(d0, d1, rtol=1e-12)


# ----------------------------------------------------------------------------------------------
# Whole block: library composition and brute force
# ----------------------------------------------------------------------------------------------
class _Round(torch.autograd.Function):
    """Rounds in the forward pass; passes the gradient through unchanged (the oracle's backward
    treats a rounding point's derivative as 1)."""
    @staticmethod
    def forward(ctx, x, fn):
        return fn(x)

    @staticmethod
    def backward(ctx, g):
        return g, None


class _GradRound(torch.autograd.Function):
    """Identity in the forward pass; rounds the gradient that flows back through it."""
    @staticmethod
    def forward(ctx, x, fn):
        ctx.fn = fn
        return x.view_as(x)

    @staticmethod
    def backward(ctx, g):
        return ctx.fn(g), None


def torch_bf16(x, point=None):
    """bf16 rounding by torch's own conversions: float64 -> float32 -> bfloat16 -> float64."""
    return x.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def skip_point(off, base=torch_bf16):
    """A rounding hook that rounds at every named point except `off`."""
    return lambda x, point=None: x if point == off else base(x, point)


def torch_block_t(h, temb, pos, mask, w, d, T, image_ids=None, rnd=None, flash=False):
    """The block composed from torch library routines in float64 (F.linear, F.rms_norm,
    F.scaled_dot_product_attention with enable_gqa and a boolean mask, complex RoPE, F.silu) on
    float64 tensors h, temb (or None) and the weight dict w (tensors; autograd follows them).
    rnd(x, point): a rounding hook applied at the named points of the bf16 model (x1, q, k, v, g,
    p, o, og, x2, a) in the forward pass, and to the gradients that enter the backward's matrix
    products (dz, dgt, du, dy, do, dgraw, dq, dk, dv, ds). With a hook, attention is written out
    (repeat_interleave, masked torch.softmax, then the rounded probabilities times V; flash=True
    rounds exp(s - rowmax) and divides by the unrounded row sum afterwards)."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    R = (lambda x, n: x) if rnd is None else (lambda x, n: _Round.apply(x, lambda y: rnd(y, n)))
    GR = (lambda x, n: x) if rnd is None else (lambda x, n: _GradRound.apply(x, lambda y: rnd(y, n)))
    B, L, H = h.shape
    nh, nkv, hd = d.num_heads, d.num_kv_heads, d.head_dim
    one = lambda key: 1 + w[key] if w.get(key) is not None else None
    if temb is not None:
        ps, pt, pg, qs, qt, qg = (temb.view(B, 6, H) + w["scale_shift_table"]).unbind(1)
        ps, pt, pg, qs, qt, qg = (u[:, None, :] for u in (ps, pt, pg, qs, qt, qg))
    else:
        ps = pt = qs = qt = torch.zeros((), dtype=torch.float64)
        pg = qg = torch.ones((), dtype=torch.float64)
    x = R((1 + ps) * F.rms_norm(h, (H,), weight=one("norm1_w"), eps=d.eps) + pt, "x1")
    q = GR(F.linear(x, w["to_q"]), "dq").view(B, L, nh, hd).transpose(1, 2)
    k = GR(F.linear(x, w["to_k"]), "dk").view(B, L, nkv, hd).transpose(1, 2)
    v = GR(R(F.linear(x, w["to_v"]), "v"), "dv").view(B, L, nkv, hd).transpose(1, 2)
    q = F.rms_norm(q, (hd,), weight=one("norm_q_w"), eps=d.eps)
    k = F.rms_norm(k, (hd,), weight=one("norm_k_w"), eps=d.eps)
    if pos is not None:
        freqs = []
        for a, da in enumerate(d.axes_dims):
            inv = 1.0 / (d.rope_theta ** (torch.arange(0, da, 2, dtype=torch.float64) / da))
            freqs.append(torch.outer(t(pos)[:, a], inv))
        rot = torch.polar(torch.ones(L, hd // 2, dtype=torch.float64), torch.cat(freqs, dim=1))
        q = torch.view_as_real(torch.view_as_complex(q.reshape(B, nh, L, hd // 2, 2).contiguous()) * rot).flatten(-2)
        k = torch.view_as_real(torch.view_as_complex(k.reshape(B, nkv, L, hd // 2, 2).contiguous()) * rot).flatten(-2)
    q, k = R(q, "q"), R(k, "k")
    valid = torch.ones(B, L, dtype=torch.bool)
    if mask is not None:
        valid[:, :T] = torch.from_numpy(np.asarray(mask).astype(bool))
    am = valid[:, None, None, :]
    if image_ids is not None:
        ids = torch.from_numpy(np.asarray(image_ids))
        j = torch.arange(L)
        vis = (j[None, :] <= j[:, None]) | ((ids[:, None] >= 0) & (ids[:, None] == ids[None, :]))
        am = am & vis[None, None]
    if rnd is None:
        o = F.scaled_dot_product_attention(q, k, v, attn_mask=am, enable_gqa=True)
    else:
        kk, vv = k.repeat_interleave(nh // nkv, dim=1), v.repeat_interleave(nh // nkv, dim=1)
        s = GR((q @ kk.transpose(-1, -2)) / math.sqrt(hd), "ds").masked_fill(~am, float("-inf"))
        if flash:
            e = torch.exp(s - s.amax(dim=-1, keepdim=True))
            o = (R(e, "p") @ vv) / e.sum(dim=-1, keepdim=True)
        else:
            o = R(torch.softmax(s, dim=-1), "p") @ vv
    o = GR(R(o.transpose(1, 2).reshape(B, L, nh * hd), "o"), "do")
    gate = GR(R(F.linear(x, w["to_gate"]), "g"), "dgraw")
    og = R(o * torch.sigmoid(gate), "og")
    h = h + pg * GR(F.linear(og, w["to_out"]), "dy")
    x2 = R((1 + qs) * F.rms_norm(h, (H,), weight=one("norm2_w"), eps=d.eps) + qt, "x2")
    a = R(F.silu(GR(F.linear(x2, w["ff_gate"]), "dgt")) * GR(F.linear(x2, w["ff_up"]), "du"), "a")
    return h + qg * GR(F.linear(a, w["ff_down"]), "dz")


def torch_block(h, temb, pos, mask, w, d, T, image_ids=None, rnd=None, flash=False):
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    wt = {key: (None if val is None else t(val)) for key, val in w.items()}
    return torch_block_t(t(h), None if temb is None else t(temb), pos, mask, wt, d, T, image_ids=image_ids,
                         rnd=rnd, flash=flash).numpy()


@pytest.mark.parametrize("case", ["gqa2", "gqa4_tiny_axes", "mha_nomask", "unmodulated"])
def test_block_matches_library_composition(case):
    if case == "gqa2":
        wl, inp = micro_inputs()
        d = MICRO
    elif case == "gqa4_tiny_axes":
        d = S.BlockDims(hidden=64, num_heads=4, num_kv_heads=1, head_dim=16, intermediate=40,
                        axes_dims=(4, 6, 6), rope_theta=1000.0, eps=1e-5)
        wl, inp = micro_inputs(seed=12, B=1, T=5, grid=(3, 2), valid=(4,), dims=d)
    elif case == "mha_nomask":
        d = replace(MICRO, num_kv_heads=4)
        wl, inp = micro_inputs(seed=13, valid=None, dims=d)
    else:
        d = MICRO
        wl, inp = micro_inputs(seed=14, modulated=False)
        inp["temb"] = None
        inp["position_ids"] = None
    w = inp["weights"]
    ref = torch_block(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], w, d, wl.T)
    got = O.block_forward(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], w, d, wl.T)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-11)


def brute_block(h, temb, pos, mask, w, d, T):
    """Scalar loops over one block, straight from the definitions (no vector operations)."""
    B, L, H = h.shape
    nh, nkv, hd, I, eps = d.num_heads, d.num_kv_heads, d.head_dim, d.intermediate, d.eps
    G = nh // nkv

    def norm_row(vals, wt):
        ms = sum(float(u) * float(u) for u in vals) / len(vals)
        r = 1.0 / math.sqrt(ms + eps)
        return [float(vals[j]) * r * (1.0 + float(wt[j])) for j in range(len(vals))]

    def lin(xrow, W):
        return [sum(float(xrow[j]) * float(W[n][j]) for j in range(len(xrow))) for n in range(len(W))]

    def rotate(vec, p):
        out = list(vec)
        off = 0
        for a, da in enumerate(d.axes_dims):
            for i in range(da // 2):
                ang = float(p[a]) * d.rope_theta ** (-(2.0 * i) / da)
                c, s = math.cos(ang), math.sin(ang)
                x0, x1 = vec[off + 2 * i], vec[off + 2 * i + 1]
                out[off + 2 * i] = x0 * c - x1 * s
                out[off + 2 * i + 1] = x0 * s + x1 * c
            off += da
        return out

    res = np.zeros((B, L, H))
    tab = w["scale_shift_table"]
    for b in range(B):
        mod = [[float(temb[b][c * H + j]) + float(tab[c][j]) for j in range(H)] for c in range(6)]
        x1 = []
        for i in range(L):
            nr = norm_row(h[b][i], w["norm1_w"])
            x1.append([(1 + mod[0][j]) * nr[j] + mod[1][j] for j in range(H)])
        qf = [lin(x1[i], w["to_q"]) for i in range(L)]
        kf = [lin(x1[i], w["to_k"]) for i in range(L)]
        vf = [lin(x1[i], w["to_v"]) for i in range(L)]
        gf = [lin(x1[i], w["to_gate"]) for i in range(L)]
        qh = [[rotate(norm_row(qf[i][hh * hd:(hh + 1) * hd], w["norm_q_w"]), pos[i]) for hh in range(nh)] for i in range(L)]
        kh = [[rotate(norm_row(kf[i][hh * hd:(hh + 1) * hd], w["norm_k_w"]), pos[i]) for hh in range(nkv)] for i in range(L)]
        ok = [j >= T or (mask is None) or bool(mask[b][j]) for j in range(L)]
        og = [[0.0] * (nh * hd) for _ in range(L)]
        for hq in range(nh):
            kvh = hq // G
            for i in range(L):
                sc = [sum(qh[i][hq][e] * kh[j][kvh][e] for e in range(hd)) / math.sqrt(hd) for j in range(L)]
                mx = max(sc[j] for j in range(L) if ok[j])
                p = [math.exp(sc[j] - mx) if ok[j] else 0.0 for j in range(L)]
                z = sum(p)
                for e in range(hd):
                    o = sum(p[j] * vf[j][kvh * hd + e] for j in range(L)) / z
                    gate = 1.0 / (1.0 + math.exp(-gf[i][hq * hd + e]))
                    og[i][hq * hd + e] = o * gate
        for i in range(L):
            ao = lin(og[i], w["to_out"])
            h1 = [float(h[b][i][j]) + mod[2][j] * ao[j] for j in range(H)]
            nr = norm_row(h1, w["norm2_w"])
            x2 = [(1 + mod[3][j]) * nr[j] + mod[4][j] for j in range(H)]
            gg = lin(x2, w["ff_gate"])
            uu = lin(x2, w["ff_up"])
            act = [gg[n] / (1.0 + math.exp(-gg[n])) * uu[n] for n in range(I)]
            dn = lin(act, w["ff_down"])
            for j in range(H):
                res[b][i][j] = h1[j] + mod[5][j] * dn[j]
    return res


def test_block_matches_bruteforce_loops():
    # Micro shape after the model test fixture of [ARTICLE] §六: 4 query / 2 kv heads, head dim 8,
    # a 2x2 latent grid, text rows at the origin, trailing text tokens padded.
    wl, inp = micro_inputs(seed=21)
    ref = brute_block(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], inp["weights"], MICRO, wl.T)
    got = O.block_forward(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], inp["weights"], MICRO, wl.T)
    np.testing.assert_allclose(got, ref, rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# Block invariants the pages fix
# ----------------------------------------------------------------------------------------------
def test_zero_gates_give_identity():
    # [ARTICLE] §四.2: both branches enter through their gates; gates of zero leave h unchanged.
    wl, inp = micro_inputs(seed=31)
    H = MICRO.hidden
    w = dict(inp["weights"])
    tab = w["scale_shift_table"].astype(np.float64).copy()
    temb = inp["temb"].astype(np.float64)
    tab[2] = -temb[0, 2 * H:3 * H]
    tab[5] = -temb[0, 5 * H:6 * H]
    w["scale_shift_table"] = tab
    got = O.block_forward(inp["h"][:1], temb[:1], inp["position_ids"], inp["mask"][:1], w, MICRO, wl.T)
    np.testing.assert_array_equal(got, inp["h"][:1].astype(np.float64))


def test_zero_output_projections_give_identity():
    wl, inp = micro_inputs(seed=32)
    w = dict(inp["weights"])
    w["to_out"] = np.zeros_like(w["to_out"])
    w["ff_down"] = np.zeros_like(w["ff_down"])
    got = O.block_forward(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], w, MICRO, wl.T)
    np.testing.assert_array_equal(got, inp["h"].astype(np.float64))


def test_padded_text_cannot_change_valid_rows():
    # [API] encoder_attention_mask marks valid text tokens; padded tokens are masked as keys.
    wl, inp = micro_inputs(seed=33)
    args = (inp["temb"], inp["position_ids"], inp["mask"], inp["weights"], MICRO, wl.T)
    a = O.block_forward(inp["h"], *args)
    h2 = inp["h"].copy()
    g = np.random.default_rng(7)
    for b, v in enumerate(wl.valid):
        h2[b, v:wl.T] = 5 * g.standard_normal(h2[b, v:wl.T].shape)
    c = O.block_forward(h2, *args)
    for b, v in enumerate(wl.valid):
        keep = np.r_[0:v, wl.T:wl.L]
        np.testing.assert_array_equal(a[b, keep], c[b, keep])
        assert np.abs(a[b, v:wl.T] - c[b, v:wl.T]).max() > 1e-3


def test_null_mask_equals_all_true_mask():
    wl, inp = micro_inputs(seed=34)
    all_true = np.ones_like(inp["mask"])
    a = O.block_forward(inp["h"], inp["temb"], inp["position_ids"], None, inp["weights"], MICRO, wl.T)
    b = O.block_forward(inp["h"], inp["temb"], inp["position_ids"], all_true, inp["weights"], MICRO, wl.T)
    np.testing.assert_array_equal(a, b)


def test_batch_rows_are_independent():
    # A CFG pair batched as B=2 equals two B=1 calls; swapping the pair swaps the outputs.
    wl, inp = micro_inputs(seed=35)
    args = (inp["position_ids"],)
    full = O.block_forward(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], inp["weights"], MICRO, wl.T)
    for b in range(2):
        one = O.block_forward(inp["h"][b:b + 1], inp["temb"][b:b + 1], inp["position_ids"], inp["mask"][b:b + 1],
                              inp["weights"], MICRO, wl.T)
        np.testing.assert_allclose(one[0], full[b], rtol=1e-13, atol=1e-13)
    sw = O.block_forward(inp["h"][::-1], inp["temb"][::-1], inp["position_ids"], inp["mask"][::-1],
                         inp["weights"], MICRO, wl.T)
    np.testing.assert_allclose(sw[::-1], full, rtol=1e-13, atol=1e-13)
    del args


def test_gqa_equals_mha_with_repeated_kv_weights():
    # Spec invariant: GQA equals MHA whose K/V projections repeat each kv head G times.
    wl, inp = micro_inputs(seed=36)
    w = dict(inp["weights"])
    d = MICRO
    G = d.num_heads // d.num_kv_heads
    rep = lambda W: np.repeat(W.reshape(d.num_kv_heads, d.head_dim, -1), G, axis=0).reshape(d.num_heads * d.head_dim, -1)
    wm = dict(w, to_k=rep(w["to_k"]), to_v=rep(w["to_v"]))
    a = O.block_forward(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], w, d, wl.T)
    b = O.block_forward(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], wm, replace(d, num_kv_heads=d.num_heads), wl.T)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)


def test_row_subset_equals_full_rows():
    wl, inp = micro_inputs(seed=37)
    rows = np.array([0, 3, 4, 7])
    args = (inp["temb"], inp["position_ids"], inp["mask"], inp["weights"], MICRO, wl.T)
    full = O.block_forward(inp["h"], *args)
    sub = O.block_forward(inp["h"], *args, rows=rows)
    np.testing.assert_allclose(sub, full[:, rows], rtol=1e-13, atol=1e-13)


def test_rows_with_zero_positions_never_rotate():
    # With a single image (t = 0 for every token) the first axis' pairs of every head are never
    # rotated: changing only t-axis frequencies (theta of that chunk) cannot change anything.
    wl, inp = micro_inputs(seed=38)
    assert np.all(inp["position_ids"][:, 0] == 0)
    ang = O.rope_angles(inp["position_ids"], MICRO.axes_dims, MICRO.rope_theta)
    assert np.all(ang[:, : MICRO.axes_dims[0] // 2] == 0)


# ----------------------------------------------------------------------------------------------
# Backward pass (R20): against torch autograd through the library composition, and against
# central finite differences of the oracle's own forward
# ----------------------------------------------------------------------------------------------
def _bwd_case(case):
    if case == "gqa2":
        wl, inp = micro_inputs(seed=60)
        return MICRO, wl, inp, None
    if case == "mha_nomask":
        d = replace(MICRO, num_kv_heads=4)
        wl, inp = micro_inputs(seed=61, valid=None, dims=d)
        return d, wl, inp, None
    if case == "unmodulated":
        wl, inp = micro_inputs(seed=62, modulated=False)
        inp["temb"] = None
        inp["position_ids"] = None
        return MICRO, wl, inp, None
    # block-causal: text, a condition block, the target block (no query is left without a key)
    wl, inp = micro_inputs(seed=63, B=2, T=4, grid=(2, 3), valid=(3, 4))
    return MICRO, wl, inp, np.array([-1, -1, -1, -1, 0, 0, 0, 1, 1, 1])


@pytest.mark.parametrize("case", ["gqa2", "mha_nomask", "unmodulated", "block_causal"])
def test_block_backward_matches_autograd(case):
    d, wl, inp, ids = _bwd_case(case)
    w = inp["weights"]
    g = np.random.default_rng(70)
    dh_out = g.standard_normal(inp["h"].shape)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64)).requires_grad_(True)
    ht = t(inp["h"])
    tt = None if inp["temb"] is None else t(inp["temb"])
    wt = {key: (None if val is None else t(val)) for key, val in w.items()}
    out = torch_block_t(ht, tt, inp["position_ids"], inp["mask"], wt, d, wl.T, image_ids=ids)
    out.backward(torch.from_numpy(dh_out))
    dh, dtemb, grads = O.block_backward(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], w, d, wl.T, dh_out,
                                        image_ids=ids)
    np.testing.assert_allclose(dh, ht.grad.numpy(), rtol=1e-9, atol=1e-10)
    if tt is not None:
        np.testing.assert_allclose(dtemb, tt.grad.numpy(), rtol=1e-9, atol=1e-10)
    for key, val in wt.items():
        if val is None:
            assert grads[key] is None
            continue
        np.testing.assert_allclose(grads[key], val.grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=key)


def test_block_backward_finite_differences():
    # <grad, v> against (f(x + e v) - f(x - e v)) / 2e . dh_out for random directions v in h, temb
    # and three weights: only the oracle's forward enters the reference
    d, wl, inp, _ = _bwd_case("gqa2")
    w = inp["weights"]
    g = np.random.default_rng(71)
    dh_out = g.standard_normal(inp["h"].shape)
    args = (inp["position_ids"], inp["mask"])
    dh, dtemb, grads = O.block_backward(inp["h"], inp["temb"], *args, w, d, wl.T, dh_out)
    f = lambda h, temb, ww: float(np.sum(O.block_forward(h, temb, *args, ww, d, wl.T) * dh_out))
    eps = 1e-5
    checks = [("h", dh), ("temb", dtemb)] + [(k, grads[k]) for k in ("to_k", "norm_q_w", "ff_down", "scale_shift_table")]
    for name, grad in checks:
        vdir = g.standard_normal(grad.shape)
        def at(sign):
            h, temb, ww = inp["h"].astype(np.float64), inp["temb"].astype(np.float64), dict(w)
            if name == "h":
                h = h + sign * eps * vdir
            elif name == "temb":
                temb = temb + sign * eps * vdir
            else:
                ww[name] = w[name].astype(np.float64) + sign * eps * vdir
            return f(h, temb, ww)
        fd = (at(+1) - at(-1)) / (2 * eps)
        an = float(np.sum(grad * vdir))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), f"{name}: finite difference {fd} vs {an}"


def test_attention_and_norm_backward_match_autograd():
    g = np.random.default_rng(72)
    B, nh, nkv, L, hd = 2, 4, 2, 7, 8
    q, k, v, do = (g.standard_normal(s) for s in ((B, nh, L, hd), (B, nkv, L, hd), (B, nkv, L, hd), (B, nh, L, hd)))
    valid = np.ones((B, L), bool)
    valid[1, :2] = False
    tq, tk, tv = (torch.from_numpy(a).requires_grad_(True) for a in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(valid)[:, None, None, :], enable_gqa=True)
    o.backward(torch.from_numpy(do))
    dq, dk, dv = O.attention_backward(q, k, v, valid, do)
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)
    x = g.standard_normal((3, 5, 16))
    wgt = 0.1 * g.standard_normal(16)
    dy = g.standard_normal(x.shape)
    tx, tw = torch.from_numpy(x).requires_grad_(True), torch.from_numpy(wgt).requires_grad_(True)
    F.rms_norm(tx, (16,), weight=1 + tw, eps=1e-5).backward(torch.from_numpy(dy))
    dx, dw = O.rms_norm_backward(x, wgt, 1e-5, dy)
    np.testing.assert_allclose(dx, tx.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dw, tw.grad.numpy(), rtol=1e-10, atol=1e-12)


# ----------------------------------------------------------------------------------------------
# Time path
# ----------------------------------------------------------------------------------------------
def test_timestep_embedding_closed_forms():
    # [ARTICLE] §四.5: cos first, input time scaled by 1000, width 256.
    e0 = O.timestep_embedding(np.array([0.0]))
    np.testing.assert_array_equal(e0[0, :128], 1.0)
    np.testing.assert_array_equal(e0[0, 128:], 0.0)
    t = np.array([0.7, 0.123])
    e = O.timestep_embedding(t)
    np.testing.assert_allclose(e[:, :128] ** 2 + e[:, 128:] ** 2, 1.0, rtol=1e-14)
    np.testing.assert_allclose(e[:, 0], np.cos(1000 * t), rtol=1e-14)
    np.testing.assert_allclose(e[:, 128], np.sin(1000 * t), rtol=1e-12, atol=1e-14)
    # frequency of column 64 is 10000^(-1/2) = 1/100
    np.testing.assert_allclose(e[:, 64], np.cos(10 * t), rtol=1e-13)


def test_time_path_matches_library_composition():
    H = 24
    tw = S.time_weights(3, H, 256, "f32")
    t = np.array([0.0, 0.7, 1.0])
    temb, e = O.time_path(t, tw)
    tt = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    emb = tt(O.timestep_embedding(t))
    e_ref = F.linear(F.gelu(F.linear(emb, tt(tw["lin1_w"]), tt(tw["lin1_b"])), approximate="tanh"),
                     tt(tw["lin2_w"]), tt(tw["lin2_b"]))
    m_ref = F.linear(F.gelu(e_ref, approximate="tanh"), tt(tw["mod_w"]), tt(tw["mod_b"]))
    np.testing.assert_allclose(e, e_ref.numpy(), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(temb, m_ref.numpy(), rtol=1e-13, atol=1e-14)
    assert temb.shape == (3, 6 * H)


# ----------------------------------------------------------------------------------------------
# Text fusion and backbone
# ----------------------------------------------------------------------------------------------
TEXT_MICRO = S.TextDims(hidden=32, num_heads=4, num_kv_heads=4, head_dim=8, intermediate=24, num_layers=3,
                        num_layerwise_blocks=2, num_refiner_blocks=2, eps=1e-5)


def text_case(seed=41, B=2, T=5, valid=(4, 2)):
    tw = S.text_weights(seed, TEXT_MICRO, "f32")
    enc = S.normal(seed, "enc", (B, T, TEXT_MICRO.num_layers, TEXT_MICRO.hidden))
    return tw, enc, S.text_mask(B, T, valid)


def test_text_fusion_layer_permutation_invariance():
    # [ARTICLE] §四.1: layerwise attention over the layer axis has no positions, so permuting the
    # layers together with the compressor weights leaves the fused text unchanged.
    tw, enc, mask = text_case()
    td = S.text_block_dims(TEXT_MICRO)
    a = O.text_fusion(enc, mask, tw, td)
    perm = np.array([2, 0, 1])
    tw2 = dict(tw, compress_w=tw["compress_w"][perm])
    b = O.text_fusion(enc[:, :, perm], mask, tw2, td)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)


def test_text_fusion_token_permutation_equivariance():
    # Refiner blocks have no RoPE: permuting tokens and the mask permutes the output.
    tw, enc, mask = text_case(seed=42)
    td = S.text_block_dims(TEXT_MICRO)
    a = O.text_fusion(enc, mask, tw, td)
    perm = np.array([3, 0, 4, 1, 2])
    b = O.text_fusion(enc[:, perm], mask[:, perm], tw, td)
    np.testing.assert_allclose(b, a[:, perm], rtol=1e-11, atol=1e-12)


def test_text_fusion_padded_tokens_cannot_change_valid_tokens():
    tw, enc, mask = text_case(seed=43)
    td = S.text_block_dims(TEXT_MICRO)
    a = O.text_fusion(enc, mask, tw, td)
    enc2 = enc.copy()
    enc2[0, 4:] = 9.0
    enc2[1, 2:] = -3.0
    b = O.text_fusion(enc2, mask, tw, td)
    np.testing.assert_array_equal(a[0, :4], b[0, :4])
    np.testing.assert_array_equal(a[1, :2], b[1, :2])


def torch_text_fusion(enc, mask, tw, td, rnd=None):
    B, T, NL, D = enc.shape
    x = enc.reshape(B * T, NL, D)
    for bw in tw["layerwise"]:
        x = torch_block(x, None, None, None, bw, td, 0, rnd=rnd)
    y = F.linear(torch.from_numpy(np.ascontiguousarray(np.swapaxes(x, 1, 2))),
                 torch.from_numpy(tw["compress_w"].astype(np.float64))[None]).squeeze(-1).numpy()
    y = y.reshape(B, T, D)
    for bw in tw["refiner"]:
        y = torch_block(y, None, None, mask, bw, td, T, rnd=rnd)
    return y


def test_text_fusion_matches_library_composition():
    tw, enc, mask = text_case(seed=44)
    td = S.text_block_dims(TEXT_MICRO)
    np.testing.assert_allclose(O.text_fusion(enc, mask, tw, td), torch_text_fusion(enc, mask, tw, td),
                               rtol=1e-11, atol=1e-12)


def micro_backbone(seed=51, B=1, T=16, grid=(8, 8), valid=(12,), in_ch=64, layers=2):
    d = S.BlockDims(hidden=32, num_heads=4, num_kv_heads=2, head_dim=8, intermediate=16, axes_dims=(2, 2, 4))
    wl = S.Workload("mb", seed, "f32", B, T, grid, valid, dims=d, text=TEXT_MICRO, num_layers=layers,
                    in_channels=in_ch, timestep_embed_dim=16)
    mw = S.model_weights(seed, wl)
    inp = S.backbone_inputs(wl)
    return wl, d, mw, inp


def test_backbone_quickstart_output_shape():
    g = json.load(open(os.path.join(GOLDEN, "quickstart_shape.json")))
    wl, d, mw, inp = micro_backbone(B=g["batch"], T=g["text_seq"], grid=tuple(g["grid"]), valid=None,
                                    in_ch=g["in_channels"])
    out = O.backbone_forward(inp["x"], inp["enc"], inp["timestep"], inp["position_ids"], inp["mask"], mw, d,
                             S.text_block_dims(TEXT_MICRO), wl.T, time_dim=16)
    assert list(out.shape) == g["printed_shape"]


def torch_backbone(wl, d, mw, inp, td, rnd=None):
    """The backbone composed from torch routines in float64, with the rounding hook of R13."""
    R = (lambda x, n: x) if rnd is None else rnd
    tt = lambda a: torch.from_numpy(np.asarray(a, np.float64))
    tw = mw["time"]
    emb = R(tt(O.timestep_embedding(inp["timestep"], 16)), "temb_in")
    e = F.linear(R(F.gelu(F.linear(emb, tt(tw["lin1_w"]), tt(tw["lin1_b"])), approximate="tanh"), "temb_act"),
                 tt(tw["lin2_w"]), tt(tw["lin2_b"]))
    temb = F.linear(R(F.gelu(e, approximate="tanh"), "temb_e"), tt(tw["mod_w"]), tt(tw["mod_b"]))
    fused = R(tt(torch_text_fusion(inp["enc"], inp["mask"], mw["text"], td, rnd=rnd)), "text_fused")
    txt = F.linear(fused, tt(mw["txt_in_w"]), tt(mw["txt_in_b"]))
    img = F.linear(tt(inp["x"]), tt(mw["img_in_w"]), tt(mw["img_in_b"]))
    h = torch.cat([txt, img], dim=1).numpy()
    for bw in mw["blocks"]:
        h = torch_block(h, temb.numpy(), inp["position_ids"], inp["mask"], bw, d, wl.T, rnd=rnd)
    hi = tt(h[:, wl.T:])
    scale, shift = (tt(mw["final_table"])[None] + e[:, None]).unbind(1)
    x = R((1 + scale[:, None]) * F.rms_norm(hi, (d.hidden,), eps=d.eps) + shift[:, None], "final_x")
    return F.linear(x, tt(mw["final_w"]), tt(mw["final_b"])).numpy(), temb.numpy(), txt.numpy()


def test_backbone_matches_library_composition():
    wl, d, mw, inp = micro_backbone(seed=52, B=2, T=4, grid=(2, 3), valid=(3, 1), in_ch=8)
    td = S.text_block_dims(TEXT_MICRO)
    got = O.backbone_forward(inp["x"], inp["enc"], inp["timestep"], inp["position_ids"], inp["mask"], mw, d,
                             td, wl.T, time_dim=16)
    ref = torch_backbone(wl, d, mw, inp, td)[0]
    assert got.shape == (2, wl.N, 8)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)


def test_backbone_padded_text_cannot_change_velocity():
    wl, d, mw, inp = micro_backbone(seed=53, B=2, T=4, grid=(2, 2), valid=(3, 2), in_ch=8)
    td = S.text_block_dims(TEXT_MICRO)
    run = lambda enc: O.backbone_forward(inp["x"], enc, inp["timestep"], inp["position_ids"], inp["mask"], mw, d,
                                         td, wl.T, time_dim=16)
    a = run(inp["enc"])
    enc2 = inp["enc"].copy()
    enc2[0, 3:] = 4.0
    enc2[1, 2:] = -4.0
    np.testing.assert_array_equal(a, run(enc2))


# ----------------------------------------------------------------------------------------------
# Defaults and work accounting
# ----------------------------------------------------------------------------------------------
def test_defaults_match_api_page():
    g = json.load(open(os.path.join(GOLDEN, "krea2_defaults.json")))
    m = S.ModelDims()
    b, t = m.block, m.text
    assert (m.in_channels, m.num_layers, m.timestep_embed_dim) == (g["in_channels"], g["num_layers"], g["timestep_embed_dim"])
    assert (b.head_dim, b.num_heads, b.num_kv_heads, b.intermediate) == (
        g["attention_head_dim"], g["num_attention_heads"], g["num_key_value_heads"], g["intermediate_size"])
    assert b.hidden == g["hidden_size"] == b.head_dim * b.num_heads
    assert tuple(b.axes_dims) == tuple(g["axes_dims_rope"]) and sum(b.axes_dims) == b.head_dim
    assert (b.rope_theta, b.eps) == (g["rope_theta"], g["norm_eps"])
    assert (t.hidden, t.num_layers, t.num_heads, t.num_kv_heads, t.intermediate, t.num_layerwise_blocks,
            t.num_refiner_blocks) == (g["text_hidden_dim"], g["num_text_layers"], g["text_num_attention_heads"],
                                      g["text_num_key_value_heads"], g["text_intermediate_size"],
                                      g["num_layerwise_text_blocks"], g["num_refiner_text_blocks"])


def test_block_flops_full_size():
    # Per token GEMM work of the full-size block: 2H(2 nh hd + 2 nkv hd) + 2 nh hd H + 6 H I.
    d = S.BlockDims()
    per_tok = 2 * 6144 * (2 * 6144 + 2 * 1536) + 2 * 6144 * 6144 + 6 * 6144 * 16384
    assert per_tok == 868_220_928
    wl = S.WORKLOADS["block1024"]
    f = O.block_flops(d, wl.B, wl.L, [wl.N + v for v in wl.valid])
    assert abs(f - 8.9650e12) / 8.9650e12 < 1e-4


# ----------------------------------------------------------------------------------------------
# bf16 operand rounding (the bf16 model's operand precision)
# ----------------------------------------------------------------------------------------------
def test_bf16_round_known_values():
    # bf16 keeps 7 mantissa bits: spacing 2^-7 at 1.0; halfway cases go to the even mantissa
    v = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -12, -2.5, 3.0e38, 1e-40, 0.0])
    r = O.bf16_round(v)
    np.testing.assert_array_equal(r[:4], [1.0, 1.0, 1 + 2 ** -6, 1 + 2 ** -7])
    assert r[4] == -2.5 and r[7] == 0.0


def test_bf16_round_matches_library_conversion():
    x = np.random.default_rng(2).standard_normal(100000).astype(np.float32) * 37
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.bf16_round(x), ref)


BLOCK_POINTS = ("x1", "q", "k", "v", "g", "p", "o", "og", "x2", "a")
BWD_POINTS = ("dz", "dgt", "du", "dy", "do", "dgraw", "dq", "dk", "dv", "ds")


def _np_hook(off):
    """The oracle's rounding at every named point except `off`."""
    return lambda x, point=None: x if point == off else O.bf16_round(x)


def _rnd_cases():
    d4 = S.BlockDims(hidden=64, num_heads=4, num_kv_heads=1, head_dim=16, intermediate=40,
                     axes_dims=(4, 6, 6), rope_theta=1000.0, eps=1e-5)
    yield "gqa2", MICRO, *micro_inputs(seed=61), None
    yield "gqa4", d4, *micro_inputs(seed=62, B=1, T=5, grid=(3, 2), valid=(4,), dims=d4), None
    wl, inp = micro_inputs(seed=63, modulated=False)
    inp["temb"], inp["position_ids"] = None, None
    yield "unmodulated", MICRO, wl, inp, None
    wl, inp = micro_inputs(seed=64, B=2, T=4, grid=(2, 3), valid=(3, 4))
    yield "block_causal", MICRO, wl, inp, np.array([-1, -1, -1, -1, 0, 0, 0, 1, 1, 1])


@pytest.mark.parametrize("flash", [False, True])
def test_block_bf16_mode_matches_library_composition(flash):
    # R13: the oracle's bf16 mode against the torch composition with torch's own bf16 conversion at
    # the same named points, in both softmax rounding forms; and it is not the exact function.
    for name, d, wl, inp, ids in _rnd_cases():
        args = (inp["h"], inp["temb"], inp["position_ids"], inp["mask"], inp["weights"], d, wl.T)
        got = O.block_forward(*args, rnd=O.bf16_round, image_ids=ids, flash=flash)
        ref = torch_block(*args, image_ids=ids, rnd=torch_bf16, flash=flash)
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11, err_msg=name)
        exact = O.block_forward(*args, image_ids=ids)
        assert np.abs(got - exact).max() > 1e-6 * np.sqrt(np.mean(exact ** 2)), name


def test_block_bf16_each_point_is_applied_where_the_composition_applies_it():
    # Switching one named point off on both sides keeps them equal (the point sits at the same place
    # in both) and changes the result (the point is applied), for every point of the block.
    _, d, wl, inp, _ = next(_rnd_cases())
    args = (inp["h"], inp["temb"], inp["position_ids"], inp["mask"], inp["weights"], d, wl.T)
    full = O.block_forward(*args, rnd=O.bf16_round)
    rms = np.sqrt(np.mean(full ** 2))
    for point in BLOCK_POINTS:
        got = O.block_forward(*args, rnd=_np_hook(point))
        ref = torch_block(*args, rnd=skip_point(point))
        np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11, err_msg=point)
        assert np.abs(got - full).max() > 1e-6 * rms, f"point {point} has no effect"


def test_block_bf16_mode_forms_and_identity_hook():
    # An identity hook gives the exact function bit for bit; the two softmax rounding forms agree
    # without rounding and differ with it.
    _, d, wl, inp, _ = next(_rnd_cases())
    args = (inp["h"], inp["temb"], inp["position_ids"], inp["mask"], inp["weights"], d, wl.T)
    exact = O.block_forward(*args)
    np.testing.assert_array_equal(O.block_forward(*args, rnd=lambda x, point=None: x), exact)
    np.testing.assert_allclose(O.block_forward(*args, flash=True), exact, rtol=1e-12, atol=1e-13)
    a = O.block_forward(*args, rnd=O.bf16_round)
    b = O.block_forward(*args, rnd=O.bf16_round, flash=True)
    assert np.abs(a - b).max() > 1e-7 * np.sqrt(np.mean(exact ** 2))
    # rounding every point leaves zero gates the identity (weights, h and temb are bf16 values)
    w = dict(inp["weights"])
    H = d.hidden
    tab = w["scale_shift_table"].astype(np.float64).copy()
    tab[2] = -inp["temb"][0, 2 * H:3 * H]
    tab[5] = -inp["temb"][0, 5 * H:6 * H]
    w["scale_shift_table"] = tab
    got = O.block_forward(inp["h"][:1], inp["temb"][:1], inp["position_ids"], inp["mask"][:1], w, d, wl.T,
                          rnd=O.bf16_round)
    np.testing.assert_array_equal(got, inp["h"][:1].astype(np.float64))


DELTA_FREE = ("ff_down", "ff_gate", "ff_up", "norm2_w", "to_out", "to_v", "to_gate")


def _bwd_rnd(case, hook_np, hook_t):
    d, wl, inp, ids = _bwd_case(case)
    w = inp["weights"]
    dh_out = np.random.default_rng(72).standard_normal(inp["h"].shape)
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64)).requires_grad_(True)
    ht = t(inp["h"])
    tt = None if inp["temb"] is None else t(inp["temb"])
    wt = {key: (None if val is None else t(val)) for key, val in w.items()}
    out = torch_block_t(ht, tt, inp["position_ids"], inp["mask"], wt, d, wl.T, image_ids=ids, rnd=hook_t)
    out.backward(torch.from_numpy(dh_out))
    dh, dtemb, grads = O.block_backward(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], w, d, wl.T, dh_out,
                                        rnd=hook_np, image_ids=ids)
    ref = {key: val.grad.numpy() for key, val in wt.items() if val is not None}
    ref["h"] = ht.grad.numpy()
    got = {key: val for key, val in grads.items() if val is not None}
    got["h"] = dh
    if tt is not None:
        ref["temb"], got["temb"] = tt.grad.numpy(), dtemb
    return got, ref


@pytest.mark.parametrize("case", ["gqa2", "block_causal"])
def test_block_backward_bf16_mode_matches_autograd_with_hooks(case):
    # R20 in bf16 mode against autograd through the composition, with forward rounding (straight
    # through) and gradient rounding at the same named points. The oracle's softmax gradient uses
    # rowsum(dO * O) with O the attention output the model holds (rounded P and o), autograd uses
    # rowsum(dP * P) with P unrounded; with "p" and "o" off the two are the same quantity, so every
    # gradient must agree. With every point on, the gradients that do not pass through the softmax
    # gradient must still agree exactly.
    hook_np = lambda x, point=None: x if point in ("p", "o") else O.bf16_round(x)
    hook_t = lambda x, point=None: x if point in ("p", "o") else torch_bf16(x)
    got, ref = _bwd_rnd(case, hook_np, hook_t)
    for key in ref:
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-9, atol=1e-10, err_msg=key)
    got, ref = _bwd_rnd(case, O.bf16_round, torch_bf16)
    for key in DELTA_FREE:
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-9, atol=1e-10, err_msg=key)


def test_block_backward_bf16_each_point_is_applied():
    d, wl, inp, _ = _bwd_case("gqa2")
    w = inp["weights"]
    dh_out = np.random.default_rng(73).standard_normal(inp["h"].shape)
    run = lambda r: O.block_backward(inp["h"], inp["temb"], inp["position_ids"], inp["mask"], w, d, wl.T, dh_out,
                                     rnd=r)
    full = run(O.bf16_round)
    flat = lambda res: np.concatenate([res[0].ravel(), res[1].ravel()] +
                                      [v.ravel() for v in res[2].values() if v is not None])
    f = flat(full)
    for point in BLOCK_POINTS + BWD_POINTS:
        diff = np.abs(flat(run(_np_hook(point))) - f).max()
        assert diff > 1e-6 * np.sqrt(np.mean(f ** 2)), f"point {point} has no effect on the backward"


def test_time_text_backbone_bf16_mode_match_library_composition():
    # R13's time-path, text and final-layer points, against the torch compositions with the hook.
    # Each point is checked where it acts first (time path -> temb, text -> the text rows, final
    # layer -> the velocity): downstream, later rounding points can absorb a small change.
    wl, d, mw, inp = micro_backbone(seed=54, B=2, T=4, grid=(2, 3), valid=(3, 1), in_ch=8)
    td = S.text_block_dims(TEXT_MICRO)
    run = lambda r: O.backbone_forward(inp["x"], inp["enc"], inp["timestep"], inp["position_ids"], inp["mask"], mw,
                                       d, td, wl.T, time_dim=16, rnd=r)
    got = run(O.bf16_round)
    ref, _, _ = torch_backbone(wl, d, mw, inp, td, rnd=torch_bf16)
    np.testing.assert_allclose(got, ref, rtol=1e-10, atol=1e-11)
    parts = lambda r: (O.time_path(inp["timestep"], mw["time"], 16, rnd=r)[0],
                       O.text_embed(inp["enc"], inp["mask"], mw, td, rnd=r), run(r))
    full = parts(O.bf16_round)
    where = {"temb_in": 0, "temb_act": 0, "temb_e": 0, "text_fused": 1, "final_x": 2}
    for point, i in where.items():
        a = parts(_np_hook(point))
        b = torch_backbone(wl, d, mw, inp, td, rnd=skip_point(point))
        for x, y in zip(a, (b[1], b[2], b[0])):
            np.testing.assert_allclose(x, y, rtol=1e-10, atol=1e-11, err_msg=point)
        assert np.abs(a[i] - full[i]).max() > 1e-7 * np.sqrt(np.mean(full[i] ** 2)), f"point {point} has no effect"


def test_float32_product_form():
    # R13's f32_products form: the products are float32 matrix products (torch's float32 matmul on the
    # same operands), and without rounding points the block stays within float32 accuracy of the
    # exact function; with them it is a different realisation of the bf16 model than the float64 form.
    g = np.random.default_rng(80)
    a, b = g.standard_normal((3, 7, 33)), g.standard_normal((33, 5))
    ref = (torch.from_numpy(a).float() @ torch.from_numpy(b).float()).double().numpy()
    np.testing.assert_allclose(O._mm32(a, b), ref, rtol=1e-5, atol=1e-5)
    _, d, wl, inp, _ = next(_rnd_cases())
    args = (inp["h"], inp["temb"], inp["position_ids"], inp["mask"], inp["weights"], d, wl.T)
    exact = O.block_forward(*args)
    rms = np.sqrt(np.mean(exact ** 2))
    assert np.abs(O.block_forward(*args, f32_products=True) - exact).max() < 1e-5 * rms
    c = O.block_forward(*args, rnd=O.bf16_form(flash=True, f32_products=True))
    np.testing.assert_array_equal(c, O.block_forward(*args, rnd=O.bf16_round, flash=True, f32_products=True))
    assert np.abs(c - O.block_forward(*args, rnd=O.bf16_round, flash=True)).max() > 0.0
    dh_out = g.standard_normal(inp["h"].shape)
    bx = O.block_backward(*args, dh_out)
    bf = O.block_backward(*args, dh_out, flash=True, f32_products=True)
    np.testing.assert_allclose(bf[0], bx[0], rtol=1e-4, atol=1e-5 * np.abs(bx[0]).max())
