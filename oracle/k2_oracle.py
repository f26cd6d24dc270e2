"""CPU oracle for the Krea 2 single-stream MMDiT block, its text fusion, time path and backbone.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and the CPU-baseline leg of
bench.py may import this module. The product path (flow_matching_diffusion_amd) never imports,
calls or links it, and it shares no code with the HIP kernels.

Everything is plain NumPy in float64: a matrix product (`@`) is the only library primitive used
as a step; there is no blocking, fusion or reordering beyond what the definitions state.

Sources (cited by page title and section; the pages hold no code listing we follow line by line):
  [API]      diffusers v0.43.0 model page "Krea2Transformer2DModel" (constructor signature and
             parameter list; forward() parameters and return value).
  [ARTICLE]  article "Diffusers 中的 Krea2Transformer2DModel：Krea 2 单流 MMDiT 流匹配 Transformer
             架构全解", sections 一 (positioning) .. 八 (summary); §四.1..§四.6 are the module items
             (1 TextFusion, 2 TransformerBlock, 3 Attention, 4 RMSNorm, 5 TimestepEmbedding,
             6 FinalLayer) and the unnumbered "data flow" list that opens §四.
  [PIPELINE] diffusers v0.43.0 pipeline page "Krea 2" (Krea2Pipeline, prepare_position_ids,
             get_text_hidden_states, the guidance convention).
  [QWEN21]   diffusers model page "QwenImage21Transformer2DModel" (block-causal attention item;
             build_token_metadata and its image_ids).

Readings where the pages are silent or garbled (each restated where it is used):
  R1  modulation = temb split in 6 chunks + per-block table; x -> (1 + scale) * norm(x) + shift;
      h -> h + gate * branch (the article's block code lost its '=' and '+' signs).
  R2  RMSNorm: x / sqrt(mean(x^2) + eps) * (1 + w); eps inside the root; w is zero-centred.
  R3  softmax scale 1/sqrt(head_dim) (scaled-dot-product default).
  R4  GQA: query head hq reads kv head hq // (num_heads / num_kv_heads) (repeat_interleave).
  R5  mask: key padding only, text keys only; image keys always valid; no causal mask.
  R6  sigmoid output gate: elementwise on the concatenated heads, computed from the attention
      input, applied before the output projection.
  R7  no bias in q/k/v/gate/out/SwiGLU projections; img_in, time MLP, time_mod_proj, txt_in and
      the final projection carry biases.
  R8  RoPE: interleaved adjacent pairs (2i, 2i+1); head dim split (t, h, w) in that order; pair i
      of an axis with width d turns by pos * theta^(-2i/d); applied after the q/k norm.
  R9  SwiGLU: down(silu(gate(x)) * up(x)).
  R10 time path: s = 1000 t; emb = [cos(s f_k)] ++ [sin(s f_k)], f_k = 10000^(-k/half), k < half;
      e = lin2(gelu_tanh(lin1(emb))); temb = mod_proj(gelu_tanh(e)).
  R11 final layer: (scale, shift) = table[0] + e, table[1] + e (e: time embedding before the
      GELU); out = proj((1 + scale) * RMSNorm(h_img) + shift); the norm has no weight by default.
  R12 text fusion block: pre-norm block with the same attention (q/k norm, sigmoid gate), MHA,
      no RoPE, no modulation; layer compressor Linear(num_layers, 1) without bias; txt_in is a
      plain Linear with bias.
  R13 bf16 operands: the model runs in bfloat16 ([PIPELINE] examples load it with
      torch_dtype=bfloat16) and RMSNorm computes in float32 and casts back to the model dtype
      ([ARTICLE] §四.4). With `rnd=bf16_round` the oracle rounds to bf16 exactly where the bf16
      model holds a bf16 tensor that a later step consumes. Each such place is a named rounding
      point, and rnd(x, point) is called with its name, so a caller can switch single points off:
        block: "x1", "x2" (modulated norm outputs), "q", "k" (after norm and RoPE), "v", "g" (the
               projections), "p" (the attention probabilities entering the P V product), "o" (the
               attention output, a bf16 tensor in the bf16 model), "og" (the gated attention output
               entering the out projection), "a" (the SwiGLU activation entering the down product);
        time path: "temb_in", "temb_act", "temb_e" (the three time-MLP inputs);
        text: "text_fused" (the fused text before txt_in); final layer: "final_x";
        sampler: "latents" (the transformer input drawn from the float state).
      Elementwise steps between two points (the gate product, SiLU, modulation) run in full
      precision. Everything else (residual stream, statistics, softmax, accumulation) stays
      float64. rnd=None is the exact function.
      Softmax rounding form: the plain definition rounds the normalised probabilities (softmax,
      then the bf16 P V product), which is the default. flash=True takes the other legitimate form
      of the same bf16 model, that of fused (flash) attention: the unnormalised exp(s - rowmax) is
      rounded for the product and the row sum is taken before rounding and divided at the end. The
      two forms differ only in where the probabilities are rounded. f32_products=True is a third
      legitimate form: every matrix product accumulates in float32, as matrix cores do, instead of
      float64. In the fused form the running maximum may lag the row maximum (a fused kernel that
      rescales only on large growth): lag_seed draws that lag, which re-draws the probabilities'
      rounding. The spread between these forms measures how much any bf16 implementation may
      legitimately differ from the plain one (a small change anywhere re-draws the rounding of
      every later point).
  R14 sampler shift ([PIPELINE] Krea2Pipeline, scheduler and is_distilled parameters): mu is the
      straight line through (base_image_seq_len, base_shift) = (256, 0.5) and
      (max_image_seq_len, max_shift) = (6400, 1.15) evaluated at the image token count; the
      distilled checkpoint uses mu = 1.15. The named "exponential time shift" is taken as
      sigma -> e^mu / (e^mu + (1/sigma - 1)), which fixes sigma = 1 and is the identity at mu = 0.
  R15 sigma grid ([PIPELINE] __call__, sigmas parameter): linspace(1, 1/N, N), shifted, then a
      terminal 0 appended (N + 1 values); the transformer is called at timestep t = sigma_i (its
      time path multiplies by 1000, R10).
  R16 update ([PIPELINE] __call__, guidance_scale parameter): v = cond + g (cond - uncond), with the
      uncond pass skipped when g <= 0; the Euler step is x <- x + (sigma_{i+1} - sigma_i) v. The
      latent state is kept in float32 between steps.
  R17 block-causal attention ([QWEN21], block-causal attention item and build_token_metadata):
      query i may attend key j iff j <= i or i and j lie in the same image block, where image_ids
      gives -1 for tokens outside every image block and one id >= 0 per block; it combines with
      the key-padding mask of R5 (both must allow the key). A query left with no key gets a zero
      attention output (its softmax has no terms).
  R20 backward pass ([ARTICLE] §四 data flow and §六: the model is trained, and its test matrix
      includes training and gradient checkpointing): the gradient of the block's output with
      respect to its input h, its modulation input temb and every weight, by the chain rule through
      the forward's steps, the forward recomputed from h (checkpointing). In bf16 mode the forward
      part rounds at the same named points as block_forward (R13: "p" normalised, "o" the bf16
      attention output), and the backward's matrix-product operands are bf16 as well: the
      gradients that enter a product ("dz", "dgt", "du", "dy", "do", "dgraw", "dq", "dk", "dv")
      and dS inside attention ("ds"), with float32 accumulation and float32 weight gradients. The
      rounded attention output enters the gate's and the softmax's gradients.
"""
from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def _f64(a):
    return None if a is None else np.asarray(a, dtype=F64)


def _id(x, point=None):
    return x


def bf16_form(flash=False, f32_products=False, lag_seed=None):
    """bf16 rounding at R13's named points in one of R13's legitimate forms: the returned rounding
    function carries the softmax rounding form, the product accumulation type and (fused form
    only) the seed of the running-maximum lag, which block_forward reads when its own arguments
    are left at None, so the form also reaches the blocks inside text fusion and the backbone."""
    def rnd(x, point=None):
        return bf16_round(x)
    rnd.flash, rnd.f32_products, rnd.lag_seed = bool(flash), bool(f32_products), lag_seed
    return rnd


def _mm32(a, b):
    """Matrix product with float32 operands and float32 accumulation, widened back to float64: how
    matrix cores accumulate (the emulation R13 calls f32_products)."""
    return (np.asarray(a, np.float32) @ np.asarray(b, np.float32)).astype(F64)


def bf16_round(x, point=None):
    """Round to the nearest bfloat16 (ties to even) via float32; returns float64 (R13).
    A bfloat16 is the upper 16 bits of a float32, so rounding adds half of the dropped range
    (0x7FFF, plus 1 when the kept lsb is odd) and clears the low 16 bits. point names the rounding
    point (R13); every point rounds the same way here."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(F64)


# ----------------------------------------------------------------------------------------------
# Elementwise pieces
# ----------------------------------------------------------------------------------------------
def rms_norm(x, weight, eps):
    """Zero-centred RMSNorm, [ARTICLE] §四.4 (effective multiplier 1 + weight; statistics in
    full precision) with eps inside the root (R2); the eps value is norm_eps of [API]."""
    x = _f64(x)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    if weight is not None:
        y = y * (1.0 + _f64(weight))
    return y


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    return x * sigmoid(x)


def gelu_tanh(x):
    """GELU with the tanh approximation ([ARTICLE] §四.5 names GELU-tanh for the time MLP)."""
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


# ----------------------------------------------------------------------------------------------
# Rotary position embedding
# ----------------------------------------------------------------------------------------------
def rope_angles(position_ids, axes_dims, theta):
    """Rotation angle of every (token, pair): [API] axes_dims_rope / rope_theta and the
    position_ids parameter; [ARTICLE] §一 (3-axis RoPE of the Flux family) and §四.3 (R8).
    Returns (L, sum(axes_dims) / 2)."""
    pos = _f64(position_ids)
    cols = []
    for a, d in enumerate(axes_dims):
        i = np.arange(d // 2, dtype=F64)
        freq = float(theta) ** (-2.0 * i / d)
        cols.append(pos[:, a:a + 1] * freq[None, :])
    return np.concatenate(cols, axis=1)


def apply_rope(x, angles):
    """Rotate adjacent pairs (x[2i], x[2i+1]) by angles[..., i] (R8). x: (..., L, hd)."""
    c, s = np.cos(angles), np.sin(angles)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


# ----------------------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------------------
def attention(q, k, v, key_valid, visible=None, rnd=None, flash=False, f32_products=False, lag_seed=None):
    """Softmax attention with GQA and a key mask, [ARTICLE] §四.3.
    q: (B, nh, Lq, hd); k, v: (B, nkv, Lk, hd); key_valid: (B, Lk) bool or None; visible: (Lq, Lk)
    bool or None, which keys each query may attend (the same for every batch row and head; R17).
    Query head hq reads kv head hq // (nh / nkv) (repeat_interleave, R4); scale 1/sqrt(hd) (R3).
    A query row with no allowed key returns zeros (R17). rnd rounds the probabilities at "p" where
    they enter the P V product (R13); flash selects where (R13's softmax rounding form);
    f32_products accumulates the two products in float32 (R13); lag_seed (fused form): the
    probabilities are formed against a running maximum that lags the row maximum by a seeded
    amount in [0, 8) (log2 units), as a fused kernel that rescales only on large growth holds them,
    which scales exp(s - max) by 2^lag before rounding and cancels in the division. Heads are taken
    one at a time, which bounds memory and changes no arithmetic."""
    r = rnd or _id
    mm = _mm32 if f32_products else np.matmul
    B, nh, Lq, hd = q.shape
    nkv, Lk = k.shape[1], k.shape[2]
    g = nh // nkv
    allowed = np.ones((B, Lq, Lk), dtype=bool)
    if key_valid is not None:
        allowed &= np.asarray(key_valid, dtype=bool)[:, None, :]
    if visible is not None:
        allowed &= visible[None]
    some = allowed.any(axis=-1, keepdims=True)
    out = np.empty((B, nh, Lq, v.shape[-1]), dtype=F64)
    lag = None
    if flash and lag_seed is not None:
        lag = np.random.default_rng(lag_seed).random((B, nh, Lq, 1)) * 8.0 * math.log(2.0)
    for hq in range(nh):
        kh, vh = _f64(k[:, hq // g]), _f64(v[:, hq // g])
        s = mm(_f64(q[:, hq]), np.swapaxes(kh, -1, -2)) / math.sqrt(hd)
        s = np.where(allowed, s, -np.inf)
        s = s - np.where(some, np.max(s, axis=-1, keepdims=True), 0.0)
        e = np.exp(s if lag is None else s + lag[:, hq])
        denom = np.where(some, np.sum(e, axis=-1, keepdims=True), 1.0)
        if flash:
            out[:, hq] = mm(r(e, "p"), vh) / denom
        else:
            out[:, hq] = mm(r(e / denom, "p"), vh)
    return out


def block_causal_visible(image_ids, rows=None):
    """(Lq, L) bool: query i may attend key j iff j <= i or both carry the same image id >= 0 (R17).
    image_ids: (L,) ints; rows: the query indices (None = all)."""
    ids = np.asarray(image_ids)
    L = ids.size
    qi = np.arange(L) if rows is None else np.asarray(rows)
    j = np.arange(L)
    same = (ids[qi][:, None] >= 0) & (ids[qi][:, None] == ids[None, :])
    return (j[None, :] <= qi[:, None]) | same


def key_valid_mask(B, L, T, mask):
    """(B, L) key validity: text key j < T is valid iff mask[b, j]; image keys always (R5).
    mask None means every text token is valid ([API] encoder_attention_mask)."""
    kv = np.ones((B, L), dtype=bool)
    if mask is not None:
        kv[:, :T] = np.asarray(mask).astype(bool)
    return kv


# ----------------------------------------------------------------------------------------------
# The single-stream block
# ----------------------------------------------------------------------------------------------
def modulation(temb, table):
    """[ARTICLE] §四.2: temb (B, 6H) unflattened to (B, 6, H) plus the block's (6, H) table;
    chunks are prescale, preshift, pregate, postscale, postshift, postgate (R1)."""
    B = temb.shape[0]
    H = table.shape[1]
    return _f64(temb).reshape(B, 6, H) + _f64(table)[None]


def block_forward(h, temb, position_ids, mask, w, dims, T, rows=None, intermediates=False, rnd=None,
                  image_ids=None, flash=None, f32_products=None):
    """One Krea2TransformerBlock forward ([ARTICLE] §四.2 block, §四.3 attention, §四.4 norm).

    h: (B, L, H) residual stream; temb: (B, 6H) or None (no modulation: text-fusion blocks);
    position_ids: (L, 3) or None (no RoPE); mask: (B, T) or None; w: weight dict (nn.Linear
    (out, in) layout); dims: BlockDims-like; T: text tokens at the start of the sequence.
    rows: optional sorted sequence indices; only those output rows are computed (keys and
    values still come from every row). rnd: rounding of R13 at its named points (None = exact);
    flash: R13's softmax rounding form; f32_products: every matrix product accumulates in float32
    (R13); both default to the form rnd carries (bf16_form), else False. image_ids: (L,) block ids for the block-causal attention of R17 (None = every key
    visible).
    Returns (B, len(rows) or L, H) float64.
    """
    flash = getattr(rnd, "flash", False) if flash is None else flash
    f32_products = getattr(rnd, "f32_products", False) if f32_products is None else f32_products
    lag_seed = getattr(rnd, "lag_seed", None)
    rnd = rnd or _id
    mm = _mm32 if f32_products else np.matmul
    h = _f64(h)
    B, L, H = h.shape
    nh, nkv, hd, eps = dims.num_heads, dims.num_kv_heads, dims.head_dim, dims.eps
    rows = np.arange(L) if rows is None else np.asarray(rows)
    R = rows.size
    out = {}

    if temb is not None:
        mod = modulation(temb, w["scale_shift_table"])
        ps, pt, pg, qs, qt, qg = (mod[:, i, None, :] for i in range(6))
    else:
        ps = pt = qs = qt = 0.0
        pg = qg = 1.0

    # (1 + prescale) * norm1(h) + preshift
    x1 = rnd((1.0 + ps) * rms_norm(h, w["norm1_w"], eps) + pt, "x1")
    out["x1"] = x1

    # projections (R7: no bias); k and v for every row, q and gate for the requested rows
    k = mm(x1, _f64(w["to_k"]).T)
    v = rnd(mm(x1, _f64(w["to_v"]).T), "v")
    xr = x1[:, rows]
    q = mm(xr, _f64(w["to_q"]).T)
    graw = rnd(mm(xr, _f64(w["to_gate"]).T), "g")

    q = q.reshape(B, R, nh, hd).transpose(0, 2, 1, 3)
    k = k.reshape(B, L, nkv, hd).transpose(0, 2, 1, 3)
    v = v.reshape(B, L, nkv, hd).transpose(0, 2, 1, 3)

    # per-head q/k RMSNorm over head_dim, then RoPE (R8)
    q = rms_norm(q, w["norm_q_w"], eps)
    k = rms_norm(k, w["norm_k_w"], eps)
    if position_ids is not None:
        ang = rope_angles(position_ids, dims.axes_dims, dims.rope_theta)
        q = apply_rope(q, ang[rows][None, None])
        k = apply_rope(k, ang[None, None])
    q, k = rnd(q, "q"), rnd(k, "k")
    out["q"], out["k"], out["v"], out["g"] = q, k, v, graw

    vis = None if image_ids is None else block_causal_visible(image_ids, rows)
    o = attention(q, k, v, key_valid_mask(B, L, T, mask), vis, rnd=rnd, flash=flash, f32_products=f32_products,
                  lag_seed=lag_seed)
    o = rnd(o.transpose(0, 2, 1, 3).reshape(B, R, nh * hd), "o")
    og = rnd(o * sigmoid(graw), "og")                        # R6
    out["o"], out["og"] = o, og

    h1 = h[:, rows] + pg * mm(og, _f64(w["to_out"]).T)
    out["h1"] = h1
    x2 = rnd((1.0 + qs) * rms_norm(h1, w["norm2_w"], eps) + qt, "x2")
    out["x2"] = x2
    a = rnd(silu(mm(x2, _f64(w["ff_gate"]).T)) * mm(x2, _f64(w["ff_up"]).T), "a")   # R9
    out["a"] = a
    h2 = h1 + qg * mm(a, _f64(w["ff_down"]).T)
    out["out"] = h2
    return (h2, out) if intermediates else h2


# ----------------------------------------------------------------------------------------------
# Backward pass of the block (R20)
# ----------------------------------------------------------------------------------------------
def rms_norm_backward(x, weight, eps, dy):
    """Gradients of y = x r (1 + w), r = 1/sqrt(mean(x^2) + eps), over the last axis, for the output
    gradient dy: returns (dx, dw summed over all leading axes)."""
    x, dy = _f64(x), _f64(dy)
    H = x.shape[-1]
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    mult = 1.0 + (_f64(weight) if weight is not None else 0.0)
    dw = (dy * x * r).reshape(-1, H).sum(axis=0)
    g = dy * mult
    dx = r * g - x * r ** 3 * np.sum(g * x, axis=-1, keepdims=True) / H
    return dx, dw


def attention_backward(q, k, v, key_valid, do, visible=None, rnd=None, o=None, f32_products=False):
    """Gradients of attention() (same arguments) for the output gradient do (B, nh, Lq, hd):
    returns (dq, dk, dv) with dk, dv summed over the query heads that share each kv head (R4).
    With P the softmax probabilities and O = P V: dV = P^T dO, dP = dO V^T,
    dS = P (dP - rowsum(dO * O)), dQ = dS K / sqrt(hd), dK = dS^T Q / sqrt(hd). rnd (R20) rounds P
    (at "p", normalised, as in attention()) and dS (at "ds") where they become matrix-product
    operands; o, if given, is the forward output O as the model holds it (R20), used in
    rowsum(dO * O). f32_products: the products accumulate in float32 (R13)."""
    r = rnd or _id
    mm = _mm32 if f32_products else np.matmul
    nh, nkv, hd = q.shape[1], k.shape[1], q.shape[-1]
    g = nh // nkv
    kk = np.repeat(_f64(k), g, axis=1)
    vv = np.repeat(_f64(v), g, axis=1)
    s = mm(_f64(q), np.swapaxes(kk, -1, -2)) / math.sqrt(hd)
    allowed = np.ones(s.shape, dtype=bool)
    if key_valid is not None:
        allowed &= key_valid[:, None, None, :]
    if visible is not None:
        allowed &= visible[None, None]
    s = np.where(allowed, s, -np.inf)
    some = allowed.any(axis=-1, keepdims=True)
    s = s - np.where(some, np.max(s, axis=-1, keepdims=True), 0.0)
    p = np.exp(s)
    p = p / np.where(some, np.sum(p, axis=-1, keepdims=True), 1.0)
    do = _f64(do)
    o = mm(p, vv) if o is None else _f64(o)
    dvv = mm(np.swapaxes(r(p, "p"), -1, -2), do)
    dp = mm(do, np.swapaxes(vv, -1, -2))
    delta = np.sum(do * o, axis=-1, keepdims=True)
    ds = r(p * (dp - delta), "ds")
    dq = mm(ds, kk) / math.sqrt(hd)
    dkk = mm(np.swapaxes(ds, -1, -2), _f64(q)) / math.sqrt(hd)
    B, _, Lk, _ = k.shape
    dk = dkk.reshape(B, nkv, g, Lk, hd).sum(axis=2)
    dv = dvv.reshape(B, nkv, g, Lk, hd).sum(axis=2)
    return dq, dk, dv


def block_backward(h, temb, position_ids, mask, w, dims, T, dh_out, rnd=None, image_ids=None, flash=None,
                   f32_products=None):
    """Gradients of block_forward (same arguments) for the output gradient dh_out (B, L, H), by the
    chain rule through every step of the forward (R20). The forward is recomputed from h.
    Returns (dh, dtemb or None, grads) where grads holds the gradient of every weight in w (same
    keys and shapes; None for an absent norm weight). rnd as in block_forward; it also rounds the
    backward's matrix-product operands (R20). flash and f32_products as in block_forward (flash
    applies to the recomputed forward's attention)."""
    flash = getattr(rnd, "flash", False) if flash is None else flash
    f32_products = getattr(rnd, "f32_products", False) if f32_products is None else f32_products
    mm = _mm32 if f32_products else np.matmul
    r = rnd or _id
    h = _f64(h)
    dh2 = _f64(dh_out)
    B, L, H = h.shape
    nh, nkv, hd, eps = dims.num_heads, dims.num_kv_heads, dims.head_dim, dims.eps
    M = B * L
    # ---- forward, keeping what the backward needs
    if temb is not None:
        mod = modulation(temb, w["scale_shift_table"])
        ps, pt, pg, qs, qt, qg = (mod[:, i, None, :] for i in range(6))
    else:
        ps = pt = qs = qt = 0.0
        pg = qg = 1.0
    n1 = rms_norm(h, w["norm1_w"], eps)
    x1 = r((1.0 + ps) * n1 + pt, "x1")
    qraw = mm(x1, _f64(w["to_q"]).T).reshape(B, L, nh, hd).transpose(0, 2, 1, 3)
    kraw = mm(x1, _f64(w["to_k"]).T).reshape(B, L, nkv, hd).transpose(0, 2, 1, 3)
    v = r(mm(x1, _f64(w["to_v"]).T), "v").reshape(B, L, nkv, hd).transpose(0, 2, 1, 3)
    graw = r(mm(x1, _f64(w["to_gate"]).T), "g")
    qn = rms_norm(qraw, w["norm_q_w"], eps)
    kn = rms_norm(kraw, w["norm_k_w"], eps)
    ang = None
    if position_ids is not None:
        ang = rope_angles(position_ids, dims.axes_dims, dims.rope_theta)
        qn, kn = apply_rope(qn, ang[None, None]), apply_rope(kn, ang[None, None])
    q, k = r(qn, "q"), r(kn, "k")
    key_valid = key_valid_mask(B, L, T, mask)
    vis = None if image_ids is None else block_causal_visible(image_ids)
    o = r(attention(q, k, v, key_valid, vis, rnd=rnd, flash=flash, f32_products=f32_products,
                    lag_seed=getattr(rnd, "lag_seed", None)), "o")   # the attention output as the model holds it
    oc = o.transpose(0, 2, 1, 3).reshape(B, L, nh * hd)
    sg = sigmoid(graw)
    og = r(oc * sg, "og")
    y = mm(og, _f64(w["to_out"]).T)
    h1 = h + pg * y
    n2 = rms_norm(h1, w["norm2_w"], eps)
    x2 = r((1.0 + qs) * n2 + qt, "x2")
    gt = mm(x2, _f64(w["ff_gate"]).T)
    u = mm(x2, _f64(w["ff_up"]).T)
    sgt = sigmoid(gt)
    a = r(gt * sgt * u, "a")
    z = mm(a, _f64(w["ff_down"]).T)
    # ---- backward, step by step in reverse
    grads = {}
    flat = lambda t: t.reshape(M, -1)
    dqg = np.sum(dh2 * z, axis=1)
    dz = r(qg * dh2, "dz")
    grads["ff_down"] = mm(flat(dz).T, flat(a))
    da = mm(dz, _f64(w["ff_down"]))
    dgt = r(da * u * sgt * (1.0 + gt * (1.0 - sgt)), "dgt")      # silu'(x) = s(x) (1 + x (1 - s(x)))
    du = r(da * gt * sgt, "du")
    grads["ff_gate"] = mm(flat(dgt).T, flat(x2))
    grads["ff_up"] = mm(flat(du).T, flat(x2))
    dx2 = mm(dgt, _f64(w["ff_gate"])) + mm(du, _f64(w["ff_up"]))
    dqs = np.sum(dx2 * n2, axis=1)
    dqt = np.sum(dx2, axis=1)
    dh1_n, grads["norm2_w"] = rms_norm_backward(h1, w["norm2_w"], eps, (1.0 + qs) * dx2)
    dh1 = dh2 + dh1_n
    dpg = np.sum(dh1 * y, axis=1)
    dy = r(pg * dh1, "dy")
    grads["to_out"] = mm(flat(dy).T, flat(og))
    dog = mm(dy, _f64(w["to_out"]))
    do = r(dog * sg, "do").reshape(B, L, nh, hd).transpose(0, 2, 1, 3)
    dgraw = r(dog * oc * sg * (1.0 - sg), "dgraw")
    dq, dk, dv = attention_backward(q, k, v, key_valid, do, vis, rnd=rnd, o=o, f32_products=f32_products)
    if ang is not None:                                      # the rotation's transpose turns back
        dq, dk = apply_rope(dq, -ang[None, None]), apply_rope(dk, -ang[None, None])
    dqraw, grads["norm_q_w"] = rms_norm_backward(qraw, w["norm_q_w"], eps, dq)
    dkraw, grads["norm_k_w"] = rms_norm_backward(kraw, w["norm_k_w"], eps, dk)
    dqraw = r(dqraw.transpose(0, 2, 1, 3).reshape(B, L, nh * hd), "dq")
    dkraw = r(dkraw.transpose(0, 2, 1, 3).reshape(B, L, nkv * hd), "dk")
    dv = r(dv.transpose(0, 2, 1, 3).reshape(B, L, nkv * hd), "dv")
    grads["to_q"] = mm(flat(dqraw).T, flat(x1))
    grads["to_k"] = mm(flat(dkraw).T, flat(x1))
    grads["to_v"] = mm(flat(dv).T, flat(x1))
    grads["to_gate"] = mm(flat(dgraw).T, flat(x1))
    dx1 = (mm(dqraw, _f64(w["to_q"])) + mm(dkraw, _f64(w["to_k"])) + mm(dv, _f64(w["to_v"]))
           + mm(dgraw, _f64(w["to_gate"])))
    dps = np.sum(dx1 * n1, axis=1)
    dpt = np.sum(dx1, axis=1)
    dh_n, grads["norm1_w"] = rms_norm_backward(h, w["norm1_w"], eps, (1.0 + ps) * dx1)
    dh = dh1 + dh_n
    dtemb = None
    if temb is not None:
        dmod = np.stack([dps, dpt, dpg, dqs, dqt, dqg], axis=1)    # (B, 6, H), the chunk order of R1
        dtemb = dmod.reshape(B, 6 * H)
        grads["scale_shift_table"] = dmod.sum(axis=0)
    for key in ("norm1_w", "norm2_w", "norm_q_w", "norm_k_w"):
        if w.get(key) is None:
            grads[key] = None
    return dh, dtemb, grads


# ----------------------------------------------------------------------------------------------
# Time path
# ----------------------------------------------------------------------------------------------
def timestep_embedding(t, dim=256, max_period=10000.0, time_scale=1000.0):
    """Cos-first sinusoidal embedding of 1000 t, width dim ([ARTICLE] §四.5; [API]
    timestep_embed_dim; constants of R10)."""
    t = _f64(t)
    half = dim // 2
    freqs = max_period ** (-np.arange(half, dtype=F64) / half)
    arg = (time_scale * t)[:, None] * freqs[None, :]
    return np.concatenate([np.cos(arg), np.sin(arg)], axis=1)


def time_path(t, tw, dim=256, rnd=None):
    """time_embed -> GELU -> time_mod_proj ([ARTICLE] data flow of §四; R10; rnd: R13).
    Returns (temb (B, 6H), e (B, H)) where e is time_embed's output (before the GELU)."""
    rnd = rnd or _id
    emb = rnd(timestep_embedding(t, dim), "temb_in")
    h1 = rnd(gelu_tanh(emb @ _f64(tw["lin1_w"]).T + _f64(tw["lin1_b"])), "temb_act")
    e = h1 @ _f64(tw["lin2_w"]).T + _f64(tw["lin2_b"])
    temb = rnd(gelu_tanh(e), "temb_e") @ _f64(tw["mod_w"]).T + _f64(tw["mod_b"])
    return temb, e


# ----------------------------------------------------------------------------------------------
# Text fusion
# ----------------------------------------------------------------------------------------------
def text_fusion(enc, mask, tw, tdims, rnd=None):
    """Krea2TextFusion ([ARTICLE] §四.1; R12): layerwise blocks over the layer axis of every
    token, Linear(num_layers, 1) over the layer axis, refiner blocks over tokens with the mask.
    enc: (B, T, num_layers, D). Returns (B, T, D)."""
    enc = _f64(enc)
    B, T, NL, D = enc.shape
    x = enc.reshape(B * T, NL, D)
    for bw in tw["layerwise"]:
        x = block_forward(x, None, None, None, bw, tdims, T=0, rnd=rnd)
    y = np.tensordot(x, _f64(tw["compress_w"]), axes=([1], [0])).reshape(B, T, D)
    for bw in tw["refiner"]:
        y = block_forward(y, None, None, mask, bw, tdims, T=T, rnd=rnd)
    return y


# ----------------------------------------------------------------------------------------------
# Backbone
# ----------------------------------------------------------------------------------------------
def final_layer(h_img, e, table, norm_w, w, b, eps, rnd=None):
    """Krea2FinalLayer ([ARTICLE] §四.6; R11)."""
    rnd = rnd or _id
    scale = _f64(table)[0][None, None] + _f64(e)[:, None, :]
    shift = _f64(table)[1][None, None] + _f64(e)[:, None, :]
    x = rnd((1.0 + scale) * rms_norm(h_img, norm_w, eps) + shift, "final_x")
    return x @ _f64(w).T + _f64(b)


def text_embed(enc, mask, mw, tdims, rnd=None):
    """The backbone's text rows before the first block ([ARTICLE] data flow of §四): txt_in applied to
    the text-fusion output. Neither depends on the timestep or the latents. Returns (B, T, hidden)."""
    r = rnd or _id
    fused = r(text_fusion(enc, mask, mw["text"], tdims, rnd=rnd), "text_fused")
    return fused @ _f64(mw["txt_in_w"]).T + _f64(mw["txt_in_b"])


def backbone_stem(x, enc, t, mask, mw, tdims, time_dim=256, rnd=None):
    """What the backbone computes before its first block ([ARTICLE] data flow of §四): the time path,
    the text rows txt_in(text_fusion(enc)) and the image rows img_in(x), concatenated [text, image].
    Returns (h (B, T + N, hidden), temb (B, 6 hidden), e (B, hidden))."""
    temb, e = time_path(t, mw["time"], time_dim, rnd=rnd)
    txt = text_embed(enc, mask, mw, tdims, rnd=rnd)
    img = _f64(x) @ _f64(mw["img_in_w"]).T + _f64(mw["img_in_b"])
    return np.concatenate([txt, img], axis=1), temb, e


def backbone_head(h, e, mw, dims, T, rnd=None):
    """What follows the last block: the image rows only, through the final layer (R11)."""
    return final_layer(h[:, T:], e, mw["final_table"], mw.get("final_norm_w"), mw["final_w"], mw["final_b"],
                       dims.eps, rnd=rnd)


def backbone_forward(x, enc, t, position_ids, mask, mw, dims, tdims, T, time_dim=256, rnd=None):
    """Krea2Transformer2DModel.forward ([API] forward; [ARTICLE] data flow of §四):
    time path, text fusion + txt_in, img_in, concat [text, image], blocks, image rows only,
    final layer. mw["blocks"] may be any iterable of block weights (it is walked once).
    Returns the velocity (B, N, in_channels)."""
    h, temb, e = backbone_stem(x, enc, t, mask, mw, tdims, time_dim, rnd=rnd)
    for bw in mw["blocks"]:
        h = block_forward(h, temb, position_ids, mask, bw, dims, T=T, rnd=rnd)
    return backbone_head(h, e, mw, dims, T, rnd=rnd)


# ----------------------------------------------------------------------------------------------
# Sampler: flow-match Euler with the resolution-aware shift and CFG (R14 - R16)
# ----------------------------------------------------------------------------------------------
SHIFT_DEFAULTS = dict(base_shift=0.5, max_shift=1.15, base_image_seq_len=256, max_image_seq_len=6400,
                      distilled_mu=1.15)


def shift_mu(image_seq_len, distilled=False, base_shift=0.5, max_shift=1.15, base_image_seq_len=256,
             max_image_seq_len=6400, distilled_mu=1.15):
    """mu for an image of image_seq_len tokens: the line through the two (length, shift) points (R14)."""
    if distilled:
        return float(distilled_mu)
    slope = (max_shift - base_shift) / (max_image_seq_len - base_image_seq_len)
    return float(base_shift + slope * (image_seq_len - base_image_seq_len))


def time_shift(mu, sigma):
    """Exponential time shift e^mu / (e^mu + (1/sigma - 1)) (R14); sigma in (0, 1]."""
    sigma = np.asarray(sigma, dtype=F64)
    return math.exp(mu) / (math.exp(mu) + (1.0 / sigma - 1.0))


def flow_sigmas(num_steps, image_seq_len, distilled=False, **shift):
    """The N + 1 noise levels of the sampler (R15): shifted linspace(1, 1/N, N) then 0."""
    base = np.linspace(1.0, 1.0 / num_steps, num_steps, dtype=F64)
    mu = shift_mu(image_seq_len, distilled, **shift)
    return np.concatenate([time_shift(mu, base), [0.0]])


def cfg_velocity(v_cond, v_uncond, guidance):
    """Krea 2's guidance convention: cond + g (cond - uncond); cond alone when g <= 0 (R16)."""
    v_cond = _f64(v_cond)
    if guidance <= 0:
        return v_cond
    return v_cond + guidance * (v_cond - _f64(v_uncond))


def euler_step(x, v, sigma, sigma_next):
    """x + (sigma_next - sigma) v (R16)."""
    return _f64(x) + (float(sigma_next) - float(sigma)) * _f64(v)


def denoise_step(x, enc, enc_neg, mask, mask_neg, position_ids, mw, dims, tdims, T, sigma, sigma_next, guidance,
                 time_dim=256, rnd=None):
    """One sampler step on a single image: the transformer on the (cond, uncond) pair at t = sigma
    (cond only when guidance <= 0), the guidance combine and the Euler update. x: (1, N, C) latents;
    enc / enc_neg: (1, T, layers, D) prompt and negative-prompt stacks; masks (1, T) or None.
    The transformer input is x in the operand precision (rnd), the state stays float64."""
    r = rnd or _id
    xin = r(_f64(x), "latents")
    if guidance > 0:
        xb = np.concatenate([xin, xin], axis=0)
        eb = np.concatenate([_f64(enc), _f64(enc_neg)], axis=0)
        mb = None if mask is None else np.concatenate([mask, mask_neg], axis=0)
        t = np.array([sigma, sigma], dtype=F64)
        v = backbone_forward(xb, eb, t, position_ids, mb, mw, dims, tdims, T, time_dim=time_dim, rnd=rnd)
        vel = cfg_velocity(v[:1], v[1:], guidance)
    else:
        t = np.array([sigma], dtype=F64)
        vel = backbone_forward(xin, enc, t, position_ids, mask, mw, dims, tdims, T, time_dim=time_dim, rnd=rnd)
    return euler_step(x, vel, sigma, sigma_next)


# ----------------------------------------------------------------------------------------------
# Work accounting (used by the CPU baseline to express its throughput)
# ----------------------------------------------------------------------------------------------
def block_flops(dims, B, L, valid_keys, rows=None):
    """Algorithmic FLOPs of one block: every GEMM over the computed rows; attention over valid
    keys only; elementwise work not counted. valid_keys: per batch row, number of valid keys."""
    H, nh, nkv, hd, I = dims.hidden, dims.num_heads, dims.num_kv_heads, dims.head_dim, dims.intermediate
    R = L if rows is None else len(rows)
    kv = 2 * B * L * H * (2 * nkv * hd)
    per_row = 2 * H * (2 * nh * hd) + 2 * nh * hd * H + 3 * 2 * H * I
    attn = sum(4 * hd * nh * R * vk for vk in valid_keys)
    return kv + B * R * per_row + attn
