"""Python binding of libk2 — the MI355X (gfx950) Krea 2 single-stream MMDiT block library.

Argument marshalling only: every step of the computation runs in the HIP kernels behind the C ABI
(include/k2.h). PyTorch provides device memory (torch.empty) and the current HIP stream. Importing
this package does not load the library; the first call does, and fails loudly if it is not built.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

from . import _abi
from ._abi import K2Error, check, load

__all__ = ["K2Error", "load", "block_cfg", "text_cfg", "model_cfg", "block_forward", "block_workspace_layout",
           "timestep_modulation_forward", "text_fusion_forward", "backbone_forward", "upload",
           "profile_enable", "profile_reset", "profile_query", "DTYPES"]

DTYPES = {"f32": _abi.K2_F32, "bf16": _abi.K2_BF16}


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_tensor(t, name, dtype=None, shape=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


# ------------------------------------------------------------------------------------------------
# Configs
# ------------------------------------------------------------------------------------------------
def block_cfg(dims, dtype: str) -> _abi.BlockCfg:
    """k2_block_cfg from a BlockDims-like object (hidden, num_heads, num_kv_heads, head_dim,
    intermediate, axes_dims, rope_theta, eps)."""
    c = _abi.BlockCfg()
    c.hidden, c.num_heads, c.num_kv_heads = dims.hidden, dims.num_heads, dims.num_kv_heads
    c.head_dim, c.intermediate = dims.head_dim, dims.intermediate
    c.axes_dims[:] = list(dims.axes_dims)
    c.rope_theta, c.eps, c.dtype = float(dims.rope_theta), float(dims.eps), DTYPES[dtype]
    return c


def text_cfg(tdims, dtype: str) -> _abi.TextCfg:
    c = _abi.TextCfg()
    c.block.hidden, c.block.num_heads, c.block.num_kv_heads = tdims.hidden, tdims.num_heads, tdims.num_kv_heads
    c.block.head_dim, c.block.intermediate = tdims.head_dim, tdims.intermediate
    c.block.axes_dims[:] = [0, 0, 0]
    c.block.rope_theta, c.block.eps, c.block.dtype = 1000.0, float(tdims.eps), DTYPES[dtype]
    c.num_layers, c.num_layerwise_blocks, c.num_refiner_blocks = (tdims.num_layers, tdims.num_layerwise_blocks,
                                                                  tdims.num_refiner_blocks)
    return c


def model_cfg(dims, tdims, num_layers: int, in_channels: int, timestep_embed_dim: int, dtype: str) -> _abi.ModelCfg:
    c = _abi.ModelCfg()
    c.block = block_cfg(dims, dtype)
    c.text = text_cfg(tdims, dtype)
    c.num_layers, c.in_channels, c.timestep_embed_dim = num_layers, in_channels, timestep_embed_dim
    return c


# ------------------------------------------------------------------------------------------------
# Weights: host arrays -> device tensors (a copy; matrices in the operand dtype, the rest float32)
# ------------------------------------------------------------------------------------------------
_MATRICES = {"to_q", "to_k", "to_v", "to_gate", "to_out", "ff_gate", "ff_up", "ff_down", "lin1_w", "lin2_w", "mod_w",
             "img_in_w", "txt_in_w", "final_w"}


def upload(tree, dtype: str, device="cuda"):
    """Copy a (nested) dict/list of host arrays to the device: nn.Linear matrices in the operand dtype
    (values are already representable), everything else float32."""
    torch = _torch()
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    if isinstance(tree, dict):
        out = {}
        for k, v in tree.items():
            if isinstance(v, (dict, list)):
                out[k] = upload(v, dtype, device)
            elif v is None:
                out[k] = None
            else:
                t = torch.as_tensor(v)
                out[k] = t.to(device=device, dtype=td if k in _MATRICES else torch.float32).contiguous()
        return out
    if isinstance(tree, list):
        return [upload(v, dtype, device) for v in tree]
    raise TypeError(type(tree))


def _block_weights(w: dict) -> _abi.BlockWeights:
    s = _abi.BlockWeights()
    for n in _abi.BLOCK_WEIGHT_FIELDS:
        t = w.get(n)
        setattr(s, n, None if t is None else t.data_ptr())
    return s


def _block_weight_array(ws: list):
    arr = (_abi.BlockWeights * max(1, len(ws)))()
    for i, w in enumerate(ws):
        arr[i] = _block_weights(w)
    return arr


def _time_weights(w: dict) -> _abi.TimeWeights:
    s = _abi.TimeWeights()
    for n in _abi.TIME_WEIGHT_FIELDS:
        t = w.get(n)
        setattr(s, n, None if t is None else t.data_ptr())
    return s


def _mask_u8(mask):
    if mask is None:
        return None
    torch = _torch()
    return mask if mask.dtype == torch.uint8 else mask.to(torch.uint8)


def _workspace(nbytes: int, device, workspace):
    torch = _torch()
    if workspace is not None:
        return workspace
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------------------------
# Entry points
# ------------------------------------------------------------------------------------------------
@dataclass
class BlockLayout:
    x1: int
    q: int
    k: int
    vt: int
    g: int
    og: int
    x2: int
    a: int
    rope: int
    mod: int
    reach: int
    total: int
    ldvt: int


def block_workspace_layout(cfg, B: int, T: int, N: int) -> BlockLayout:
    lay = _abi.BlockLayout()
    check(load().k2_block_workspace_layout_query(ctypes.byref(cfg), B, T, N, ctypes.byref(lay)))
    return BlockLayout(lay.x1, lay.q, lay.k, lay.vt, lay.g, lay.og, lay.x2, lay.a, lay.rope, lay.mod, lay.reach,
                       lay.total, lay.ldvt)


def block_forward(cfg, weights: dict, h, temb, position_ids, mask, T: int, out=None, workspace=None, stream=None,
                  image_ids=None):
    """k2_block_forward, or k2_block_forward_block_causal when image_ids ((T+N,) int32 device tensor) is
    given. h: (B, T+N, hidden) float32; temb (B, 6 hidden) float32 or None; position_ids (T+N, 3)
    float32 or None; mask (B, T) bool/uint8 or None. Returns the output residual stream."""
    torch = _torch()
    lib = load()
    _dev_tensor(h, "h", torch.float32)
    B, L, _ = h.shape
    N = L - T
    out = torch.empty_like(h) if out is None else _dev_tensor(out, "out", torch.float32, h.shape)
    mask = _mask_u8(mask)
    pos_rows, pos_cols = (position_ids.shape if position_ids is not None else (0, 0))
    ws_bytes = lib.k2_block_workspace_bytes(ctypes.byref(cfg), B, T, N)
    ws = _workspace(ws_bytes, h.device, workspace)
    bw = _block_weights(weights)
    if image_ids is None:
        check(lib.k2_block_forward(ctypes.byref(cfg), ctypes.byref(bw), B, T, N, _ptr(h), _ptr(out), _ptr(temb),
                                   _ptr(position_ids), pos_rows, pos_cols, _ptr(mask), _ptr(ws), ws.numel(),
                                   _stream(stream)))
    else:
        _dev_tensor(image_ids, "image_ids", torch.int32, (L,))
        check(lib.k2_block_forward_block_causal(ctypes.byref(cfg), ctypes.byref(bw), B, T, N, _ptr(h), _ptr(out),
                                                _ptr(temb), _ptr(position_ids), pos_rows, pos_cols, _ptr(mask),
                                                _ptr(image_ids), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def block_forward_static_ws(cfg, weights: dict, h, temb, position_ids, mask, T: int, out=None, stream=None):
    """k2_block_forward_static_ws: k2_block_forward with the library's static device scratch instead of
    a workspace (nothing is allocated by the library; `out` is allocated here only when not given)."""
    torch = _torch()
    lib = load()
    _dev_tensor(h, "h", torch.float32)
    B, L, _ = h.shape
    out = torch.empty_like(h) if out is None else _dev_tensor(out, "out", torch.float32, h.shape)
    mask = _mask_u8(mask)
    pos_rows, pos_cols = (position_ids.shape if position_ids is not None else (0, 0))
    bw = _block_weights(weights)
    check(lib.k2_block_forward_static_ws(ctypes.byref(cfg), ctypes.byref(bw), B, T, L - T, _ptr(h), _ptr(out),
                                         _ptr(temb), _ptr(position_ids), pos_rows, pos_cols, _ptr(mask),
                                         _stream(stream)))
    return out


def block_backward_workspace_bytes(cfg, B: int, T: int, N: int) -> int:
    return load().k2_block_backward_workspace_bytes(ctypes.byref(cfg), B, T, N)


def block_backward(cfg, weights: dict, h, temb, position_ids, mask, T: int, grad_out, want=None, workspace=None,
                   stream=None):
    """k2_block_backward: gradients of the block for grad_out (the gradient of its output), the forward
    recomputed from h. want: weight names whose gradients to compute (None = every weight present).
    Returns (grad_in (B, L, hidden), grad_temb (B, 6 hidden) or None, {name: float32 gradient})."""
    torch = _torch()
    lib = load()
    _dev_tensor(h, "h", torch.float32)
    _dev_tensor(grad_out, "grad_out", torch.float32, h.shape)
    B, L, H = h.shape
    N = L - T
    mask = _mask_u8(mask)
    pos_rows, pos_cols = (position_ids.shape if position_ids is not None else (0, 0))
    grad_in = torch.empty_like(h)
    grad_temb = None if temb is None else torch.empty_like(temb)
    gs = _abi.BlockGrads()
    out = {}
    for n in _abi.BLOCK_WEIGHT_FIELDS:
        t = weights.get(n)
        if t is None or (want is not None and n not in want):
            setattr(gs, n, None)
            continue
        out[n] = torch.empty(t.shape, dtype=torch.float32, device=h.device)
        setattr(gs, n, out[n].data_ptr())
    ws = _workspace(lib.k2_block_backward_workspace_bytes(ctypes.byref(cfg), B, T, N), h.device, workspace)
    bw = _block_weights(weights)
    check(lib.k2_block_backward(ctypes.byref(cfg), ctypes.byref(bw), B, T, N, _ptr(h), _ptr(temb), _ptr(position_ids),
                                pos_rows, pos_cols, _ptr(mask), _ptr(grad_out), _ptr(grad_in), _ptr(grad_temb),
                                ctypes.byref(gs), _ptr(ws), ws.numel(), _stream(stream)))
    return grad_in, grad_temb, out


def timestep_modulation_forward(hidden: int, temb_dim: int, dtype: str, weights: dict, timestep, stream=None):
    """k2_timestep_modulation_forward. Returns (temb (B, 6 hidden), e (B, hidden)) float32."""
    torch = _torch()
    lib = load()
    _dev_tensor(timestep, "timestep", torch.float32)
    B = timestep.shape[0]
    cfg = _abi.TimeCfg(hidden, temb_dim, DTYPES[dtype])
    temb = torch.empty(B, 6 * hidden, dtype=torch.float32, device=timestep.device)
    e = torch.empty(B, hidden, dtype=torch.float32, device=timestep.device)
    ws = _workspace(lib.k2_timestep_modulation_workspace_bytes(ctypes.byref(cfg), B), timestep.device, None)
    tw = _time_weights(weights)
    check(lib.k2_timestep_modulation_forward(ctypes.byref(cfg), ctypes.byref(tw), B, _ptr(timestep), _ptr(temb),
                                             _ptr(e), _ptr(ws), ws.numel(), _stream(stream)))
    return temb, e


def text_fusion_forward(cfg, weights: dict, enc, mask, stream=None):
    """k2_text_fusion_forward. enc (B, T, num_layers, D) in the operand dtype. Returns (B, T, D) float32."""
    torch = _torch()
    lib = load()
    _dev_tensor(enc, "encoder_hidden_states")
    B, T, NL, D = enc.shape
    mask = _mask_u8(mask)
    out = torch.empty(B, T, D, dtype=torch.float32, device=enc.device)
    lw = _block_weight_array(weights["layerwise"])
    rf = _block_weight_array(weights["refiner"])
    tw = _abi.TextWeights(lw, weights["compress_w"].data_ptr(), rf)
    ws = _workspace(lib.k2_text_fusion_workspace_bytes(ctypes.byref(cfg), B, T), enc.device, None)
    check(lib.k2_text_fusion_forward(ctypes.byref(cfg), ctypes.byref(tw), B, T, _ptr(enc), _ptr(mask), _ptr(out),
                                     _ptr(ws), ws.numel(), _stream(stream)))
    return out


def _model_weights(w: dict):
    keep = []
    mw = _abi.ModelWeights()
    for n in ("img_in_w", "img_in_b", "txt_in_w", "txt_in_b", "final_table", "final_norm_w", "final_w", "final_b"):
        t = w.get(n)
        setattr(mw, n, None if t is None else t.data_ptr())
    mw.time = _time_weights(w["time"])
    lw = _block_weight_array(w["text"]["layerwise"])
    rf = _block_weight_array(w["text"]["refiner"])
    mw.text = _abi.TextWeights(lw, w["text"]["compress_w"].data_ptr(), rf)
    blocks = _block_weight_array(w["blocks"])
    mw.blocks = ctypes.cast(blocks, ctypes.POINTER(_abi.BlockWeights))
    keep += [lw, rf, blocks]
    return mw, keep


def backbone_forward(cfg, weights: dict, x, enc, timestep, position_ids, mask, workspace=None, stream=None):
    """k2_backbone_forward. x (B, N, in_channels) and enc (B, T, num_layers, D) in the operand dtype;
    timestep (B,) float32; position_ids (T+N, 3) float32. Returns the velocity (B, N, in_channels) float32."""
    torch = _torch()
    lib = load()
    _dev_tensor(x, "hidden_states")
    _dev_tensor(timestep, "timestep", torch.float32)
    B, N, C = x.shape
    T = enc.shape[1] if enc is not None else 0
    mask = _mask_u8(mask)
    out = torch.empty(B, N, C, dtype=torch.float32, device=x.device)
    mw, keep = _model_weights(weights)
    ws = _workspace(lib.k2_backbone_workspace_bytes(ctypes.byref(cfg), B, T, N), x.device, workspace)
    check(lib.k2_backbone_forward(ctypes.byref(cfg), ctypes.byref(mw), B, T, N, _ptr(x), _ptr(enc), _ptr(timestep),
                                  _ptr(position_ids), position_ids.shape[0], position_ids.shape[1], _ptr(mask),
                                  _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    del keep
    return out


def backbone_workspace_bytes(cfg, B: int, T: int, N: int) -> int:
    return load().k2_backbone_workspace_bytes(ctypes.byref(cfg), B, T, N)


def text_embed_workspace_bytes(cfg, B: int, T: int) -> int:
    return load().k2_text_embed_workspace_bytes(ctypes.byref(cfg), B, T)


def text_embed(cfg, weights: dict, enc, mask, workspace=None, stream=None):
    """k2_text_embed: txt_in(text_fusion(enc)) for the backbone's text rows, (B, T, hidden) float32.
    enc (B, T, layers, D) in the operand dtype; mask (B, T) or None."""
    torch = _torch()
    lib = load()
    _dev_tensor(enc, "encoder_hidden_states")
    B, T = enc.shape[0], enc.shape[1]
    mask = _mask_u8(mask)
    out = torch.empty(B, T, cfg.block.hidden, dtype=torch.float32, device=enc.device)
    mw, keep = _model_weights(weights)
    ws = _workspace(lib.k2_text_embed_workspace_bytes(ctypes.byref(cfg), B, T), enc.device, workspace)
    check(lib.k2_text_embed(ctypes.byref(cfg), ctypes.byref(mw), B, T, _ptr(enc), _ptr(mask), _ptr(out), _ptr(ws),
                            ws.numel(), _stream(stream)))
    del keep
    return out


def backbone_cached_workspace_bytes(cfg, B: int, T: int, N: int) -> int:
    return load().k2_backbone_cached_workspace_bytes(ctypes.byref(cfg), B, T, N)


def backbone_forward_cached(cfg, weights: dict, x, txt_h, timestep, position_ids, mask, workspace=None, stream=None):
    """k2_backbone_forward_cached: the backbone with its text rows from text_embed (txt_h (B, T, hidden)
    float32, or None when T = 0). Returns the velocity (B, N, in_channels) float32."""
    torch = _torch()
    lib = load()
    _dev_tensor(x, "hidden_states")
    _dev_tensor(timestep, "timestep", torch.float32)
    B, N, C = x.shape
    T = 0
    if txt_h is not None:
        _dev_tensor(txt_h, "txt_h", torch.float32)
        T = txt_h.shape[1]
    mask = _mask_u8(mask)
    out = torch.empty(B, N, C, dtype=torch.float32, device=x.device)
    mw, keep = _model_weights(weights)
    ws = _workspace(lib.k2_backbone_cached_workspace_bytes(ctypes.byref(cfg), B, T, N), x.device, workspace)
    check(lib.k2_backbone_forward_cached(ctypes.byref(cfg), ctypes.byref(mw), B, T, N, _ptr(x), _ptr(txt_h),
                                         _ptr(timestep), _ptr(position_ids), position_ids.shape[0],
                                         position_ids.shape[1], _ptr(mask), _ptr(out), _ptr(ws), ws.numel(),
                                         _stream(stream)))
    del keep
    return out


# ------------------------------------------------------------------------------------------------
# Sampler
# ------------------------------------------------------------------------------------------------
def shift_cfg(**kw) -> _abi.ShiftCfg:
    """k2_shift_cfg with the defaults of k2_shift_cfg_default, fields overridden by keyword."""
    c = _abi.ShiftCfg()
    load().k2_shift_cfg_default(ctypes.byref(c))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def flow_sigmas(num_steps: int, image_seq_len: int, distilled: bool = False, cfg=None):
    """k2_flow_sigmas (host): the num_steps + 1 noise levels as a float32 NumPy array."""
    import numpy as np
    out = (ctypes.c_float * (num_steps + 1))()
    check(load().k2_flow_sigmas(None if cfg is None else ctypes.byref(cfg), num_steps, image_seq_len,
                                1 if distilled else 0, out))
    return np.frombuffer(out, dtype=np.float32).copy()


def cfg_euler_update(x, v_cond, v_uncond, guidance: float, sigma: float, sigma_next: float, out=None, stream=None):
    """k2_cfg_euler_update on float32 device tensors of equal size; returns x_out (x itself if out is x)."""
    torch = _torch()
    _dev_tensor(x, "x", torch.float32)
    _dev_tensor(v_cond, "v_cond", torch.float32)
    if v_uncond is not None:
        _dev_tensor(v_uncond, "v_uncond", torch.float32)
    out = torch.empty_like(x) if out is None else out
    check(load().k2_cfg_euler_update(_ptr(x), _ptr(out), _ptr(v_cond), _ptr(v_uncond), x.numel(), guidance, sigma,
                                     sigma_next, _stream(stream)))
    return out


def denoise_workspace_bytes(cfg, T: int, N: int, guided: bool) -> int:
    return load().k2_denoise_workspace_bytes(ctypes.byref(cfg), T, N, 1 if guided else 0)


def denoise_step(cfg, weights: dict, latents, enc, position_ids, mask, sigma: float, sigma_next: float,
                 guidance: float, workspace=None, stream=None):
    """k2_denoise_step: latents (1, N, in_channels) float32, updated in place; enc (G, T, layers, D) in the
    operand dtype with G = 2 (prompt, negative prompt) when guidance > 0, else 1; mask (G, T) or None."""
    torch = _torch()
    lib = load()
    _dev_tensor(latents, "latents", torch.float32)
    _, N, _ = latents.shape
    T = enc.shape[1] if enc is not None else 0
    mask = _mask_u8(mask)
    mw, keep = _model_weights(weights)
    ws = _workspace(lib.k2_denoise_workspace_bytes(ctypes.byref(cfg), T, N, 1 if guidance > 0 else 0),
                    latents.device, workspace)
    check(lib.k2_denoise_step(ctypes.byref(cfg), ctypes.byref(mw), T, N, _ptr(latents), _ptr(enc), _ptr(mask),
                              _ptr(position_ids), position_ids.shape[0], position_ids.shape[1], sigma, sigma_next,
                              guidance, _ptr(ws), ws.numel(), _stream(stream)))
    del keep
    return latents


def denoise_cached_workspace_bytes(cfg, T: int, N: int, guided: bool) -> int:
    return load().k2_denoise_cached_workspace_bytes(ctypes.byref(cfg), T, N, 1 if guided else 0)


def denoise_step_cached(cfg, weights: dict, latents, txt_h, position_ids, mask, sigma: float, sigma_next: float,
                        guidance: float, workspace=None, stream=None):
    """k2_denoise_step_cached: denoise_step with the text rows txt_h (G, T, hidden) float32 from text_embed
    (computed once per prompt pair), or None when T = 0."""
    torch = _torch()
    lib = load()
    _dev_tensor(latents, "latents", torch.float32)
    _, N, _ = latents.shape
    T = 0
    if txt_h is not None:
        _dev_tensor(txt_h, "txt_h", torch.float32)
        T = txt_h.shape[1]
    mask = _mask_u8(mask)
    mw, keep = _model_weights(weights)
    ws = _workspace(lib.k2_denoise_cached_workspace_bytes(ctypes.byref(cfg), T, N, 1 if guidance > 0 else 0),
                    latents.device, workspace)
    check(lib.k2_denoise_step_cached(ctypes.byref(cfg), ctypes.byref(mw), T, N, _ptr(latents), _ptr(txt_h),
                                     _ptr(mask), _ptr(position_ids), position_ids.shape[0], position_ids.shape[1],
                                     sigma, sigma_next, guidance, _ptr(ws), ws.numel(), _stream(stream)))
    del keep
    return latents


def profile_enable(on: bool = True):
    load().k2_profile_enable(1 if on else 0)


def profile_filter(kernel=None):
    """Record only `kernel` while profiling is enabled (None = every kernel)."""
    load().k2_profile_filter(None if kernel is None else kernel.encode())


def profile_reset():
    load().k2_profile_reset()


def profile_query(kernel: str):
    """(total_ms, launches) of the kernel recorded since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int()
    check(load().k2_profile_query(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def mfma_rate_probe(iters: int, blocks: int, out, stream=None):
    """k2_mfma_rate_probe: enqueue the matrix-core rate probe (blocks * iters * 524288 bf16 FLOP).
    out: a float32 device tensor of at least one element."""
    torch = _torch()
    _dev_tensor(out, "out", torch.float32)
    check(load().k2_mfma_rate_probe(int(iters), int(blocks), _ptr(out), _stream(stream)))
