"""The C ABI on the host: libk2.so loads, exports every function include/k2.h declares, the binding
declares the same set, defaults equal the API page's, and host validation rejects bad arguments
with the documented status before any HIP call (so these run without a GPU)."""
import ctypes
import json
import os
import re

import pytest

import flow_matching_diffusion_amd as k2
from flow_matching_diffusion_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "k2.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "krea2_defaults.json")

OK, ENULL, ESHAPE, ECONFIG, EDTYPE, EWS, EALIGN = 0, -1, -2, -3, -4, -5, -7


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*(k2_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("k2_block_forward", "k2_backbone_forward", "k2_text_fusion_forward", "k2_timestep_modulation_forward"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    lib = k2.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_binding_declares_the_same_functions():
    assert sorted(_abi.SIGNATURES) == declared_functions()


def test_defaults_match_api_page():
    g = json.load(open(GOLDEN))
    lib = k2.load()
    m = _abi.ModelCfg()
    lib.k2_model_cfg_default(ctypes.byref(m))
    b, t = m.block, m.text
    assert (b.hidden, b.num_heads, b.num_kv_heads, b.head_dim, b.intermediate) == (
        g["hidden_size"], g["num_attention_heads"], g["num_key_value_heads"], g["attention_head_dim"],
        g["intermediate_size"])
    assert list(b.axes_dims) == g["axes_dims_rope"]
    assert b.rope_theta == pytest.approx(g["rope_theta"]) and b.eps == pytest.approx(g["norm_eps"])
    assert (m.num_layers, m.in_channels, m.timestep_embed_dim) == (g["num_layers"], g["in_channels"],
                                                                    g["timestep_embed_dim"])
    assert (t.block.hidden, t.block.num_heads, t.block.num_kv_heads, t.block.intermediate, t.num_layers,
            t.num_layerwise_blocks, t.num_refiner_blocks) == (
        g["text_hidden_dim"], g["text_num_attention_heads"], g["text_num_key_value_heads"],
        g["text_intermediate_size"], g["num_text_layers"], g["num_layerwise_text_blocks"],
        g["num_refiner_text_blocks"])


# ------------------------------------------------------------------------------------------------
# Validation (fake, never dereferenced device addresses; every case fails before a launch)
# ------------------------------------------------------------------------------------------------
FAKE = 0x7F0000000000


def good_cfg():
    c = _abi.BlockCfg()
    k2.load().k2_block_cfg_default(ctypes.byref(c))
    return c


def good_weights():
    w = _abi.BlockWeights()
    for i, n in enumerate(_abi.BLOCK_WEIGHT_FIELDS):
        setattr(w, n, FAKE + 0x1000000 * (i + 1))
    return w


def call_block(cfg=None, w=None, B=1, T=4, N=4, hin=FAKE, hout=FAKE, temb=FAKE, pos=FAKE, rows=8, cols=3,
               mask=None, ws=FAKE, ws_bytes=None, use_cfg=True):
    lib = k2.load()
    cfg = good_cfg() if cfg is None else cfg
    w = good_weights() if w is None else w
    if ws_bytes is None:
        ws_bytes = 0  # forces a workspace error unless the case fails earlier
    return lib.k2_block_forward(ctypes.byref(cfg) if use_cfg else None, ctypes.byref(w), B, T, N, hin, hout, temb,
                                pos, rows, cols, mask, ws, ws_bytes, None)


def test_block_validation_codes():
    lib = k2.load()
    assert call_block(use_cfg=False) == ENULL
    c = good_cfg(); c.axes_dims[0] = 30
    assert call_block(cfg=c) == ECONFIG and b"sum(axes_dims)" in lib.k2_last_error()
    c = good_cfg(); c.axes_dims[0] = 31; c.axes_dims[1] = 49
    assert call_block(cfg=c) == ECONFIG
    c = good_cfg(); c.hidden = 6000
    assert call_block(cfg=c) == ECONFIG
    c = good_cfg(); c.num_kv_heads = 16
    assert call_block(cfg=c) == ECONFIG  # 48 % 16 == 0 but G = 3 is unsupported
    c = good_cfg(); c.num_kv_heads = 5
    assert call_block(cfg=c) == ECONFIG
    c = good_cfg(); c.head_dim = 96; c.num_heads = 64; c.axes_dims[:] = [32, 32, 32]
    assert call_block(cfg=c) == ECONFIG
    c = good_cfg(); c.dtype = 7
    assert call_block(cfg=c) == EDTYPE
    # position_ids must be (T + N, 3): the article's ValueError on its shape
    assert call_block(rows=7) == ESHAPE and b"position_ids" in lib.k2_last_error()
    assert call_block(cols=2) == ESHAPE
    assert call_block(B=0) == ESHAPE
    assert call_block(T=-1) == ESHAPE
    # one batch row's keys must fit one 2 GiB buffer range (bf16: 1536 columns x 2 bytes per token),
    # and B * (T + N) rows a 32-bit index
    L_max = 0x7FFFFFF0 // (12 * 128 * 2)
    assert call_block(T=512, N=L_max - 512, rows=L_max) == EWS   # passes validation, fails on ws
    assert call_block(T=512, N=L_max - 511, rows=L_max + 1) == ESHAPE and b"too long" in lib.k2_last_error()
    assert call_block(B=65535, T=512, N=40000, rows=40512) == ESHAPE and b"2^31" in lib.k2_last_error()
    w = good_weights(); w.to_k = None
    assert call_block(w=w) == ENULL
    assert call_block(temb=None) == ENULL
    w = good_weights(); w.scale_shift_table = None
    assert call_block(w=w) == ECONFIG  # temb given for an unmodulated block
    assert call_block(hin=None) == ENULL
    need = lib.k2_block_workspace_bytes(ctypes.byref(good_cfg()), 1, 4, 4)
    assert need > 0
    assert call_block(ws_bytes=need - 1) == EWS
    assert call_block(ws=FAKE + 8, ws_bytes=need) == EWS
    assert call_block(ws=None, ws_bytes=need) == ENULL
    # every other device pointer must be 16-byte aligned (the kernels move 16 bytes per lane)
    assert call_block(hin=FAKE + 4) == EALIGN and b"16-byte" in lib.k2_last_error()
    assert call_block(hout=FAKE + 8) == EALIGN
    assert call_block(temb=FAKE + 12) == EALIGN
    w = good_weights(); w.norm_q_w = FAKE + 0x100004
    assert call_block(w=w) == EALIGN
    w = good_weights(); w.ff_down = FAKE + 0x100002
    assert call_block(w=w) == EALIGN


def test_block_backward_validation_codes():
    lib = k2.load()
    grads = _abi.BlockGrads()

    def call(B=1, T=4, N=4, rows=8, gout=FAKE, gin=FAKE + 0x10000000, ws_bytes=0):
        return lib.k2_block_backward(ctypes.byref(good_cfg()), ctypes.byref(good_weights()), B, T, N, FAKE, FAKE,
                                     FAKE, rows, 3, None, gout, gin, None, ctypes.byref(grads), FAKE, ws_bytes, None)

    assert call(gout=None) == ENULL
    assert call(gin=FAKE) == ECONFIG  # grad_in aliases hidden_in
    # the attention backward addresses a batch row's query rows (48 x 128 bf16 per token) through
    # one 2 GiB buffer range
    L_max = 0x7FFFFFF0 // (48 * 128 * 2)
    assert call(T=512, N=L_max - 512, rows=L_max) == EWS  # passes validation, fails on ws
    assert call(T=512, N=L_max - 511, rows=L_max + 1) == ESHAPE and b"too long for the backward" in lib.k2_last_error()


def test_workspace_layout_is_ordered_and_aligned():
    lib = k2.load()
    lay = k2.block_workspace_layout(good_cfg(), 2, 512, 4096)
    offs = [lay.x1, lay.q, lay.k, lay.vt, lay.g, lay.og, lay.x2, lay.a, lay.rope, lay.mod]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.total == lib.k2_block_workspace_bytes(ctypes.byref(good_cfg()), 2, 512, 4096)
    assert lay.ldvt % 64 == 0 and lay.ldvt >= 4608
    # short sequences (the layerwise text-fusion stage): 32 key slots per V^T row
    assert k2.block_workspace_layout(good_cfg(), 1024, 0, 12).ldvt == 32
    assert k2.block_workspace_layout(good_cfg(), 2, 0, 33).ldvt == 64


def test_time_and_text_and_backbone_validation():
    lib = k2.load()
    tc = _abi.TimeCfg(6144, 256, 1)
    tw = _abi.TimeWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert lib.k2_timestep_modulation_forward(ctypes.byref(tc), ctypes.byref(tw), 2, FAKE, FAKE, None, FAKE, 0,
                                              None) == EWS
    assert lib.k2_timestep_modulation_forward(ctypes.byref(tc), ctypes.byref(tw), 0, FAKE, FAKE, None, FAKE, 0,
                                              None) == ESHAPE
    tc.timestep_embed_dim = 250
    assert lib.k2_timestep_modulation_forward(ctypes.byref(tc), ctypes.byref(tw), 2, FAKE, FAKE, None, FAKE, 0,
                                              None) == ECONFIG

    t = _abi.TextCfg()
    lib.k2_text_cfg_default(ctypes.byref(t))
    blocks = (_abi.BlockWeights * 2)(good_weights(), good_weights())
    for b in blocks:
        b.scale_shift_table = None
    tw = _abi.TextWeights(blocks, FAKE, blocks)
    assert lib.k2_text_fusion_forward(ctypes.byref(t), ctypes.byref(tw), 2, 512, FAKE, None, FAKE, FAKE, 0,
                                      None) == EWS
    tw.compress_w = None
    assert lib.k2_text_fusion_forward(ctypes.byref(t), ctypes.byref(tw), 2, 512, FAKE, None, FAKE, FAKE, 0,
                                      None) == ENULL
    tw.compress_w = FAKE
    blocks[0].scale_shift_table = FAKE
    assert lib.k2_text_fusion_forward(ctypes.byref(t), ctypes.byref(tw), 2, 512, FAKE, None, FAKE, FAKE, 0,
                                      None) == ECONFIG
    blocks[0].scale_shift_table = None

    m = _abi.ModelCfg()
    lib.k2_model_cfg_default(ctypes.byref(m))
    m.num_layers = 2
    mb = (_abi.BlockWeights * 2)(good_weights(), good_weights())
    mw = _abi.ModelWeights()
    for n in ("img_in_w", "img_in_b", "txt_in_w", "txt_in_b", "final_table", "final_w", "final_b"):
        setattr(mw, n, FAKE)
    mw.time = _abi.TimeWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    mw.text = tw
    mw.blocks = ctypes.cast(mb, ctypes.POINTER(_abi.BlockWeights))
    args = lambda rows, ws_bytes: lib.k2_backbone_forward(ctypes.byref(m), ctypes.byref(mw), 2, 512, 4096, FAKE, FAKE,
                                                          FAKE, FAKE, rows, 3, None, FAKE, FAKE, ws_bytes, None)
    assert args(4608, 0) == EWS
    assert args(4607, 0) == ESHAPE
    m.block.axes_dims[2] = 46
    assert args(4608, 0) == ECONFIG
    m.block.axes_dims[2] = 48

    # text-path cache: the cached backbone needs txt_h, not the text weights, and a smaller workspace
    cached = lambda txt_h, ws_bytes: lib.k2_backbone_forward_cached(
        ctypes.byref(m), ctypes.byref(mw), 2, 512, 4096, FAKE, txt_h, FAKE, FAKE, 4608, 3, None, FAKE, FAKE, ws_bytes,
        None)
    assert cached(FAKE, 0) == EWS
    assert cached(None, 0) == ENULL
    mw.text = _abi.TextWeights(None, None, None)
    mw.txt_in_w = None
    assert cached(FAKE, 0) == EWS  # text weights are not needed
    assert args(4608, 0) == ENULL  # ... but the uncached backbone needs them
    full = lib.k2_backbone_workspace_bytes(ctypes.byref(m), 2, 512, 4096)
    small = lib.k2_backbone_cached_workspace_bytes(ctypes.byref(m), 2, 512, 4096)
    assert 0 < small < full
    assert lib.k2_backbone_cached_workspace_bytes(ctypes.byref(m), 2, 0, 4096) == \
        lib.k2_backbone_workspace_bytes(ctypes.byref(m), 2, 0, 4096)
    mw.text = tw
    mw.txt_in_w = FAKE
    embed = lambda enc, out, ws_bytes: lib.k2_text_embed(ctypes.byref(m), ctypes.byref(mw), 2, 512, enc, None, out,
                                                         FAKE, ws_bytes, None)
    assert embed(FAKE, FAKE, 0) == EWS
    assert embed(None, FAKE, 1 << 40) == ENULL
    assert embed(FAKE, None, 1 << 40) == ENULL
    assert lib.k2_text_embed_workspace_bytes(ctypes.byref(m), 2, 512) > 0
    step = lambda txt_h, ws_bytes: lib.k2_denoise_step_cached(ctypes.byref(m), ctypes.byref(mw), 512, 4096, FAKE,
                                                              txt_h, None, FAKE, 4608, 3, 1.0, 0.9, 4.5, FAKE,
                                                              ws_bytes, None)
    assert step(FAKE, 0) == EWS
    assert step(None, 1 << 40) == ENULL
    assert lib.k2_denoise_cached_workspace_bytes(ctypes.byref(m), 512, 4096, 1) < \
        lib.k2_denoise_workspace_bytes(ctypes.byref(m), 512, 4096, 1)


def test_static_scratch_block_forward_validation():
    # the entry point without a workspace rejects a call whose scratch exceeds the static array, before
    # any device work (fake pointers are never touched)
    lib = k2.load()
    cap = lib.k2_block_forward_static_ws_max_bytes()
    assert cap == 128 << 20
    cfg = good_cfg()
    assert lib.k2_block_workspace_bytes(ctypes.byref(cfg), 1, 256, 1024) <= cap   # the 512^2 block fits
    need = lib.k2_block_workspace_bytes(ctypes.byref(cfg), 2, 512, 4096)
    assert need > cap
    w = good_weights()
    call = lambda B, T, N, rows: lib.k2_block_forward_static_ws(ctypes.byref(cfg), ctypes.byref(w), B, T, N, FAKE, FAKE,
                                                                  FAKE, FAKE, rows, 3, None, None)
    assert call(2, 512, 4096, 4608) == EWS and b"static scratch" in lib.k2_last_error()
    assert call(1, 256, 1024, 1279) == ESHAPE      # the usual validation comes first
    assert lib.k2_block_forward_static_ws(None, ctypes.byref(w), 1, 4, 4, FAKE, FAKE, FAKE, FAKE, 8, 3, None,
                                          None) == ENULL
