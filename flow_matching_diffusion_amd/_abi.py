"""ctypes declarations of include/k2.h and the loader of libk2.so (no computation here)."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libk2.so")

K2_F32, K2_BF16 = 0, 1
STATUS = {0: "K2_OK", -1: "K2_ERR_NULL", -2: "K2_ERR_SHAPE", -3: "K2_ERR_CONFIG", -4: "K2_ERR_DTYPE",
          -5: "K2_ERR_WORKSPACE", -6: "K2_ERR_HIP",
          -7: "K2_ERR_ALIGN"}

BLOCK_WEIGHT_FIELDS = ("scale_shift_table", "norm1_w", "norm2_w", "norm_q_w", "norm_k_w", "to_q", "to_k", "to_v",
                       "to_gate", "to_out", "ff_gate", "ff_up", "ff_down")
TIME_WEIGHT_FIELDS = ("lin1_w", "lin1_b", "lin2_w", "lin2_b", "mod_w", "mod_b")


class BlockCfg(ctypes.Structure):
    _fields_ = [("hidden", c_int), ("num_heads", c_int), ("num_kv_heads", c_int), ("head_dim", c_int),
                ("intermediate", c_int), ("axes_dims", c_int * 3), ("rope_theta", c_float), ("eps", c_float),
                ("dtype", c_int)]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in BLOCK_WEIGHT_FIELDS]


class BlockGrads(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in BLOCK_WEIGHT_FIELDS]


class BlockLayout(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in ("x1", "q", "k", "vt", "g", "og", "x2", "a", "rope", "mod", "reach", "total")] + \
               [("ldvt", c_int)]


class TimeCfg(ctypes.Structure):
    _fields_ = [("hidden", c_int), ("timestep_embed_dim", c_int), ("dtype", c_int)]


class TimeWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in TIME_WEIGHT_FIELDS]


class TextCfg(ctypes.Structure):
    _fields_ = [("block", BlockCfg), ("num_layers", c_int), ("num_layerwise_blocks", c_int),
                ("num_refiner_blocks", c_int)]


class TextWeights(ctypes.Structure):
    _fields_ = [("layerwise", POINTER(BlockWeights)), ("compress_w", c_void_p), ("refiner", POINTER(BlockWeights))]


class ModelCfg(ctypes.Structure):
    _fields_ = [("block", BlockCfg), ("text", TextCfg), ("num_layers", c_int), ("in_channels", c_int),
                ("timestep_embed_dim", c_int)]


class ModelWeights(ctypes.Structure):
    _fields_ = [("img_in_w", c_void_p), ("img_in_b", c_void_p), ("txt_in_w", c_void_p), ("txt_in_b", c_void_p),
                ("time", TimeWeights), ("text", TextWeights), ("blocks", POINTER(BlockWeights)),
                ("final_table", c_void_p), ("final_norm_w", c_void_p), ("final_w", c_void_p), ("final_b", c_void_p)]


class ShiftCfg(ctypes.Structure):
    _fields_ = [("base_shift", c_float), ("max_shift", c_float), ("base_image_seq_len", c_int),
                ("max_image_seq_len", c_int), ("distilled_mu", c_float)]


# name -> (restype, argtypes): every function declared in include/k2.h
SIGNATURES = {
    "k2_block_cfg_default": (None, [POINTER(BlockCfg)]),
    "k2_text_cfg_default": (None, [POINTER(TextCfg)]),
    "k2_model_cfg_default": (None, [POINTER(ModelCfg)]),
    "k2_block_workspace_bytes": (c_size_t, [POINTER(BlockCfg), c_int, c_int, c_int]),
    "k2_block_workspace_layout_query": (c_int, [POINTER(BlockCfg), c_int, c_int, c_int, POINTER(BlockLayout)]),
    "k2_block_forward": (c_int, [POINTER(BlockCfg), POINTER(BlockWeights), c_int, c_int, c_int, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
    "k2_block_forward_block_causal": (c_int, [POINTER(BlockCfg), POINTER(BlockWeights), c_int, c_int, c_int, c_void_p,
                                              c_void_p, c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p,
                                              c_void_p, c_size_t, c_void_p]),
    "k2_block_backward_workspace_bytes": (c_size_t, [POINTER(BlockCfg), c_int, c_int, c_int]),
    "k2_block_backward": (c_int, [POINTER(BlockCfg), POINTER(BlockWeights), c_int, c_int, c_int, c_void_p, c_void_p,
                                  c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                  POINTER(BlockGrads), c_void_p, c_size_t, c_void_p]),
    "k2_timestep_modulation_workspace_bytes": (c_size_t, [POINTER(TimeCfg), c_int]),
    "k2_timestep_modulation_forward": (c_int, [POINTER(TimeCfg), POINTER(TimeWeights), c_int, c_void_p, c_void_p,
                                               c_void_p, c_void_p, c_size_t, c_void_p]),
    "k2_text_fusion_workspace_bytes": (c_size_t, [POINTER(TextCfg), c_int, c_int]),
    "k2_text_fusion_forward": (c_int, [POINTER(TextCfg), POINTER(TextWeights), c_int, c_int, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_size_t, c_void_p]),
    "k2_backbone_workspace_bytes": (c_size_t, [POINTER(ModelCfg), c_int, c_int, c_int]),
    "k2_backbone_forward": (c_int, [POINTER(ModelCfg), POINTER(ModelWeights), c_int, c_int, c_int, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p, c_size_t,
                                    c_void_p]),
    "k2_text_embed_workspace_bytes": (c_size_t, [POINTER(ModelCfg), c_int, c_int]),
    "k2_text_embed": (c_int, [POINTER(ModelCfg), POINTER(ModelWeights), c_int, c_int, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_size_t, c_void_p]),
    "k2_backbone_cached_workspace_bytes": (c_size_t, [POINTER(ModelCfg), c_int, c_int, c_int]),
    "k2_backbone_forward_cached": (c_int, [POINTER(ModelCfg), POINTER(ModelWeights), c_int, c_int, c_int, c_void_p,
                                           c_void_p, c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                           c_size_t, c_void_p]),
    "k2_shift_cfg_default": (None, [POINTER(ShiftCfg)]),
    "k2_flow_sigmas": (c_int, [POINTER(ShiftCfg), c_int, c_int, c_int, POINTER(c_float)]),
    "k2_cfg_euler_update": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_float, c_float, c_float,
                                    c_void_p]),
    "k2_denoise_workspace_bytes": (c_size_t, [POINTER(ModelCfg), c_int, c_int, c_int]),
    "k2_denoise_step": (c_int, [POINTER(ModelCfg), POINTER(ModelWeights), c_int, c_int, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_int, c_int, c_float, c_float, c_float, c_void_p, c_size_t, c_void_p]),
    "k2_denoise_cached_workspace_bytes": (c_size_t, [POINTER(ModelCfg), c_int, c_int, c_int]),
    "k2_denoise_step_cached": (c_int, [POINTER(ModelCfg), POINTER(ModelWeights), c_int, c_int, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_int, c_int, c_float, c_float, c_float, c_void_p, c_size_t,
                                       c_void_p]),
    "k2_last_error": (c_char_p, []),
    "k2_block_forward_static_ws_max_bytes": (c_size_t, []),
    "k2_block_forward_static_ws": (c_int, [POINTER(BlockCfg), POINTER(BlockWeights), c_int, c_int, c_int, c_void_p,
                                           c_void_p, c_void_p, c_void_p, c_int, c_int, c_void_p, c_void_p]),
    "k2_mfma_rate_probe": (c_int, [c_int, c_int, c_void_p, c_void_p]),
    "k2_profile_enable": (None, [c_int]),
    "k2_profile_filter": (None, [c_char_p]),
    "k2_profile_reset": (None, []),
    "k2_profile_query": (c_int, [c_char_p, POINTER(c_double), POINTER(c_int)]),
}

_lib = None


def load(path: str | None = None):
    """Load libk2.so (built in-tree by __graft_entry__.build()); raises if it is missing."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libk2.so is not built ({p} missing): run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


class K2Error(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code


def check(code: int):
    if code != 0:
        raise K2Error(code, load().k2_last_error().decode())
