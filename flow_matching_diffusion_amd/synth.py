"""Seeded synthetic inputs for the Krea 2 single-stream block, its text fusion and the backbone.

This module only draws random numbers and lays out inputs; it computes nothing of the method.
Both the HIP path (through the binding) and the CPU oracle (in tests and the bench's CPU leg)
receive the arrays made here, so the two sides always see the same numbers.

Shapes and defaults follow the Krea2Transformer2DModel API page (constructor signature and the
forward contract) and the Krea2Pipeline page (position ids: text rows at the origin, image rows
(0, h, w) over the latent grid; text padded to a fixed length with a boolean validity mask).

Rules:
  * one generator per tensor: NumPy PCG64 seeded with (workload seed, crc32(tensor name));
  * weights, tables and zero-centred norm weights ~ N(0, 0.02); activations ~ N(0, 1);
  * bf16 workloads round every matrix operand the kernels read in bf16 to bf16 here (RNE, via torch),
    and hand the rounded values, widened back to float32, to the oracle.
"""
from __future__ import annotations

import dataclasses
import zlib
from dataclasses import dataclass, field

import numpy as np

WEIGHT_SIGMA = 0.02


# ----------------------------------------------------------------------------------------------
# Dimensions
# ----------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class BlockDims:
    """One single-stream block (defaults: the Krea2Transformer2DModel constructor)."""
    hidden: int = 6144
    num_heads: int = 48
    num_kv_heads: int = 12
    head_dim: int = 128
    intermediate: int = 16384
    axes_dims: tuple = (32, 48, 48)
    rope_theta: float = 1000.0
    eps: float = 1e-5


@dataclass(frozen=True)
class TextDims:
    """Text-fusion stage (defaults: text_* arguments of the same constructor)."""
    hidden: int = 2560
    num_heads: int = 20
    num_kv_heads: int = 20
    head_dim: int = 128
    intermediate: int = 6912
    num_layers: int = 12
    num_layerwise_blocks: int = 2
    num_refiner_blocks: int = 2
    eps: float = 1e-5


@dataclass(frozen=True)
class ModelDims:
    block: BlockDims = field(default_factory=BlockDims)
    text: TextDims = field(default_factory=TextDims)
    num_layers: int = 28
    in_channels: int = 64
    timestep_embed_dim: int = 256


# ----------------------------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str                 # "f32" or "bf16": the type of matrix operands
    B: int
    T: int
    grid: tuple                # latent grid (gh, gw); N = gh * gw image tokens
    valid: tuple | None        # valid text tokens per batch row (right padding); None = no mask
    t: tuple | None = None     # timesteps in [0,1] (temb from the time path) ...
    t_uniform: bool = False    # ... or drawn ~U[0,1] from the seed
    dims: BlockDims = field(default_factory=BlockDims)
    text: TextDims | None = None
    num_layers: int = 1
    in_channels: int = 64
    timestep_embed_dim: int = 256
    note: str = ""

    @property
    def N(self) -> int:
        return self.grid[0] * self.grid[1]

    @property
    def L(self) -> int:
        return self.T + self.N

    @property
    def M(self) -> int:
        return self.B * self.L


TINY_DIMS = BlockDims(hidden=256, num_heads=4, num_kv_heads=1, head_dim=64, intermediate=512,
                      axes_dims=(16, 24, 24))

WORKLOADS = {
    "tiny": Workload("tiny", 0, "f32", 1, 16, (8, 8), (12,), t_uniform=True, dims=TINY_DIMS,
                     timestep_embed_dim=256,
                     note="tiny single block, fp32, B=1, 16 text tokens (last 4 masked) + 8x8 grid"),
    "block512": Workload("block512", 1, "bf16", 1, 256, (32, 32), (192,),
                         note="full-size block at 512^2, bf16, B=1, temb ~N(0,1)"),
    "block1024": Workload("block1024", 2, "bf16", 2, 512, (64, 64), (300, 16), t=(0.7, 0.7),
                          note="full-size block at 1024^2, bf16, B=2 CFG pair, t=0.7"),
    "backbone1024": Workload("backbone1024", 3, "bf16", 2, 512, (64, 64), (300, 16), t=(0.7, 0.7),
                             text=TextDims(), num_layers=28,
                             note="28-block backbone with text fusion at 1024^2, bf16, B=2"),
    "block2048": Workload("block2048", 4, "bf16", 1, 512, (128, 128), None,
                          note="long-sequence block at 2048^2, bf16, B=1, no mask"),
}


# ----------------------------------------------------------------------------------------------
# Random numbers
# ----------------------------------------------------------------------------------------------
def rng(seed: int, name: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, zlib.crc32(name.encode())])))


def normal(seed: int, name: str, shape, sigma: float = 1.0) -> np.ndarray:
    a = rng(seed, name).standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def uniform(seed: int, name: str, shape) -> np.ndarray:
    return rng(seed, name).random(size=shape, dtype=np.float32)


def round_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even) and widen back to float32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def as_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(a) if dtype == "bf16" else a


# ----------------------------------------------------------------------------------------------
# Input layout helpers (the pipeline's position-id and mask conventions)
# ----------------------------------------------------------------------------------------------
def position_ids(T: int, gh: int, gw: int) -> np.ndarray:
    """(T + gh*gw, 3) float32: text rows all zero; image row T + h*gw + w holds (0, h, w)."""
    pos = np.zeros((T + gh * gw, 3), dtype=np.float32)
    pos[T:, 1] = np.repeat(np.arange(gh, dtype=np.float32), gw)
    pos[T:, 2] = np.tile(np.arange(gw, dtype=np.float32), gh)
    return pos


def text_mask(B: int, T: int, valid) -> np.ndarray | None:
    """(B, T) uint8, nonzero = valid text token, right padded; None when no mask is given."""
    if valid is None:
        return None
    m = np.zeros((B, T), dtype=np.uint8)
    for b, v in enumerate(valid):
        m[b, :v] = 1
    return m


# ----------------------------------------------------------------------------------------------
# Weights
# ----------------------------------------------------------------------------------------------
def block_weights(seed: int, prefix: str, d: BlockDims, dtype: str, modulated: bool = True) -> dict:
    """nn.Linear weights in (out, in) layout; tables and zero-centred norm weights in float32."""
    H, nh, nkv, hd, I = d.hidden, d.num_heads, d.num_kv_heads, d.head_dim, d.intermediate
    s = WEIGHT_SIGMA
    w = {}
    if modulated:
        w["scale_shift_table"] = normal(seed, prefix + "scale_shift_table", (6, H), s)
    w["norm1_w"] = normal(seed, prefix + "norm1_w", (H,), s)
    w["norm2_w"] = normal(seed, prefix + "norm2_w", (H,), s)
    w["norm_q_w"] = normal(seed, prefix + "norm_q_w", (hd,), s)
    w["norm_k_w"] = normal(seed, prefix + "norm_k_w", (hd,), s)
    shapes = {"to_q": (nh * hd, H), "to_k": (nkv * hd, H), "to_v": (nkv * hd, H),
              "to_gate": (nh * hd, H), "to_out": (H, nh * hd),
              "ff_gate": (I, H), "ff_up": (I, H), "ff_down": (H, I)}
    for k, shp in shapes.items():
        w[k] = as_dtype(normal(seed, prefix + k, shp, s), dtype)
    return w


def time_weights(seed: int, H: int, temb_dim: int, dtype: str) -> dict:
    s = WEIGHT_SIGMA
    return {
        "lin1_w": as_dtype(normal(seed, "time.lin1_w", (H, temb_dim), s), dtype),
        "lin1_b": normal(seed, "time.lin1_b", (H,), s),
        "lin2_w": as_dtype(normal(seed, "time.lin2_w", (H, H), s), dtype),
        "lin2_b": normal(seed, "time.lin2_b", (H,), s),
        "mod_w": as_dtype(normal(seed, "time.mod_w", (6 * H, H), s), dtype),
        "mod_b": normal(seed, "time.mod_b", (6 * H,), s),
    }


def text_block_dims(t: TextDims) -> BlockDims:
    return BlockDims(hidden=t.hidden, num_heads=t.num_heads, num_kv_heads=t.num_kv_heads,
                     head_dim=t.head_dim, intermediate=t.intermediate, axes_dims=(0, 0, 0), eps=t.eps)


def text_weights(seed: int, t: TextDims, dtype: str) -> dict:
    bd = text_block_dims(t)
    return {
        "layerwise": [block_weights(seed, f"text.layerwise{i}.", bd, dtype, modulated=False)
                      for i in range(t.num_layerwise_blocks)],
        "compress_w": normal(seed, "text.compress_w", (t.num_layers,), WEIGHT_SIGMA),
        "refiner": [block_weights(seed, f"text.refiner{i}.", bd, dtype, modulated=False)
                    for i in range(t.num_refiner_blocks)],
    }


def model_weights(seed: int, wl: Workload, dtype: str | None = None, blocks: bool = True) -> dict:
    dtype = dtype or wl.dtype
    d = wl.dims
    H = d.hidden
    s = WEIGHT_SIGMA
    text = wl.text or TextDims()
    w = {
        "img_in_w": as_dtype(normal(seed, "img_in_w", (H, wl.in_channels), s), dtype),
        "img_in_b": normal(seed, "img_in_b", (H,), s),
        "txt_in_w": as_dtype(normal(seed, "txt_in_w", (H, text.hidden), s), dtype),
        "txt_in_b": normal(seed, "txt_in_b", (H,), s),
        "time": time_weights(seed, H, wl.timestep_embed_dim, dtype),
        "text": text_weights(seed, text, dtype),
        "final_table": normal(seed, "final_table", (2, H), s),
        "final_w": as_dtype(normal(seed, "final_w", (wl.in_channels, H), s), dtype),
        "final_b": normal(seed, "final_b", (wl.in_channels,), s),
    }
    if blocks:
        w["blocks"] = [block_weights(seed, f"blocks{i}.", d, dtype) for i in range(wl.num_layers)]
    return w


# ----------------------------------------------------------------------------------------------
# Inputs
# ----------------------------------------------------------------------------------------------
def timesteps(wl: Workload) -> np.ndarray | None:
    if wl.t is not None:
        return np.asarray(wl.t, dtype=np.float32)
    if wl.t_uniform:
        return uniform(wl.seed, "timestep", (wl.B,))
    return None


def block_inputs(wl: Workload, with_weights: bool = True) -> dict:
    """Inputs of one block forward: residual stream h (fp32), temb or timesteps, positions, mask."""
    d = wl.dims
    inp = {
        "h": normal(wl.seed, "hidden", (wl.B, wl.L, d.hidden)),
        "position_ids": position_ids(wl.T, *wl.grid),
        "mask": text_mask(wl.B, wl.T, wl.valid),
        "T": wl.T,
        "timestep": timesteps(wl),
    }
    if inp["timestep"] is None:
        inp["temb"] = normal(wl.seed, "temb", (wl.B, 6 * d.hidden))
    else:
        inp["time_weights"] = time_weights(wl.seed, d.hidden, wl.timestep_embed_dim, wl.dtype)
    if with_weights:
        inp["weights"] = block_weights(wl.seed, "block.", d, wl.dtype)
    return inp


def backbone_inputs(wl: Workload) -> dict:
    text = wl.text or TextDims()
    return {
        "x": normal(wl.seed, "latents", (wl.B, wl.N, wl.in_channels)),
        "enc": as_dtype(normal(wl.seed, "encoder_hidden_states", (wl.B, wl.T, text.num_layers, text.hidden)),
                        wl.dtype),
        "timestep": timesteps(wl) if timesteps(wl) is not None else uniform(wl.seed, "timestep", (wl.B,)),
        "position_ids": position_ids(wl.T, *wl.grid),
        "mask": text_mask(wl.B, wl.T, wl.valid),
        "T": wl.T,
    }


def sample_rows(wl: Workload, count: int, seed: int | None = None) -> np.ndarray:
    """Seeded subset of sequence rows (0..L-1) that always holds the edges of the text and
    image segments and, where a mask is given, the last valid and first padded text token."""
    L, T = wl.L, wl.T
    must = {0, L - 1}
    if T > 0:
        must |= {T - 1, T}
    if wl.valid is not None:
        for v in wl.valid:
            must |= {max(v - 1, 0), min(v, L - 1)}
    must = sorted(r for r in must if 0 <= r < L)
    g = rng(wl.seed if seed is None else seed, "sample_rows")
    rest = np.setdiff1d(np.arange(L), must)
    extra = g.choice(rest, size=max(0, min(count - len(must), rest.size)), replace=False)
    return np.sort(np.concatenate([np.asarray(must, dtype=np.int64), extra.astype(np.int64)]))


def replace(wl: Workload, **kw) -> Workload:
    return dataclasses.replace(wl, **kw)


# ----------------------------------------------------------------------------------------------
# Device-side generation (bench workloads: same shapes and distributions, drawn on the GPU)
# ----------------------------------------------------------------------------------------------
def device_normal(seed: int, name: str, shape, sigma: float, dtype, device):
    """Seeded N(0, sigma^2) tensor drawn on the device (torch's generator), cast to dtype."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed((seed << 32) ^ zlib.crc32(name.encode()))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        t.mul_(sigma)
    return t.to(dtype)


def device_block_weights(seed: int, prefix: str, d: BlockDims, dtype: str, device, modulated: bool = True) -> dict:
    import torch
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    H, nh, nkv, hd, I = d.hidden, d.num_heads, d.num_kv_heads, d.head_dim, d.intermediate
    s = WEIGHT_SIGMA
    w = {}
    if modulated:
        w["scale_shift_table"] = device_normal(seed, prefix + "scale_shift_table", (6, H), s, torch.float32, device)
    for n, shp in (("norm1_w", (H,)), ("norm2_w", (H,)), ("norm_q_w", (hd,)), ("norm_k_w", (hd,))):
        w[n] = device_normal(seed, prefix + n, shp, s, torch.float32, device)
    shapes = {"to_q": (nh * hd, H), "to_k": (nkv * hd, H), "to_v": (nkv * hd, H), "to_gate": (nh * hd, H),
              "to_out": (H, nh * hd), "ff_gate": (I, H), "ff_up": (I, H), "ff_down": (H, I)}
    for n, shp in shapes.items():
        w[n] = device_normal(seed, prefix + n, shp, s, td, device)
    return w


def device_model_weights(seed: int, wl: Workload, device) -> dict:
    import torch
    td = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    f32 = torch.float32
    d, t = wl.dims, (wl.text or TextDims())
    H, s = d.hidden, WEIGHT_SIGMA
    tb = text_block_dims(t)
    return {
        "img_in_w": device_normal(seed, "img_in_w", (H, wl.in_channels), s, td, device),
        "img_in_b": device_normal(seed, "img_in_b", (H,), s, f32, device),
        "txt_in_w": device_normal(seed, "txt_in_w", (H, t.hidden), s, td, device),
        "txt_in_b": device_normal(seed, "txt_in_b", (H,), s, f32, device),
        "time": {
            "lin1_w": device_normal(seed, "time.lin1_w", (H, wl.timestep_embed_dim), s, td, device),
            "lin1_b": device_normal(seed, "time.lin1_b", (H,), s, f32, device),
            "lin2_w": device_normal(seed, "time.lin2_w", (H, H), s, td, device),
            "lin2_b": device_normal(seed, "time.lin2_b", (H,), s, f32, device),
            "mod_w": device_normal(seed, "time.mod_w", (6 * H, H), s, td, device),
            "mod_b": device_normal(seed, "time.mod_b", (6 * H,), s, f32, device),
        },
        "text": {
            "layerwise": [device_block_weights(seed, f"text.layerwise{i}.", tb, wl.dtype, device, modulated=False)
                          for i in range(t.num_layerwise_blocks)],
            "compress_w": device_normal(seed, "text.compress_w", (t.num_layers,), s, f32, device),
            "refiner": [device_block_weights(seed, f"text.refiner{i}.", tb, wl.dtype, device, modulated=False)
                        for i in range(t.num_refiner_blocks)],
        },
        "blocks": [device_block_weights(seed, f"blocks{i}.", d, wl.dtype, device) for i in range(wl.num_layers)],
        "final_table": device_normal(seed, "final_table", (2, H), s, f32, device),
        "final_w": device_normal(seed, "final_w", (wl.in_channels, H), s, td, device),
        "final_b": device_normal(seed, "final_b", (wl.in_channels,), s, f32, device),
    }
