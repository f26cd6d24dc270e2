"""Writes the oracle's velocity for the full backbone at 1024^2 (the 28-block Krea2Transformer2DModel
with text fusion over the (2, 512, 12, 2560) text stack, B = 2 as a CFG pair, t = 0.7) to
backbone1024_velocity.npz beside this file, for tests/test_gpu_backbone1024.py.

It calls only oracle/ (the backbone's stem, its blocks and its head, in the order
oracle.backbone_forward takes them) and the seeded generators of flow_matching_diffusion_amd.synth.
The 28 blocks' weights do not fit the host's memory at once in float64, so each block's weights are
drawn once and applied to every oracle form before the next block is drawn. Forms: the exact function
and the three bf16 realisations of reading R13 (plain, fused-softmax, float32 products). Stored in
float32 with a key of the workload, its seed and hashes of the oracle's and the generators' code.

Run: python tests/golden/backbone1024_oracle.py   (about an hour on 8 cores, 12 GB of memory)
"""
from __future__ import annotations

import ast
import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from flow_matching_diffusion_amd import synth as S  # noqa: E402
from oracle import k2_oracle as O  # noqa: E402

OUT = os.path.join(HERE, "backbone1024_velocity.npz")
FORMS = {"exact": None, "A": O.bf16_form(), "B": O.bf16_form(flash=True),
         "C": O.bf16_form(flash=True, f32_products=True)}


def code_hash(path: str) -> str:
    """sha256 of a module's syntax tree with docstrings removed: comment and docstring edits keep it."""
    tree = ast.parse(open(path).read())
    for node in ast.walk(tree):
        body = getattr(node, "body", None)
        if isinstance(body, list) and body and isinstance(body[0], ast.Expr) and \
                isinstance(getattr(body[0], "value", None), ast.Constant) and isinstance(body[0].value.value, str):
            node.body = body[1:] or [ast.Pass()]
    return hashlib.sha256(ast.dump(tree).encode()).hexdigest()[:16]


def fixture_key(wl) -> str:
    return "|".join([wl.name, str(wl.seed), str(wl.num_layers), wl.dtype,
                     code_hash(os.path.join(ROOT, "oracle", "k2_oracle.py")),
                     code_hash(os.path.join(ROOT, "flow_matching_diffusion_amd", "synth.py"))])


def streamed_backbone(wl, forms, log=print):
    """oracle.backbone_forward for every form at once, with the blocks' weights drawn one block at a
    time. Returns {form: velocity (B, N, in_channels)}."""
    inp = S.backbone_inputs(wl)
    mw = S.model_weights(wl.seed, wl, blocks=False)
    tdims = S.text_block_dims(wl.text)
    x = S.as_dtype(inp["x"], wl.dtype)
    state = {}
    for name, rnd in forms.items():
        state[name] = O.backbone_stem(x, inp["enc"], inp["timestep"], inp["mask"], mw, tdims, wl.timestep_embed_dim,
                                      rnd=rnd)
        log(f"stem {name} done")
    for i in range(wl.num_layers):
        t0 = time.time()
        bw = S.block_weights(wl.seed, f"blocks{i}.", wl.dims, wl.dtype)
        for name, rnd in forms.items():
            h, temb, e = state[name]
            state[name] = (O.block_forward(h, temb, inp["position_ids"], inp["mask"], bw, wl.dims, T=wl.T, rnd=rnd),
                           temb, e)
        del bw
        log(f"block {i + 1}/{wl.num_layers} done in {time.time() - t0:.0f} s")
    return {name: O.backbone_head(h, e, mw, wl.dims, wl.T, rnd=forms[name]) for name, (h, temb, e) in state.items()}


def main():
    wl = S.WORKLOADS["backbone1024"]
    t0 = time.time()
    vel = streamed_backbone(wl, FORMS, log=lambda m: print(m, flush=True))
    np.savez_compressed(OUT, key=np.array(fixture_key(wl)), seconds=np.array(time.time() - t0),
                        **{k: v.astype(np.float32) for k, v in vel.items()})
    print(f"wrote {OUT} in {time.time() - t0:.0f} s", flush=True)


if __name__ == "__main__":
    main()
