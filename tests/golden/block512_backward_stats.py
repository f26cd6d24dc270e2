"""Writes the bf16 model's own deviation of the block's gradients at the full-size 512^2 block
(block512: hidden 6144, 48 / 12 heads, intermediate 16384, 1280 tokens) to
block512_backward_bf16_stats.json beside this file, for the block1024 backward test
(tests/test_gpu_backward.py), where the oracle's backward is out of reach on the host.

It calls only oracle/ and the seeded generators of flow_matching_diffusion_amd.synth, on the inputs
of the block512 full-width backward test: the oracle's exact gradients and those of the three bf16
realisations of reading R13 (plain, fused-softmax, float32 products). For every gradient and
realisation it stores max, p99.9 and rms of |realisation - exact| / rms(exact), with a key of the
workload, its seed and hashes of the oracle's and the generators' code.

Run: python tests/golden/block512_backward_stats.py   (a few minutes on 8 cores)
"""
from __future__ import annotations

import json
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
from tests.golden.backbone1024_oracle import code_hash  # noqa: E402

OUT = os.path.join(HERE, "block512_backward_bf16_stats.json")
FORMS = {"A": O.bf16_form(), "B": O.bf16_form(flash=True), "C": O.bf16_form(flash=True, f32_products=True)}


def stats_key(wl) -> str:
    return "|".join([wl.name, str(wl.seed), wl.dtype, code_hash(os.path.join(ROOT, "oracle", "k2_oracle.py")),
                     code_hash(os.path.join(ROOT, "flow_matching_diffusion_amd", "synth.py"))])


def block512_inputs():
    """The block512 full-width backward test's inputs: workload, block inputs, temb, output gradient."""
    wl = S.WORKLOADS["block512"]
    inp = S.block_inputs(wl)
    temb = inp["temb"] if "temb" in inp else \
        O.time_path(inp["timestep"], inp["time_weights"], wl.timestep_embed_dim)[0].astype(np.float32)
    dh_out = np.random.default_rng(wl.seed + 1).standard_normal(inp["h"].shape).astype(np.float32)
    return wl, inp, temb, dh_out


def deviation(got: np.ndarray, ref: np.ndarray) -> dict:
    scale = float(np.sqrt(np.mean(np.square(ref, dtype=np.float64))))
    d = np.abs(got.astype(np.float64) - ref) / scale
    return {"max": float(d.max()), "p999": float(np.quantile(d, 0.999)), "rms": float(np.sqrt(np.mean(d * d)))}


def main():
    wl, inp, temb, dh_out = block512_inputs()

    def grads(rnd):
        t0 = time.time()
        dh, dtemb, gr = O.block_backward(inp["h"], temb, inp["position_ids"], inp["mask"], inp["weights"], wl.dims,
                                         wl.T, dh_out, rnd=rnd)
        print(f"  one oracle backward in {time.time() - t0:.0f} s", flush=True)
        return dict(gr, h=dh, temb=dtemb)

    exact = grads(None)
    out = {"key": stats_key(wl), "stats": {}}
    for name, rnd in FORMS.items():
        print(f"form {name}", flush=True)
        got = grads(rnd)
        for k, ref in exact.items():
            if ref is None:
                continue
            out["stats"].setdefault(k, {})[name] = deviation(got[k], ref)
        del got
    with open(OUT, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
        f.write("\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
