#!/usr/bin/env python3
"""Benchmark of the Krea 2 single-stream block forward on one MI355X.

A step is one k2_block_forward (all stages: modulation, modulated RMSNorm, q/k/v/gate projection
with q/k norm + RoPE, masked GQA attention with the sigmoid gate, output projection + gated
residual, modulated RMSNorm, SwiGLU, down projection + gated residual) over the 1024^2 CFG pair
(B=2, 512 text tokens with 300 / 16 valid + a 64x64 latent grid, L = 4608, full-size dims), with
weights and activations resident in HBM; temb is computed once before timing (the backbone
computes it once for all 28 blocks). value = algorithmic block TFLOP/s (GEMMs over every row,
attention over valid keys only). Also reported: the 28-block backbone with text fusion at the
same resolution as denoise steps/s (one call = one CFG step), the sampler on one image (with guidance
as the base checkpoint's 28 steps and without as the distilled 8 steps) as time per image, both with
the text rows computed once per prompt pair (k2_text_embed, then k2_denoise_step_cached) and with
the text path run at every step (k2_denoise_step), the block-causal block variant on the same pair
(a condition block then the target block), the block's backward pass (k2_block_backward),
per-kernel times, the roofline of the dominant kernel, the 512^2 and 2048^2 blocks (TFLOP/s, % of
peak, median and min, per-kernel split), the matrix-core rate a pure-MFMA probe sustains, and the
CPU oracle on a bounded sample. Per-step median and min come from events recorded between steps.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-backbone] [--no-cpu-baseline]
                       [--no-block-causal] [--no-backward] [--no-probe] [--no-other-blocks] [--cpu-rows R]
                       [--copy-calibration]
--copy-calibration first runs a plain elementwise copy (negation) of 1 GiB float32, a kernel of known
HBM traffic against which the rocprofv3 FETCH_SIZE / WRITE_SIZE counters are scaled.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Krea2 block TFLOP/s & % bf16 MFMA peak; denoise steps/s at 1024², B=2"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 1 << 30
KERNELS = ("modulation", "modnorm", "gemm_qkvg", "attention", "gemm_out", "gemm_swiglu", "gemm_down", "rope")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
_CSRC = os.path.join(ROOT, "flow_matching_diffusion_amd", "csrc")
_HEADERS = ("k2_device.h", "k2_kernels.h", "k2_tiles.h")
# The translation unit (and the headers it includes) that builds each kernel a traffic record covers.
KERNEL_SOURCES = {"gemm": ("gemm.hip",) + _HEADERS, "attention": ("attention.hip",) + _HEADERS,
                  "modnorm": ("elementwise.hip",) + _HEADERS}


def block_flops(d, B, L, valid_keys):
    """GEMMs over all B*L rows + attention over valid keys (4 hd nh per query-key pair)."""
    H, nh, nkv, hd, I = d.hidden, d.num_heads, d.num_kv_heads, d.head_dim, d.intermediate
    per_row = 2 * H * (2 * nh * hd + 2 * nkv * hd) + 2 * nh * hd * H + 6 * H * I
    return B * L * per_row + sum(4 * hd * nh * L * v for v in valid_keys)


def kernel_flops(d, M, name):
    H, nh, nkv, hd, I = d.hidden, d.num_heads, d.num_kv_heads, d.head_dim, d.intermediate
    return {"gemm_qkvg": 2 * M * H * (2 * nh * hd + 2 * nkv * hd), "gemm_out": 2 * M * nh * hd * H,
            "gemm_swiglu": 4 * M * H * I, "gemm_down": 2 * M * I * H}.get(name)


def source_hash(key):
    """Hash of the sources that build the kernel of traffic record `key` ("gemm_swiglu@block1024"):
    a record stays valid while they are unchanged, whatever happens to the other kernels."""
    dom = key.split("@")[0]
    files = next(v for k, v in KERNEL_SOURCES.items() if dom.startswith(k))
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(_CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_for(key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if the kernels have not
    changed since it was taken (else None)."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = t.get(key)
    if not e or e.get("source_sha") != source_hash(key):
        return None
    return e["fetch_bytes"] + e["write_bytes"]


def block_leg(k2, S, torch, dev, wl, steps, warmup):
    """k2_block_forward on workload wl (device-generated inputs of its shape): mean / median / min time
    per step, TFLOP/s and % of the bf16 peak, and the per-kernel split from further steps with events
    around every launch."""
    import ctypes

    import numpy as np
    d = wl.dims
    B, T, N, L = wl.B, wl.T, wl.N, wl.L
    f32 = torch.float32
    w = S.device_block_weights(wl.seed, "block.", d, wl.dtype, dev)
    h = S.device_normal(wl.seed, "hidden", (B, L, d.hidden), 1.0, f32, dev)
    if wl.t is not None:
        tw = S.device_model_weights(wl.seed, S.replace(wl, num_layers=0), dev)["time"]
        temb, _ = k2.timestep_modulation_forward(d.hidden, wl.timestep_embed_dim, wl.dtype, tw,
                                                 torch.tensor(wl.t, dtype=f32, device=dev))
    else:
        temb = S.device_normal(wl.seed, "temb", (B, 6 * d.hidden), 1.0, f32, dev)
    pos = torch.from_numpy(S.position_ids(T, *wl.grid)).to(dev)
    m = S.text_mask(B, T, wl.valid)
    mask = None if m is None else torch.from_numpy(m).to(dev)
    cfg = k2.block_cfg(d, wl.dtype)
    out = torch.empty_like(h)
    ws = torch.empty(k2.load().k2_block_workspace_bytes(ctypes.byref(cfg), B, T, N), dtype=torch.uint8, device=dev)

    def step():
        k2.block_forward(cfg, w, h, temb, pos, mask, T, out=out, workspace=ws)

    for _ in range(warmup):
        step()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    ms = max(wall, evs[0].elapsed_time(evs[-1]) / steps)
    valid = [L if wl.valid is None else N + v for v in (wl.valid or [L] * B)]
    flops = block_flops(d, B, L, valid)
    k2.profile_reset()
    k2.profile_filter(None)
    k2.profile_enable(True)
    nsplit = max(1, steps // 4)
    for _ in range(nsplit):
        step()
    torch.cuda.synchronize()
    k2.profile_enable(False)
    M = B * L
    kernels = {}
    for name in KERNELS:
        tot, n = k2.profile_query(name)
        if n:
            kernels[name] = {"avg_ms": round(tot / n, 4), "launches_per_step": n // nsplit}
            kf = kernel_flops(d, M, name)
            if name == "attention":
                kf = sum(4 * d.head_dim * d.num_heads * L * v for v in valid)
            if kf:
                kernels[name]["tflops"] = round(kf / (tot / n * 1e-3) / 1e12, 1)
                kernels[name]["pct_bf16_peak"] = round(100 * kf / (tot / n * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1)
    del w, h, out, ws
    torch.cuda.empty_cache()
    med = float(np.median(per))
    return {"config": {"B": B, "text_tokens": T, "valid_text": list(wl.valid or []), "grid": list(wl.grid), "L": L},
            "steps": steps, "ms_per_step": round(ms, 4), "median_ms": round(med, 4), "min_ms": round(min(per), 4),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1), "pct_bf16_peak": round(100 * flops / (ms * 1e-3) / 1e12 /
                                                                                  PEAK_BF16_TFLOPS, 2),
            "tflops_median": round(flops / (med * 1e-3) / 1e12, 1), "block_gflop": round(flops / 1e9, 1),
            "kernels": kernels}


def cpu_baseline(wl, rows):
    """The CPU oracle as it stands on a bounded sample of the same workload: batch row 0, keys and
    values for all of its rows, the whole block for `rows` sampled query rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from flow_matching_diffusion_amd import synth as S
    from oracle import k2_oracle as O

    wl1 = S.replace(wl, B=1, valid=None if wl.valid is None else wl.valid[:1],
                    t=None if wl.t is None else wl.t[:1])
    inp = S.block_inputs(wl1)
    if "temb" in inp:
        temb = inp["temb"]
    else:
        temb = O.time_path(inp["timestep"], inp["time_weights"], wl.timestep_embed_dim)[0].astype(np.float32)
    sel = S.sample_rows(wl1, rows)
    t0 = time.perf_counter()
    O.block_forward(inp["h"], temb, inp["position_ids"], inp["mask"], inp["weights"], wl.dims, wl.T, rows=sel)
    dt = time.perf_counter() - t0
    d = wl.dims
    L = wl.L
    valid = L if wl.valid is None else wl.N + wl.valid[0]
    per_row = 2 * d.hidden * (2 * d.num_heads * d.head_dim) + 2 * d.num_heads * d.head_dim * d.hidden + \
        6 * d.hidden * d.intermediate
    flops = 2 * L * d.hidden * 2 * d.num_kv_heads * d.head_dim + len(sel) * per_row + \
        4 * d.head_dim * d.num_heads * len(sel) * valid
    threads = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"value": round(flops / dt / 1e12, 4), "unit": "TFLOP/s", "cores": max(threads) if threads else 1,
            "cores_note": "BLAS threads the oracle's products ran on", "host_cpu_count": os.cpu_count(),
            "host_cpus_usable": len(os.sched_getaffinity(0)), "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"{wl.name} batch row 0: keys/values for all {L} rows + the whole block for {len(sel)} "
                      f"seeded query rows ({flops / 1e12:.3f} TFLOP), float64 NumPy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 15 untimed steps (about 0.1 s of the block at 1024^2): after 3, the first timed steps still ran
    # slow (the slowest of 20 at 7.20-7.28 ms against a median of 7.08 ms; after 15, 7.10-7.14)
    ap.add_argument("--warmup", type=int, default=15)
    ap.add_argument("--workload", default="block1024")
    ap.add_argument("--backbone-steps", type=int, default=5)
    ap.add_argument("--sampler-steps", type=int, default=3)
    ap.add_argument("--no-backbone", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-block-causal", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=4608)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--no-other-blocks", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the library runs on one GPU only; --gpus must be 1 (no multi-GPU path exists)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import flow_matching_diffusion_amd as k2
    from flow_matching_diffusion_amd import synth as S

    dev = torch.device("cuda:0")
    k2.load()
    if args.copy_calibration:
        src = torch.zeros(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    wl = S.WORKLOADS[args.workload]
    d = wl.dims
    B, T, N, L = wl.B, wl.T, wl.N, wl.L
    f32 = torch.float32

    w = S.device_block_weights(wl.seed, "block.", d, wl.dtype, dev)
    h = S.device_normal(wl.seed, "hidden", (B, L, d.hidden), 1.0, f32, dev)
    if wl.t is not None:
        tw = S.device_model_weights(wl.seed, S.replace(wl, num_layers=0), dev)["time"]
        temb, _ = k2.timestep_modulation_forward(d.hidden, wl.timestep_embed_dim, wl.dtype, tw,
                                                 torch.tensor(wl.t, dtype=f32, device=dev))
    else:
        temb = S.device_normal(wl.seed, "temb", (B, 6 * d.hidden), 1.0, f32, dev)
    pos = torch.from_numpy(S.position_ids(T, *wl.grid)).to(dev)
    m = S.text_mask(B, T, wl.valid)
    mask = None if m is None else torch.from_numpy(m).to(dev)
    cfg = k2.block_cfg(d, wl.dtype)
    out = torch.empty_like(h)
    import ctypes
    ws = torch.empty(k2.load().k2_block_workspace_bytes(ctypes.byref(cfg), B, T, N), dtype=torch.uint8, device=dev)

    def step():
        k2.block_forward(cfg, w, h, temb, pos, mask, T, out=out, workspace=ws)

    dom = "gemm_swiglu"  # the dominant kernel: its launches carry HIP events in the timed region
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    k2.profile_reset()
    k2.profile_filter(dom)
    k2.profile_enable(True)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k2.profile_enable(False)
    dom_tot, dom_n = k2.profile_query(dom)
    wall_ms = (t1 - t0) * 1e3 / args.steps
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    ev_ms = evs[0].elapsed_time(evs[-1]) / args.steps
    ms = max(wall_ms, ev_ms)
    valid_keys = [L if wl.valid is None else N + v for v in (wl.valid or [L] * B)]
    flops = block_flops(d, B, L, valid_keys)
    tflops = flops / (ms * 1e-3) / 1e12
    M = B * L
    # per-kernel split: the same steps again, every launch bracketed by events (not timed above)
    k2.profile_reset()
    k2.profile_filter(None)
    k2.profile_enable(True)
    nsplit = max(1, args.steps // 4)
    for _ in range(nsplit):
        step()
    torch.cuda.synchronize()
    k2.profile_enable(False)
    kernels = {}
    for name in KERNELS:
        tot, n = k2.profile_query(name)
        if n:
            kernels[name] = {"avg_ms": round(tot / n, 4), "launches_per_step": n // nsplit}
            kf = kernel_flops(d, M, name)
            if kf:
                kernels[name]["tflops"] = round(kf / (tot / n * 1e-3) / 1e12, 1)
                kernels[name]["pct_bf16_peak"] = round(100 * kf / (tot / n * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 1)
    kernels[dom]["avg_ms_timed_region"] = round(dom_tot / dom_n, 4)
    attn_flops = sum(4 * d.head_dim * d.num_heads * L * v for v in valid_keys)
    if "attention" in kernels:
        kernels["attention"]["tflops"] = round(attn_flops / (kernels["attention"]["avg_ms"] * 1e-3) / 1e12, 1)
        kernels["attention"]["pct_bf16_peak"] = round(100 * kernels["attention"]["tflops"] / PEAK_BF16_TFLOPS, 1)
    if "modnorm" in kernels:
        nbytes = M * d.hidden * (4 + (2 if wl.dtype == "bf16" else 4))
        kernels["modnorm"]["gbs"] = round(nbytes / (kernels["modnorm"]["avg_ms"] * 1e-3) / 1e9, 1)

    dom_flops = kernel_flops(d, M, dom)
    dom_ms = dom_tot / dom_n  # live, inside the timed region
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(f"{dom}@{wl.name}"),
                "algorithmic_per_launch": f"{dom_flops:.4e} FLOP (2*M*2I*H, M={M}, I={d.intermediate}, H={d.hidden})"}

    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic (seeded, device-generated N(0,1) activations, "
                                                           "N(0,0.02) weights)",
        "config": {"workload": wl.name, "B": B, "text_tokens": T, "valid_text": list(wl.valid or []),
                   "grid": list(wl.grid), "L": L, "hidden": d.hidden, "heads": d.num_heads, "kv_heads": d.num_kv_heads,
                   "head_dim": d.head_dim, "intermediate": d.intermediate, "timestep": list(wl.t or [])},
        "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "step_ms": {"mean": round(ms, 4), "median": round(float(np.median(per_step)), 4),
                    "min": round(min(per_step), 4), "max": round(max(per_step), 4),
                    "note": "value uses the mean over the timed region (max of wall clock and events); "
                            "median / min from events recorded between steps"},
        "pct_bf16_peak_median": round(100 * flops / (float(np.median(per_step)) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
        "block_gflop": round(flops / 1e9, 1),
        "kernels": kernels,
        "roofline": roofline,
    }

    # The matrix-core rate the part sustains with no memory traffic (k2_mfma_rate_probe), beside the
    # 2.4 GHz specification figure the percentages use.
    if not args.no_probe:
        pout = torch.zeros(4, dtype=torch.float32, device=dev)
        iters, blocks = 4000, 512
        k2.mfma_rate_probe(iters // 10, blocks, pout)
        torch.cuda.synchronize()
        pe = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        pe[0].record()
        k2.mfma_rate_probe(iters, blocks, pout)
        pe[1].record()
        torch.cuda.synchronize()
        p_tf = blocks * iters * 524288 / (pe[0].elapsed_time(pe[1]) * 1e-3) / 1e12
        result["mfma_probe"] = {"tflops": round(p_tf, 1), "pct_of_spec_peak": round(100 * p_tf / PEAK_BF16_TFLOPS, 1),
                                "block_pct_of_probe": round(100 * tflops / p_tf, 2),
                                "what": f"{blocks} workgroups x 4 waves, {iters} x 4 independent bf16 32x32x16 "
                                        "products per wave on registers, no memory traffic"}
        del pout

    # The other block workloads of the same full-size dims: the 512^2 block (B = 1, L = 1280, the small-M
    # GEMM case) and the 2048^2 long-sequence block (B = 1, L = 16896, attention-heavy), each timed like
    # the headline with its per-kernel split.
    if not args.no_other_blocks:
        legs = {}
        for name, nsteps in (("block512", max(args.steps, 50)), ("block2048", max(5, args.steps // 2))):
            legs[name] = block_leg(k2, S, torch, dev, S.WORKLOADS[name], nsteps, args.warmup)
        result["blocks"] = legs

    # The block-causal variant (k2_block_forward_block_causal) on the same pair: the image tokens as
    # a 1024-token condition block followed by the target block (condition images first, target
    # last). Text queries attend causally, condition queries the text and their own block, target
    # queries everything. Attention FLOPs count the keys each query may attend.
    if not args.no_block_causal and N > 1024:
        ids = np.concatenate([np.full(T, -1), np.zeros(1024), np.ones(N - 1024)]).astype(np.int32)
        reach = np.arange(L)
        for i in range(L - 2, -1, -1):
            if ids[i] >= 0 and ids[i + 1] == ids[i]:
                reach[i] = reach[i + 1]
        allowed = 0
        for b in range(B):
            kv = np.ones(L, bool)
            if m is not None:
                kv[:T] = m[b].astype(bool)
            allowed += int(np.cumsum(kv)[reach].sum())
        idt = torch.from_numpy(ids).to(dev)

        def bc_step():
            k2.block_forward(cfg, w, h, temb, pos, mask, T, out=out, workspace=ws, image_ids=idt)

        for _ in range(args.warmup):
            bc_step()
        torch.cuda.synchronize()
        k2.profile_reset()
        k2.profile_filter("attention")  # events around the attention launches only
        k2.profile_enable(True)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            bc_step()
        torch.cuda.synchronize()
        bc_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        k2.profile_enable(False)
        k2.profile_filter(None)
        a_tot, a_n = k2.profile_query("attention")
        bc_attn = 4 * d.head_dim * d.num_heads * allowed
        bc_flops = block_flops(d, B, L, [0] * B) + bc_attn
        a_ms = a_tot / a_n
        result["block_causal"] = {
            "layout": f"text {T} (causal) + condition block 1024 + target block {N - 1024}",
            "ms_per_step": round(bc_ms, 4), "tflops": round(bc_flops / (bc_ms * 1e-3) / 1e12, 1),
            "attention": {"avg_ms": round(a_ms, 4), "tflops": round(bc_attn / (a_ms * 1e-3) / 1e12, 1),
                          "algorithmic_tflop": round(bc_attn / 1e12, 4),
                          "bidirectional_algorithmic_tflop": round(attn_flops / 1e12, 4)}}
        del idt

    # The block's backward pass (k2_block_backward: the forward recomputed from the block input, then
    # every gradient: input, temb and all weights) on the same pair. Algorithmic FLOPs: the recompute
    # (the forward's) plus, for each projection, the input-gradient and weight-gradient products
    # (2x the forward's GEMM FLOPs), plus attention's four backward products (2x its forward).
    if not args.no_backward:
        del ws
        torch.cuda.empty_cache()
        gout = S.device_normal(wl.seed, "grad_out", (B, L, d.hidden), 1.0, f32, dev)
        bws = torch.empty(k2.block_backward_workspace_bytes(cfg, B, T, N), dtype=torch.uint8, device=dev)

        def bwd_step():
            return k2.block_backward(cfg, w, h, temb, pos, mask, T, gout, workspace=bws)

        for _ in range(max(1, args.warmup // 2)):
            res = bwd_step()
        del res
        torch.cuda.synchronize()
        nb = max(1, args.steps // 4)
        t0 = time.perf_counter()
        for _ in range(nb):
            res = bwd_step()
        torch.cuda.synchronize()
        b_ms = (time.perf_counter() - t0) * 1e3 / nb
        # per-kernel split: one more step with events around every launch (not timed above)
        k2.profile_reset()
        k2.profile_enable(True)
        res = bwd_step()
        torch.cuda.synchronize()
        k2.profile_enable(False)
        gemm_f = block_flops(d, B, L, [0] * B)
        b_flops = 3 * gemm_f + 3 * attn_flops
        bk = {}
        for name in ("gemm_qkvg", "attention", "gemm_swiglu", "gemm_plain", "transpose", "attention_bwd", "norm_bwd",
                     "gated_grad", "swiglu_bwd", "gate_bwd", "qknorm_bwd", "modnorm", "gated_add", "reduce_rows"):
            tot, n = k2.profile_query(name)
            if n:  # all launches of that kernel in the step
                bk[name] = {"ms_per_step": round(tot, 3), "launches": n}
        result["backward"] = {"ms_per_step": round(b_ms, 3), "tflops": round(b_flops / (b_ms * 1e-3) / 1e12, 1),
                              "algorithmic_tflop": round(b_flops / 1e12, 3), "kernels": bk,
                              "note": "forward recompute + all gradients; TFLOP = 3x forward GEMMs + 3x attention"}
        del res, bws, gout
        ws = None
    del w, h, out, ws
    torch.cuda.empty_cache()

    if not args.no_backbone:
        bwl = S.WORKLOADS["backbone1024"]
        mw = S.device_model_weights(bwl.seed, bwl, dev)
        x = S.device_normal(bwl.seed, "latents", (bwl.B, bwl.N, bwl.in_channels), 1.0,
                            torch.bfloat16 if bwl.dtype == "bf16" else f32, dev)
        enc = S.device_normal(bwl.seed, "encoder_hidden_states", (bwl.B, bwl.T, bwl.text.num_layers, bwl.text.hidden),
                              1.0, torch.bfloat16 if bwl.dtype == "bf16" else f32, dev)
        tt = torch.tensor(bwl.t, dtype=f32, device=dev)
        bpos = torch.from_numpy(S.position_ids(bwl.T, *bwl.grid)).to(dev)
        bm = torch.from_numpy(S.text_mask(bwl.B, bwl.T, bwl.valid)).to(dev)
        mcfg = k2.model_cfg(bwl.dims, bwl.text, bwl.num_layers, bwl.in_channels, bwl.timestep_embed_dim, bwl.dtype)
        bws = torch.empty(k2.backbone_workspace_bytes(mcfg, bwl.B, bwl.T, bwl.N), dtype=torch.uint8, device=dev)
        for _ in range(2):
            k2.backbone_forward(mcfg, mw, x, enc, tt, bpos, bm, workspace=bws)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.backbone_steps):
            v = k2.backbone_forward(mcfg, mw, x, enc, tt, bpos, bm, workspace=bws)
        torch.cuda.synchronize()
        bms = (time.perf_counter() - t0) * 1e3 / args.backbone_steps
        assert bool(torch.isfinite(v).all())
        bflops = bwl.num_layers * flops  # blocks only; text fusion and projections are extra work
        result["denoise_steps_per_s"] = round(1e3 / bms, 3)
        result["backbone"] = {"workload": bwl.name, "ms_per_step": round(bms, 2), "layers": bwl.num_layers,
                              "block_tflops_in_backbone": round(bflops / (bms * 1e-3) / 1e12, 1)}
        # the sampler on one image: k2_denoise_step (transformer on the prompt / negative-prompt pair,
        # guidance 4.5, as the base checkpoint's 28-step schedule) and without guidance (distilled, 8 steps)
        del bws
        lat = S.device_normal(bwl.seed, "latents", (1, bwl.N, bwl.in_channels), 1.0, f32, dev)
        sig = k2.flow_sigmas(28, bwl.N)
        sampler = {}
        for name, g, steps, G in (("base", 4.5, 28, 2), ("distilled", 0.0, 8, 1)):
            dws = torch.empty(k2.denoise_workspace_bytes(mcfg, bwl.T, bwl.N, g > 0), dtype=torch.uint8, device=dev)
            e, mk = enc[:G].contiguous(), bm[:G].contiguous()
            k2.denoise_step(mcfg, mw, lat, e, bpos, mk, float(sig[0]), float(sig[1]), g, workspace=dws)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(args.sampler_steps):
                k2.denoise_step(mcfg, mw, lat, e, bpos, mk, float(sig[i]), float(sig[i + 1]), g, workspace=dws)
            torch.cuda.synchronize()
            sms = (time.perf_counter() - t0) * 1e3 / args.sampler_steps
            del dws
            # the text rows once per prompt pair (k2_text_embed), then steps that reuse them
            tws = torch.empty(k2.text_embed_workspace_bytes(mcfg, G, bwl.T), dtype=torch.uint8, device=dev)
            cws = torch.empty(k2.denoise_cached_workspace_bytes(mcfg, bwl.T, bwl.N, g > 0), dtype=torch.uint8,
                              device=dev)
            txt = k2.text_embed(mcfg, mw, e, mk, workspace=tws)
            k2.denoise_step_cached(mcfg, mw, lat, txt, bpos, mk, float(sig[0]), float(sig[1]), g, workspace=cws)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            txt = k2.text_embed(mcfg, mw, e, mk, workspace=tws)
            torch.cuda.synchronize()
            tms = (time.perf_counter() - t0) * 1e3
            t0 = time.perf_counter()
            for i in range(args.sampler_steps):
                k2.denoise_step_cached(mcfg, mw, lat, txt, bpos, mk, float(sig[i]), float(sig[i + 1]), g,
                                       workspace=cws)
            torch.cuda.synchronize()
            cms = (time.perf_counter() - t0) * 1e3 / args.sampler_steps
            sampler[name] = {"guidance": g, "transformer_batch": G, "steps": steps, "timed_steps": args.sampler_steps,
                             "text_cached": {"text_embed_ms": round(tms, 2), "ms_per_step": round(cms, 2),
                                             "image_s": round((tms + steps * cms) / 1e3, 3)},
                             "text_every_step": {"ms_per_step": round(sms, 2),
                                                 "image_s": round(steps * sms / 1e3, 3)}}
            del tws, cws, txt
        assert bool(torch.isfinite(lat).all())
        result["sampler"] = sampler
        del mw, x, enc, lat
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
