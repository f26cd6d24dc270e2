"""Helpers shared by the GPU parity tests (inputs from synth, expected values from the oracle)."""
from __future__ import annotations

import ctypes
import json
import os

import numpy as np
import pytest

from flow_matching_diffusion_amd import synth as S


def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def rel_err(got, ref):
    """(max |got - ref|, rms |got - ref|) / rms(ref): the parity metric."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    d = np.abs(got - ref)
    return d.max() / rms, np.sqrt(np.mean(d * d)) / rms


TOL = {"f32": 1e-4, "bf16": 2e-2}
# How far one more bf16 realisation's error statistic can land above the largest of the three forms
# the tests compute, per kind of output; measured on the oracle alone by tests/golden/bf16_spread_study.py.
SPREAD = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "bf16_spread.json")))


def err_stats(got, ref, rms):
    """max, 99.9th percentile and rms of |got - ref| relative to rms (the exact output's), and the
    fraction of elements above the 2e-2 figure."""
    d = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    return {"max": d.max() / rms, "p999": float(np.quantile(d, 0.999)) / rms,
            "rms": float(np.sqrt(np.mean(d * d))) / rms, "frac": float(np.mean(d > TOL["bf16"] * rms))}


def spread_bound(kind, stat, realisations):
    """Largest error one more bf16 realisation may show for statistic `stat` (max, p999, rms) of an
    output of `kind` (forward, backward): SPREAD's factor times the largest of the given
    realisations' statistics (a list of err_stats-like dicts)."""
    return SPREAD["factor"][kind][stat] * max(r[stat] for r in realisations)


def _fmt(st):
    return f"max {st['max']:.3e} p99.9 {st['p999']:.3e} rms {st['rms']:.3e} >2e-2: {st['frac']:.2e}"


def parity(tag, dtype, got, oracle_fn, kind="forward"):
    """fp32: max|gpu - exact| / rms(exact) <= 1e-4.

    bf16: the bf16 model hands its matrix products bf16 operands; its deviation from the exact
    function is set by that rounding, not by the kernels, and a small change anywhere re-draws the
    rounding of every later point. The oracle computes three legitimate realisations of the bf16
    model on the same inputs (R13): A, the plain one (normalised probabilities rounded, float64
    products); B, the fused-attention softmax form; C, form B with float32 products, as matrix
    cores accumulate. The GPU is one more realisation. Asserted:
      * against the exact oracle: max, p99.9 and rms of the GPU's error are each at most the largest
        of A's, B's and C's times SPREAD's factor for that statistic and kind of output (how far one
        more realisation was seen to land above the largest of those three, on the oracle alone);
      * against A, the bf16-operand oracle: p99.9 and rms of |gpu - A| are at most sqrt(2) times the
        largest of the GPU's and the emulations' deviation from exact (times the rms factor): two
        realisations with independent rounding noise differ by that much, and only a GPU error that
        is larger than the model's or anti-correlated with it exceeds it.
    Printed for every case: the statistics of the GPU and of A, B and C against exact, of the GPU
    and of B and C against A, and whether the 2e-2 figure holds. Returns the GPU's statistics."""
    from oracle import k2_oracle as O
    assert np.all(np.isfinite(got)), f"{tag}: non-finite output"
    exact = oracle_fn(None)
    rms = float(np.sqrt(np.mean(np.asarray(exact, np.float64) ** 2)))
    g = err_stats(got, exact, rms)
    if dtype == "f32":
        print(f"{tag}: max rel err {g['max']:.3e}, rms {g['rms']:.3e}", flush=True)
        assert g["max"] <= TOL["f32"], f"{tag}: {g['max']:.3e} > {TOL['f32']}"
        return g
    em = {"A": oracle_fn(O.bf16_form()), "B": oracle_fn(O.bf16_form(flash=True)),
          "C": oracle_fn(O.bf16_form(flash=True, f32_products=True))}
    e = {k: err_stats(v, exact, rms) for k, v in em.items()}
    gA = err_stats(got, em["A"], rms)
    eA = {k: err_stats(em[k], em["A"], rms) for k in ("B", "C")}
    fac = SPREAD["factor"][kind]
    print(f"{tag}: GPU vs exact {_fmt(g)} | 2e-2 {'met' if g['max'] <= TOL['bf16'] else 'NOT met'}", flush=True)
    for k in "ABC":
        print(f"{tag}:   {k} vs exact {_fmt(e[k])}", flush=True)
    print(f"{tag}: GPU vs A {_fmt(gA)}; B vs A {_fmt(eA['B'])}; C vs A {_fmt(eA['C'])}", flush=True)
    for s in ("max", "p999", "rms"):
        bound = spread_bound(kind, s, [e[k] for k in "ABC"])
        assert g[s] <= bound, f"{tag}: GPU {s} vs exact {g[s]:.3e} > {fac[s]:.3f} x largest of A/B/C = {bound:.3e}"
    for s in ("p999", "rms"):
        lim = fac["rms"] * np.sqrt(2.0) * max([g[s]] + [e[k][s] for k in "ABC"])
        assert gA[s] <= lim, f"{tag}: GPU {s} vs A {gA[s]:.3e} > independent-noise limit {lim:.3e}"
    return g


def temb_for(wl, inp):
    """float32 temb fed to both sides: the workload's own N(0,1) vector, or the exact oracle time
    path of t (the time path has its own parity test)."""
    from oracle import k2_oracle as O
    if "temb" in inp:
        return inp["temb"]
    temb, _ = O.time_path(inp["timestep"], inp["time_weights"], wl.timestep_embed_dim)
    return temb.astype(np.float32)


def gpu_block(wl, inp, temb, h=None, mask="default", dev=None, keep_ws=False, image_ids=None):
    """Run k2_block_forward (k2_block_forward_block_causal with image_ids) on the workload's inputs;
    returns the output (and workspace)."""
    import torch
    import flow_matching_diffusion_amd as k2
    dev = dev or device()
    cfg = k2.block_cfg(wl.dims, wl.dtype)
    w = k2.upload(inp["weights"], wl.dtype, dev)
    h = inp["h"] if h is None else h
    m = inp["mask"] if isinstance(mask, str) else mask
    ht = torch.from_numpy(np.ascontiguousarray(h)).to(dev)
    tt = None if temb is None else torch.from_numpy(np.ascontiguousarray(temb, dtype=np.float32)).to(dev)
    pt = None if inp["position_ids"] is None else torch.from_numpy(inp["position_ids"]).to(dev)
    mt = None if m is None else torch.from_numpy(np.ascontiguousarray(m)).to(dev)
    B, L, _ = h.shape
    ws = torch.empty(k2.load().k2_block_workspace_bytes(ctypes.byref(cfg), B, wl.T, L - wl.T),
                     dtype=torch.uint8, device=dev)
    it = None if image_ids is None else torch.from_numpy(np.ascontiguousarray(image_ids, dtype=np.int32)).to(dev)
    out = k2.block_forward(cfg, w, ht, tt, pt, mt, wl.T, workspace=ws, image_ids=it)
    torch.cuda.synchronize()
    res = out.cpu().numpy()
    if keep_ws:
        return res, ws, cfg
    return res


def workload(name, **kw):
    wl = S.WORKLOADS[name]
    return S.replace(wl, **kw) if kw else wl
