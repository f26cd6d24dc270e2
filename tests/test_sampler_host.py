"""The sampler's host side through the C ABI (no GPU): k2_flow_sigmas against the oracle's schedule,
the shift defaults against the pipeline page's printed parameters, and host validation of
k2_cfg_euler_update / k2_denoise_step (fake device addresses, every case fails before a launch)."""
import ctypes
import json
import os

import numpy as np

import flow_matching_diffusion_amd as k2
import oracle.k2_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sampler_defaults.json")
OK, ENULL, ESHAPE, ECONFIG, EWS, EALIGN = 0, -1, -2, -3, -5, -7
FAKE = 0x7F0000000000


def test_shift_defaults_match_pipeline_page():
    g = json.load(open(GOLDEN))
    c = k2.shift_cfg()
    assert c.base_image_seq_len == g["base_image_seq_len"] and c.max_image_seq_len == g["max_image_seq_len"]
    for k in ("base_shift", "max_shift", "distilled_mu"):
        assert abs(getattr(c, k) - g[k]) < 1e-7, k


def test_flow_sigmas_match_oracle():
    for n, tokens, dist in ((28, 4096, False), (8, 4096, True), (1, 256, False), (50, 16384, False), (3, 6400, False),
                            (28, 1024, False)):
        got = k2.flow_sigmas(n, tokens, dist)
        ref = O.flow_sigmas(n, tokens, dist)
        assert got.shape == (n + 1,) and got[0] == 1.0 and got[-1] == 0.0
        np.testing.assert_allclose(got, ref, rtol=0, atol=2e-7)  # float32 rounding of the same definition


def test_flow_sigmas_custom_shift_and_errors():
    zero = k2.shift_cfg(base_shift=0.0, max_shift=0.0)
    np.testing.assert_allclose(k2.flow_sigmas(28, 4096, cfg=zero)[:-1], np.linspace(1, 1 / 28, 28), atol=1e-7)
    lib = k2.load()
    out = (ctypes.c_float * 4)()
    assert lib.k2_flow_sigmas(None, 0, 4096, 0, out) == ESHAPE
    assert lib.k2_flow_sigmas(None, 3, 0, 0, out) == ESHAPE
    assert lib.k2_flow_sigmas(None, 3, 4096, 0, None) == ENULL
    bad = k2.shift_cfg(max_image_seq_len=256)
    assert lib.k2_flow_sigmas(ctypes.byref(bad), 3, 4096, 0, out) == ECONFIG


def test_cfg_euler_update_validation():
    lib = k2.load()
    assert lib.k2_cfg_euler_update(FAKE, FAKE, FAKE, None, 64, 4.5, 1.0, 0.9, None) == ENULL  # uncond needed
    assert lib.k2_cfg_euler_update(FAKE, FAKE, None, None, 64, 0.0, 1.0, 0.9, None) == ENULL
    assert lib.k2_cfg_euler_update(FAKE + 4, FAKE, FAKE, FAKE, 64, 4.5, 1.0, 0.9, None) == EALIGN
    assert lib.k2_cfg_euler_update(FAKE, FAKE, FAKE, FAKE, 64, float("nan"), 1.0, 0.9, None) == ESHAPE
    assert lib.k2_cfg_euler_update(None, None, None, None, 0, 4.5, 1.0, 0.9, None) == OK  # nothing to do


def test_denoise_step_validation():
    from tests.test_abi import good_weights
    from flow_matching_diffusion_amd import _abi
    lib = k2.load()
    cfg = _abi.ModelCfg()
    lib.k2_model_cfg_default(ctypes.byref(cfg))
    cfg.num_layers = 1
    cfg.text.num_layerwise_blocks = 1
    cfg.text.num_refiner_blocks = 1
    bw = (_abi.BlockWeights * 1)(good_weights())
    tb = (_abi.BlockWeights * 1)(good_weights())
    tb[0].scale_shift_table = None
    tw = _abi.TextWeights(tb, FAKE, tb)
    tmw = _abi.TimeWeights(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    mw = _abi.ModelWeights()
    mw.img_in_w = mw.img_in_b = mw.txt_in_w = mw.txt_in_b = FAKE
    mw.final_table = mw.final_w = mw.final_b = FAKE
    mw.time, mw.text, mw.blocks = tmw, tw, bw
    T, N = 8, 16
    need = lib.k2_denoise_workspace_bytes(ctypes.byref(cfg), T, N, 1)
    assert need > lib.k2_denoise_workspace_bytes(ctypes.byref(cfg), T, N, 0) > 0

    def call(latents=FAKE, enc=FAKE, pos=FAKE, rows=T + N, cols=3, g=4.5, ws=FAKE, nbytes=need):
        return lib.k2_denoise_step(ctypes.byref(cfg), ctypes.byref(mw), T, N, latents, enc, None, pos, rows, cols,
                                   0.9, 0.8, g, ws, nbytes, None)

    assert call(latents=None) == ENULL
    assert call(enc=None) == ENULL
    assert call(rows=T + N - 1) == ESHAPE
    assert call(g=float("inf")) == ESHAPE
    assert call(latents=FAKE + 8) == EALIGN
    assert call(nbytes=need - 1) == EWS
