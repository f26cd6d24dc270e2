"""Pins of the oracle's sampler (flow-match Euler with the resolution-aware shift and guidance;
readings R14 - R16 of oracle/k2_oracle.py) to the pipeline page's printed parameters, closed forms
and invariants. CPU only. [PIPELINE] is the diffusers v0.43.0 pipeline page 'Krea 2'."""
import json
import math
import os

import numpy as np

import oracle.k2_oracle as O
from flow_matching_diffusion_amd import synth as S
from tests.test_oracle_pins import TEXT_MICRO, micro_backbone

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden():
    return json.load(open(os.path.join(GOLDEN, "sampler_defaults.json")))


def test_shift_parameters_are_the_pages():
    g = golden()
    for k in ("base_shift", "max_shift", "base_image_seq_len", "max_image_seq_len", "distilled_mu"):
        assert O.SHIFT_DEFAULTS[k] == g[k], k


def test_mu_line_endpoints_and_distilled():
    # [PIPELINE] Krea2Pipeline: mu from the resolution, between (256, 0.5) and (6400, 1.15); fixed 1.15
    # when distilled. A swapped slope or offset fails the endpoints.
    g = golden()
    assert math.isclose(O.shift_mu(g["base_image_seq_len"]), g["base_shift"], abs_tol=1e-15)
    assert math.isclose(O.shift_mu(g["max_image_seq_len"]), g["max_shift"], abs_tol=1e-15)
    tokens = (g["default_size"] // g["pixels_per_token"]) ** 2  # 4096 at 1024x1024
    assert tokens == 4096
    assert math.isclose(O.shift_mu(tokens), 0.5 + 0.65 * (4096 - 256) / 6144, abs_tol=1e-15)
    assert O.shift_mu(tokens, distilled=True) == g["distilled_mu"]
    assert O.shift_mu(123456, distilled=True) == g["distilled_mu"]


def test_time_shift_closed_forms():
    s = np.linspace(0.01, 1.0, 50)
    np.testing.assert_allclose(O.time_shift(0.0, s), s, rtol=0, atol=1e-15)  # identity at mu = 0
    for mu in (0.5, 0.90625, 1.15):
        assert O.time_shift(mu, 1.0) == 1.0                                   # pure noise stays put
        t = O.time_shift(mu, s)
        assert np.all(np.diff(t) > 0) and np.all(t >= s - 1e-15)               # monotone, pushed to noise
    # mu = ln 2: 2 sigma / (sigma + 1)
    np.testing.assert_allclose(O.time_shift(math.log(2.0), s), 2 * s / (s + 1), rtol=1e-14)


def test_sigma_grid():
    g = golden()
    for n, tokens, dist in ((g["steps_base"], 4096, False), (g["steps_distilled"], 4096, True), (1, 256, False)):
        sig = O.flow_sigmas(n, tokens, dist)
        assert sig.shape == (n + 1,) and sig[0] == 1.0 and sig[-1] == 0.0
        assert np.all(np.diff(sig) < 0)
    # with both shift endpoints at 0 the grid is the page's unshifted linspace(1, 1/N, N)
    sig = O.flow_sigmas(28, 4096, base_shift=0.0, max_shift=0.0)
    np.testing.assert_allclose(sig[:-1], np.linspace(1.0, 1.0 / 28, 28), rtol=0, atol=1e-15)


def test_guidance_convention():
    # [PIPELINE] guidance_scale: cond + g (cond - uncond); 0 disables guidance
    rng = np.random.default_rng(3)
    c, u = rng.standard_normal((2, 5, 7))
    np.testing.assert_array_equal(O.cfg_velocity(c, u, 0.0), c)
    np.testing.assert_array_equal(O.cfg_velocity(c, c, 4.5), c)
    np.testing.assert_allclose(O.cfg_velocity(c, u, 1.0), 2 * c - u, rtol=1e-15)
    np.testing.assert_allclose(O.cfg_velocity(c, u, 4.5), 5.5 * c - 4.5 * u, rtol=1e-14, atol=1e-14)


def test_euler_loop_on_constant_velocity_lands_on_x0_minus_v():
    # the updates telescope: sum of (sigma_{i+1} - sigma_i) over the grid is 0 - 1
    rng = np.random.default_rng(4)
    x0, v = rng.standard_normal((2, 3, 4))
    sig = O.flow_sigmas(28, 4096)
    x = x0
    for i in range(28):
        x = O.euler_step(x, v, sig[i], sig[i + 1])
    np.testing.assert_allclose(x, x0 - v, rtol=1e-12, atol=1e-12)


def _sampler_case(seed=61, T=4, grid=(2, 3), valid=(3, 2)):
    wl, d, mw, inp = micro_backbone(seed=seed, B=2, T=T, grid=grid, valid=valid, in_ch=8)
    x = inp["x"][:1]
    enc, enc_neg = inp["enc"][:1], inp["enc"][1:]
    m, mn = inp["mask"][:1], inp["mask"][1:]
    return wl, d, mw, inp, x, enc, enc_neg, m, mn


def test_denoise_step_batches_cond_and_uncond_independently():
    # the (cond, uncond) pair shares one batched transformer call; each row must equal its own
    # single-row call (batch rows are independent), and the update must use cond first
    wl, d, mw, inp, x, enc, enc_neg, m, mn = _sampler_case()
    td = S.text_block_dims(TEXT_MICRO)
    sig, sig_next, g = 0.8, 0.7, 4.5
    got = O.denoise_step(x, enc, enc_neg, m, mn, inp["position_ids"], mw, d, td, wl.T, sig, sig_next, g, time_dim=16)
    vc = O.backbone_forward(x, enc, np.array([sig]), inp["position_ids"], m, mw, d, td, wl.T, time_dim=16)
    vu = O.backbone_forward(x, enc_neg, np.array([sig]), inp["position_ids"], mn, mw, d, td, wl.T, time_dim=16)
    ref = x + (sig_next - sig) * (vc + g * (vc - vu))
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)
    # guidance 0: cond only
    got0 = O.denoise_step(x, enc, enc_neg, m, mn, inp["position_ids"], mw, d, td, wl.T, sig, sig_next, 0.0,
                          time_dim=16)
    np.testing.assert_allclose(got0, x + (sig_next - sig) * vc, rtol=1e-12, atol=1e-12)
