"""The streamed backbone that writes the 28-block fixture computes exactly oracle.backbone_forward
(checked on a small model on the CPU), and the fixture's key tracks the code it was made with."""
import importlib.util
import os

import numpy as np

from flow_matching_diffusion_amd import synth as S
from oracle import k2_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _script():
    spec = importlib.util.spec_from_file_location("bb_fixture", os.path.join(HERE, "golden", "backbone1024_oracle.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_streamed_backbone_equals_oracle_backbone():
    m = _script()
    td = S.TextDims(hidden=32, num_heads=4, num_kv_heads=4, head_dim=8, intermediate=24, num_layers=3)
    d = S.BlockDims(hidden=32, num_heads=4, num_kv_heads=2, head_dim=8, intermediate=16, axes_dims=(2, 2, 4))
    wl = S.Workload("mb", 57, "bf16", 2, 4, (2, 3), (3, 1), t=(0.7, 0.7), dims=d, text=td, num_layers=3,
                    in_channels=8, timestep_embed_dim=16)
    got = m.streamed_backbone(wl, m.FORMS, log=lambda s: None)
    mw = S.model_weights(wl.seed, wl)
    inp = S.backbone_inputs(wl)
    for name, rnd in m.FORMS.items():
        ref = O.backbone_forward(S.as_dtype(inp["x"], wl.dtype), inp["enc"], inp["timestep"], inp["position_ids"],
                                 inp["mask"], mw, d, S.text_block_dims(td), wl.T, time_dim=16, rnd=rnd)
        np.testing.assert_array_equal(got[name], ref, err_msg=name)


def test_fixture_key_ignores_docstrings_only():
    m = _script()
    src = "def f(x):\n    'doc'\n    return x + 1\n"
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        p = os.path.join(d, "a.py")
        open(p, "w").write(src)
        h0 = m.code_hash(p)
        open(p, "w").write(src.replace("'doc'", "'other doc'  # comment"))
        assert m.code_hash(p) == h0
        open(p, "w").write(src.replace("x + 1", "x + 2"))
        assert m.code_hash(p) != h0


def test_stored_model_statistics_match_the_code():
    """The committed oracle outputs (the 28-block fixture, the block512 gradient statistics) were
    written by the oracle and generators in the tree: a stale file fails here, on the CPU."""
    import json
    from tests.golden.block512_backward_stats import OUT, stats_key
    m = _script()
    fx = np.load(m.OUT, allow_pickle=False)
    assert str(fx["key"]) == m.fixture_key(S.WORKLOADS["backbone1024"])
    st = json.load(open(OUT))
    assert st["key"] == stats_key(S.WORKLOADS["block512"])
    for k in ("h", "temb", "ff_down"):
        for f in ("A", "B", "C"):
            assert 0 < st["stats"][k][f]["rms"] <= st["stats"][k][f]["p999"] <= st["stats"][k][f]["max"]


def test_block512_statistics_give_finite_backward_bounds():
    """The bound the block1024 backward test applies, computed here from the stored statistics: each
    is finite, no tighter than the largest realisation and, for max, within the spread's range."""
    import json
    from tests.golden.block512_backward_stats import OUT
    from tests.k2_testutil import SPREAD, spread_bound
    st = json.load(open(OUT))["stats"]
    for k in ("h", "temb", "ff_down"):
        for stat in ("max", "p999", "rms"):
            forms = [st[k][f] for f in ("A", "B", "C")]
            b = spread_bound("backward", stat, forms)
            top = max(f[stat] for f in forms)
            assert np.isfinite(b) and top <= b <= SPREAD["factor"]["backward"]["max"] * top, (k, stat, b)

