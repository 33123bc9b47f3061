"""Pins of the adaptive draft-length oracle (oracle/adaptive.py) against
hand-derived traces (tests/golden/adaptive_k_cases.json), an independent
vectorised formulation of the window mean, and invariants; plus planted
mistakes that the pins must catch.  CPU only."""
import dataclasses
import importlib.util
import json
import os
import sys

import numpy as np
import pytest

from oracle import adaptive as A

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "adaptive_k_cases.json")
PRESETS = {"window50": A.preset_vllm_page, "last10": A.preset_checklist}


def _params(mod, case):
    p = {"window50": mod.preset_vllm_page, "last10": mod.preset_checklist}[case["preset"]]()
    return dataclasses.replace(p, **case["overrides"])


def test_presets_as_printed(mod=A):
    d = mod.preset_vllm_page()
    assert (d.k_min, d.k_max, d.k_init, d.window, d.min_history) == (2, 8, 2, 50, 10)
    assert d.up == 0.6 + 0.1 and d.down == 0.6 - 0.1
    b = mod.preset_checklist()
    assert (b.window, b.min_history, b.up, b.down, b.k_init) == (10, 10, 0.8, 0.5, 4)


def test_golden_traces(mod=A):
    spec = json.load(open(GOLDEN))
    assert "4.3" in spec["source"]
    for case in spec["cases"]:
        got = mod.trace(_params(mod, case), [tuple(s) for s in case["steps"]])
        assert got == case["expect_k"], case["name"]


def test_golden_stats_and_batches(mod=A):
    spec = json.load(open(GOLDEN))["stats_case"]
    bank = mod.Bank(_params(mod, {"preset": spec["preset"], "overrides": {}}), spec["num_slots"])
    for bt in spec["batches"]:
        cu = np.concatenate([[0], np.cumsum(bt["gammas"])])
        k, ncu = bank.step(bt["slots"], cu, bt["accepted"])
        assert ncu == [0] + list(np.cumsum(k))
    st = bank.stats
    assert [st.sequences, st.accepted, st.drafted, st.emitted] == spec["expect_totals"]
    assert st.accept_rate() == 0.5


def _vectorised_trace(p, steps):
    """Same rule, window means from a cumulative sum of dyadic ratios (exact
    in any order), decisions applied afterwards."""
    acc = np.array([a for a, _ in steps], dtype=np.float64)
    dr = np.maximum(np.array([d for _, d in steps], dtype=np.float64), 1.0)
    r = acc / dr
    c = np.concatenate([[0.0], np.cumsum(r)])
    out, k = [], p.k_init
    for t in range(len(steps)):
        n = min(t + 1, p.window)
        if n >= p.min_history:
            m = (c[t + 1] - c[t + 1 - n]) / n
            if m > p.up:
                k = min(k + 1, p.k_max)
            elif m < p.down:
                k = max(k - 1, p.k_min)
        out.append(k)
    return out


@pytest.mark.parametrize("preset", ["window50", "last10"])
def test_matches_vectorised_window_mean(preset, mod=A):
    """Long random traces with drafted = 4 (ratios are multiples of 1/4, so
    every window sum is exact whatever the order): same k sequence."""
    rng = np.random.default_rng(5 if preset == "window50" else 6)
    p = PRESETS[preset]()
    for regime in (0.2, 0.55, 0.9):
        steps = [(int(a), 4) for a in rng.binomial(4, regime, size=400)]
        assert mod.trace(p, steps) == _vectorised_trace(p, steps), regime


def test_invariants(mod=A):
    rng = np.random.default_rng(9)
    for _ in range(20):
        p = dataclasses.replace(A.preset_vllm_page(), window=int(rng.integers(1, 30)),
                                min_history=1, k_init=int(rng.integers(2, 9)))
        steps = []
        for _ in range(300):
            d = int(rng.integers(0, 9))
            steps.append((int(rng.integers(0, d + 1)), d))
        ks = mod.trace(p, steps)
        assert all(p.k_min <= k <= p.k_max for k in ks)
        assert all(abs(a - b) <= 1 for a, b in zip([p.k_init] + ks, ks))
    # a ratio stream inside the band never moves k
    p = A.preset_vllm_page()
    assert set(mod.trace(dataclasses.replace(p, k_init=5), [(3, 5)] * 100)) == {5}


MUTANTS = [
    ("non-strict growth threshold", "if avg > p.up:", "if avg >= p.up:"),
    ("window one too long", "recent = alphas[-p.window:]", "recent = alphas[-p.window - 1:]"),
    ("acts one ratio early", "if len(recent) < p.min_history:", "if len(recent) < p.min_history - 1:"),
    ("plain decode steps not guarded", "alphas.append(accepted / max(drafted, 1))",
     "alphas.append(accepted / max(drafted, 2))"),
    ("emitted without the drawn token", "self.stats.emitted += acc + 1", "self.stats.emitted += acc"),
    ("shrinks by two", "return max(k - 1, p.k_min)", "return max(k - 2, p.k_min)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(A.__file__).read()
    assert src.count(old) == 1, old
    path = tmp_path / "adaptive_mutant.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("adaptive_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    sys.modules["adaptive_mutant"] = mod     # dataclasses look their module up
    try:
        spec.loader.exec_module(mod)
    finally:
        del sys.modules["adaptive_mutant"]
    caught = []
    for fn, kw in ((test_presets_as_printed, {}), (test_golden_traces, {}),
                   (test_golden_stats_and_batches, {}),
                   (test_matches_vectorised_window_mean, {"preset": "window50"}),
                   (test_matches_vectorised_window_mean, {"preset": "last10"}),
                   (test_invariants, {})):
        try:
            fn(mod=mod, **kw)
        except AssertionError:
            caught.append(fn.__name__)
    assert caught, f"no pin caught: {name}"
