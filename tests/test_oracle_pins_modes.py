"""Pins of the oracle's greedy and point-mass-draft verification.

As in test_oracle_pins.py, nothing here re-types the oracle's procedure.
Greedy verification is pinned against numpy's argmax (first occurrence, i.e.
the lowest id among equal maxima), hand-worked cases under tests/golden/, and
the temperature -> 0 limit of the (separately pinned) sampled oracle.
Point-mass drafts are pinned against hand-worked cases, the sampled oracle
with draft logits that make q exactly the point mass, the exact threshold
p(x) of the accept test, and an exact count over a grid of uniform pairs
that recovers the output law p (losslessness).
"""
import json
import os

import numpy as np
import pytest
from scipy import special

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rows(rows):
    return np.asarray([[float(v) for v in r] for r in rows], dtype=np.float64)


def _ragged(rng, gammas, V, dtype, sd=2.0):
    """A random packed batch (target rows only) with ragged gammas."""
    gammas = np.asarray(gammas, dtype=np.int32)
    R_t = int(gammas.sum()) + len(gammas)
    tgt = W.to_dtype(rng.standard_normal((R_t, V)) * sd, dtype)
    return gammas, W.cu_from_gammas(gammas), tgt


# ------------------------------------------------------------ greedy

def test_greedy_golden_cases(oracle_lib):
    spec = json.load(open(os.path.join(GOLDEN, "greedy_cases.json")))
    assert "流程编排" in spec["source"]
    for case in spec["cases"]:
        tgt = _rows(case["target"]).astype(np.float32)
        res = oracle_lib.verify_greedy(len(case["gammas"]), W.cu_from_gammas(case["gammas"]),
                                       tgt, np.asarray(case["tokens"], np.int32))
        assert res.out_tokens.tolist() == case["expect_tokens"], case["name"]
        assert res.num_accepted.tolist() == case["expect_accepted"], case["name"]
    # all cases packed into one ragged batch give the same per-sequence results
    gam = sum((c["gammas"] for c in spec["cases"]), [])
    V = spec["cases"][0]["V"]
    assert all(c["V"] == V for c in spec["cases"])
    tgt = np.concatenate([_rows(c["target"]) for c in spec["cases"]]).astype(np.float32)
    tok = np.asarray(sum((c["tokens"] for c in spec["cases"]), []), np.int32)
    res = oracle_lib.verify_greedy(len(gam), W.cu_from_gammas(gam), tgt, tok)
    assert res.out_tokens.tolist() == sum((c["expect_tokens"] for c in spec["cases"]), [])
    assert res.num_accepted.tolist() == sum((c["expect_accepted"] for c in spec["cases"]), [])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_greedy_argmax_is_numpy_first_occurrence(oracle_lib, dtype):
    """Row argmaxes equal numpy's argmax (first maximum).  bf16 rows of a
    narrow range hold many tied maxima, and some rows are given explicit ties
    and -inf entries."""
    rng = np.random.default_rng(11)
    gammas, cu, tgt = _ragged(rng, [0, 3, 7, 1, 0, 5, 2], 300, dtype, sd=0.4)
    vals = W.to_f64(tgt, dtype)
    vals[2, [5, 17, 250]] = vals[2].max() + 1.0          # three tied maxima
    vals[4, :] = -np.inf
    vals[5, :100] = -np.inf
    tgt = W.to_dtype(vals, dtype)
    vals = W.to_f64(tgt, dtype)
    tok = rng.integers(0, 300, size=int(cu[-1])).astype(np.int32)
    res = oracle_lib.verify_greedy(len(gammas), cu, tgt, tok, dtype=dtype)
    np.testing.assert_array_equal(res.argmax, np.argmax(vals, axis=1))
    assert res.argmax[2] == 5 and res.argmax[4] == 0


def test_greedy_is_the_zero_temperature_limit_of_sampled_verify(oracle_lib):
    """With unique argmaxes, gaps >= 1 between a row's maximum and the rest,
    T = 1e-3 and draft logits that make q the point mass at the draft token,
    every p is exactly one-hot in float64 (exp(-1000) underflows to 0).
    Then u < p(x) / 1 accepts iff x is the argmax, the residual and the bonus
    are the point mass at the argmax, and the sampled oracle must emit what
    greedy verification emits, for any uniforms."""
    rng = np.random.default_rng(5)
    V = 64
    gammas = np.asarray([4, 0, 6, 3, 8, 1, 2], np.int32)
    cu = W.cu_from_gammas(gammas)
    R_t = int(gammas.sum()) + len(gammas)
    base = rng.integers(-20, 0, size=(R_t, V)).astype(np.float64)
    top = rng.integers(0, V, size=R_t)
    base[np.arange(R_t), top] = 5.0                      # unique maximum, gap >= 5
    tgt = base.astype(np.float32)
    tok = np.empty(int(cu[-1]), np.int32)
    for b, g in enumerate(gammas):
        for i in range(g):
            row = int(cu[b]) + b + i
            tok[int(cu[b]) + i] = top[row] if rng.random() < 0.75 else (top[row] + 1) % V
    dft = np.full((int(cu[-1]), V), -np.inf, np.float32)
    dft[np.arange(int(cu[-1])), tok] = 0.0
    u = W.uniform_grid24(rng, R_t)
    greedy = oracle_lib.verify_greedy(len(gammas), cu, tgt, tok)
    sampled = oracle_lib.verify(len(gammas), cu, tgt, dft, tok, u, np.float32(1e-3))
    np.testing.assert_array_equal(greedy.out_tokens, sampled.out_tokens)
    np.testing.assert_array_equal(greedy.num_accepted, sampled.num_accepted)
    assert (greedy.num_accepted < gammas).any() and (greedy.num_accepted == gammas).any()


def test_greedy_rejects_bad_arguments(oracle_lib):
    tgt = np.zeros((2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle_lib.verify_greedy(1, W.cu_from_gammas([1]), tgt, np.asarray([4], np.int32))
    with pytest.raises(ValueError):
        oracle_lib.verify_greedy(1, W.cu_from_gammas([1]), tgt, np.asarray([-1], np.int32))


# ------------------------------------------------------------ point-mass drafts

def test_point_draft_golden_cases(oracle_lib):
    spec = json.load(open(os.path.join(GOLDEN, "point_draft_cases.json")))
    for case in spec["cases"]:
        tgt = _rows(case["target"]).astype(np.float32)
        res = oracle_lib.verify_onehot(len(case["gammas"]), W.cu_from_gammas(case["gammas"]),
                                       tgt, np.asarray(case["tokens"], np.int32),
                                       np.asarray(case["uniforms"], np.float32), case["T"])
        assert res.out_tokens.tolist() == case["expect_tokens"], case["name"]
        assert res.num_accepted.tolist() == case["expect_accepted"], case["name"]
        np.testing.assert_allclose(res.residual_sum, case["expect_residual_sum"], atol=1e-7)
        assert res.flagged.tolist() == [case.get("expect_flagged", 0)], case["name"]


@pytest.mark.parametrize("dtype,T", [("f32", 1.0), ("bf16", 0.7), ("bf16", 1.3)])
def test_point_drafts_equal_sampled_verify_with_point_mass_q(oracle_lib, dtype, T):
    """Draft logits of -inf everywhere except 0 at the draft token make
    q = softmax(l_q / T) exactly the point mass: the sampled oracle (pinned
    on its own) must then give identical outputs and diagnostics."""
    rng = np.random.default_rng(23)
    V = 500
    gammas, cu, tgt = _ragged(rng, [3, 0, 8, 1, 5, 2, 0, 4], V, dtype)
    R_d = int(cu[-1])
    tok = rng.integers(0, V, size=R_d).astype(np.int32)
    # make several drafts likely: put each draft token near its row's top
    vals = W.to_f64(tgt, dtype)
    for b, g in enumerate(gammas):
        for i in range(g):
            row = int(cu[b]) + b + i
            vals[row, tok[int(cu[b]) + i]] = vals[row].max() + rng.uniform(0.0, 8.0)
    tgt = W.to_dtype(vals, dtype)
    dft = W.to_dtype(np.full((R_d, V), -np.inf), dtype)
    dft[np.arange(R_d), tok] = W.to_dtype(np.zeros(R_d), dtype)
    u = W.uniform_grid24(rng, len(tgt))
    point = oracle_lib.verify_onehot(len(gammas), cu, tgt, tok, u, np.float32(T), dtype=dtype)
    ref = oracle_lib.verify(len(gammas), cu, tgt, dft, tok, u, np.float32(T), dtype=dtype)
    for f in ("out_tokens", "num_accepted", "flagged"):
        np.testing.assert_array_equal(getattr(point, f), getattr(ref, f), err_msg=f)
    for f in ("p_draft", "q_draft", "residual_sum"):
        np.testing.assert_array_equal(getattr(point, f), getattr(ref, f), err_msg=f)
    # the distances are reported less the error bound, which for the sampled
    # oracle includes a few ulps for q's normaliser (exact here, but bounded
    # as computed)
    for f in ("tie_final", "final_err"):
        np.testing.assert_allclose(getattr(point, f), getattr(ref, f), rtol=0, atol=1e-14,
                                   err_msg=f)
    assert 0 < (point.num_accepted > 0).sum() < len(gammas)


def test_point_draft_accept_threshold_is_p_of_x(oracle_lib):
    """n flips from 1 to 0 exactly where u crosses p(x) (scipy softmax)."""
    rng = np.random.default_rng(3)
    V = 50
    rows = rng.standard_normal((2, V)) * 1.5
    tgt = rows.astype(np.float32)
    x = int(np.argsort(rows[0])[-3])
    px = special.softmax(tgt[0].astype(np.float64))[x]
    for u0, want in ((px * (1 - 1e-5), 1), (px * (1 + 1e-5), 0)):
        res = oracle_lib.verify_onehot(1, W.cu_from_gammas([1]), tgt, np.asarray([x], np.int32),
                                       np.asarray([u0, 0.5], np.float32), 1.0)
        assert int(res.num_accepted[0]) == want, (u0, px)
        np.testing.assert_allclose(res.p_draft[0], px, rtol=1e-12)


def test_point_draft_output_law_by_grid_count(oracle_lib):
    """Lossless output: over an N x N grid of (accept uniform, draw
    uniform), the emitted first token has frequencies p within the grid's
    counting error 2/N + 2/N per token."""
    N = 512
    logits = np.log(np.asarray([0.1, 0.25, 0.05, 0.4, 0.2]))
    tgt1 = np.tile(logits.astype(np.float32), (2, 1))
    p = special.softmax(logits.astype(np.float32).astype(np.float64))
    for x in (3, 2):
        B = N * N
        gam = np.ones(B, np.int32)
        tgt = np.tile(tgt1, (B, 1))
        u0, u1 = np.meshgrid((np.arange(N) + 0.5) / N, (np.arange(N) + 0.5) / N, indexing="ij")
        u = np.stack([u0.ravel(), u1.ravel()], axis=1).astype(np.float32).ravel()
        res = oracle_lib.verify_onehot(B, W.cu_from_gammas(gam), tgt,
                                       np.full(B, x, np.int32), u, 1.0)
        first = res.out_tokens.reshape(B, 2)[:, 0]
        freq = np.bincount(first, minlength=5) / B
        np.testing.assert_allclose(freq, p, atol=4.0 / N, err_msg=f"x={x}")


def test_point_draft_edge_cases(oracle_lib):
    tgt = np.zeros((3, 6), np.float32)
    u = np.asarray([0.0, 0.2, 0.5], np.float32)
    # u = 0 always accepts a token with p(x) > 0
    res = oracle_lib.verify_onehot(1, W.cu_from_gammas([2]), tgt,
                                   np.asarray([4, 1], np.int32), u, 1.0)
    assert res.num_accepted.tolist() == [1]
    # a draft the target gives probability 0 is never accepted, even at u = 0
    tz = tgt.copy()
    tz[0, 4] = -np.inf
    res = oracle_lib.verify_onehot(1, W.cu_from_gammas([2]), tz,
                                   np.asarray([4, 1], np.int32), u, 1.0)
    assert res.num_accepted.tolist() == [0] and res.out_tokens[0] != 4
    with pytest.raises(ValueError):
        oracle_lib.verify_onehot(1, W.cu_from_gammas([2]), tgt,
                                 np.asarray([6, 1], np.int32), u, 1.0)
    with pytest.raises(ValueError):
        oracle_lib.verify_onehot(1, W.cu_from_gammas([2]), tgt,
                                 np.asarray([0, 1], np.int32), u, 0.0)
