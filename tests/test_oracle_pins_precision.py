"""Pins of the oracle's precision claims against a 60-digit reference.

The pages define p = softmax(l / T), q likewise, and the residual
norm(max(0, p - q)) exactly.  The oracle evaluates them in double with
compensated sums and reports, per final draw, a bound E on the error of every
C_k / S.  These pins check that claim from outside: Python's `decimal`
evaluates the same definitions at 60 significant digits from the exactly
widened logits (an independent evaluation, not the oracle's double
arithmetic), and the oracle must lie within its own bound.  Also pinned:
the compensated normaliser on a row whose tail is far below one ulp of its
top term, the S = 0 fallback (reachable only by rounding), the rule of flag
bit 3, and sum_k min(p_k, q_k) against scipy.
"""
import decimal
from decimal import Decimal

import numpy as np
import pytest
from scipy import special

import workloads as W
from tests.test_oracle_pins import f32, packed, run

CTX = decimal.Context(prec=60)


def exact_softmax(stored, dtype, T):
    """softmax(l / T) of one stored row at 60 digits (-inf logits give 0)."""
    l = W.to_f64(stored, dtype)
    Td = Decimal(f32(T))
    z = [None if not np.isfinite(v) else CTX.divide(Decimal(float(v)), Td) for v in l]
    M = max(v for v in z if v is not None)
    e = [Decimal(0) if v is None else CTX.exp(CTX.subtract(v, M)) for v in z]
    s = sum(e, Decimal(0))
    return [CTX.divide(x, s) for x in e]


def exact_residual_cdf(p, q):
    w = [max(Decimal(0), a - b) for a, b in zip(p, q)]
    C, run_ = [], Decimal(0)
    for x in w:
        run_ += x
        C.append(run_)
    return w, C, run_


def test_compensated_normaliser_keeps_sub_ulp_tail(oracle_lib):
    """One logit 0 and 20000 logits at -38 (T = 1): each tail term is about
    3.1e-17, below half an ulp of the running total 1, so an uncompensated
    left-to-right sum stays exactly 1 while the true normaliser is
    1 + 6.3e-13.  p of the top token must match the 60-digit value to a few
    ulps."""
    V = 20001
    row = np.full(V, -38.0)
    row[0] = 0.0
    stored = W.to_dtype(row, "f32")
    p = oracle_lib.row_softmax(stored, 1.0, "f32")
    ref = exact_softmax(stored, "f32", 1.0)
    for k in (0, 1, V - 1):
        assert abs(Decimal(float(p[k])) - ref[k]) <= Decimal(4 * 2.0 ** -53) * ref[k], k


def _near_identical_case(rng, V, dtype, T, sigma):
    """One rejected position whose draft row differs from the target row by
    noise of `sigma` logits (rounded to the dtype, so most tokens agree
    exactly): the residual is a small difference of near-equal
    distributions."""
    for _ in range(200):
        tgt = W.to_dtype(rng.normal(0.0, 2.0, size=V), dtype)
        dft = W.to_dtype(W.to_f64(tgt, dtype) + rng.normal(0.0, sigma, size=V), dtype)
        p = special.softmax(W.to_f64(tgt, dtype) / f32(T))
        q = special.softmax(W.to_f64(dft, dtype) / f32(T))
        cand = np.nonzero(q > p * (1 + 1e-6))[0]
        if cand.size:
            x = int(cand[np.argmax(q[cand])])
            return tgt, dft, x
    pytest.skip("no token with q > p")


@pytest.mark.parametrize("V,dtype,T,sigma", [
    (3, "f32", 1.0, 1e-6), (8, "f32", 0.3, 1e-5), (64, "f32", 0.05, 1e-4),
    (8, "bf16", 1.0, 2e-3), (64, "bf16", 0.3, 4e-3), (64, "bf16", 0.05, 1e-2),
    (64, "f32", 1.0, 0.5)])
def test_residual_cdf_within_reported_bound(oracle_lib, V, dtype, T, sigma):
    """For every k, |C_k / S (oracle) - C_k / S (60 digits)| <= E, S within
    E S / 2, and the token equals the exact inverse-CDF token whenever u S
    is further than E from every exact boundary."""
    rng = np.random.default_rng(V * 1000 + int(T * 100) + (dtype == "bf16"))
    for trial in range(6):
        tgt, dft, x = _near_identical_case(rng, V, dtype, T, sigma)
        u_final = float(np.float32(rng.integers(0, 1 << 24) * 2.0 ** -24))
        batch = packed([W.to_f64(tgt, dtype), W.to_f64(tgt, dtype)], [W.to_f64(dft, dtype)],
                       [1], [x], [1.0 - 2.0 ** -24, u_final], dtype)
        # re-store the exact rows (packed() rounds float64 lists to the dtype)
        batch["target_logits"][0] = tgt
        batch["target_logits"][1] = tgt
        batch["draft_logits"][0] = dft
        r = run(oracle_lib, batch, T)
        if r.num_accepted[0] != 0:
            continue                           # r rounded above u: no residual
        p = exact_softmax(tgt, dtype, T)
        q = exact_softmax(dft, dtype, T)
        w, C, S = exact_residual_cdf(p, q)
        E = float(r.final_err[0])
        assert S > 0
        S_o = Decimal(float(r.residual_sum[0]))
        assert abs(S_o - S) <= Decimal(E / 2) * S + Decimal(1e-300), (trial, float(S))
        # the oracle's C_k / S, recovered from its token choice, is checked
        # through the decision: the exact token for u * S
        t = CTX.multiply(Decimal(u_final), S)
        k_exact = next(k for k, c in enumerate(C) if c > t)
        lo = C[k_exact - 1] if k_exact else Decimal(0)
        dist = float(min(t - lo, C[k_exact] - t) / S)
        tok = int(r.out_tokens[0])
        if dist > E:
            assert tok == k_exact, (trial, tok, k_exact, dist, E)
        else:
            assert r.flagged[0] & 2
        assert (r.flagged[0] & 8 != 0) == (E > 1e-7)


def test_final_draw_bound_holds_on_every_boundary(oracle_lib):
    """The oracle's own C_k / S (rebuilt from its outputs for u on a grid of
    boundaries: a u just below C_k / S - E keeps token <= k, just above
    C_k / S + E gives token > k) agrees with the 60-digit boundaries."""
    rng = np.random.default_rng(5)
    V, dtype, T = 16, "bf16", 0.2
    tgt, dft, x = _near_identical_case(rng, V, dtype, T, 3e-3)
    p = exact_softmax(tgt, dtype, T)
    q = exact_softmax(dft, dtype, T)
    w, C, S = exact_residual_cdf(p, q)
    base = packed([W.to_f64(tgt, dtype)] * 2, [W.to_f64(dft, dtype)], [1], [x],
                  [1.0 - 2.0 ** -24, 0.5], dtype)
    base["target_logits"][:] = tgt
    base["draft_logits"][0] = dft
    r0 = run(oracle_lib, base, T)
    assert r0.num_accepted[0] == 0
    E = float(r0.final_err[0])
    for k in range(V - 1):
        if w[k] == 0:
            continue
        b = float(C[k] / S)
        for side, want_le in ((-1, True), (1, False)):
            u = b + side * (E + 4e-7)
            if not 0.0 <= u < 1.0:
                continue
            batch = dict(base, uniforms=np.array([1.0 - 2.0 ** -24, u], np.float32))
            tok = int(run(oracle_lib, batch, T).out_tokens[0])
            uf = float(np.float32(u))
            if abs(uf - b) > E:
                assert (tok <= k) == want_le, (k, side, tok)


def test_empty_residual_fallback_by_rounding(oracle_lib):
    """V = 2, f32, T = 1: target (0, -40), draft (0, -40 + 2^-18).  The draft
    token 1 has q / p = e^(2^-18) > 1, so u = 1 - 2^-24 rejects it; its
    excess 1.6e-23 is far below an ulp of the normalisers (1 + 4.2e-18
    rounds to 1), so every computed weight max(0, p - q) is 0.  The oracle
    draws from p instead (flag bit 2), with an unbounded E (bits 1 and 3);
    in exact arithmetic the residual is all on token 0, which is also what
    the fallback draws for any u."""
    tgt = [[0.0, -40.0], [0.0, 0.0]]
    dft = [[0.0, -40.0 + 2.0 ** -18]]
    assert np.float32(dft[0][1]) != np.float32(-40.0)
    for u in (0.0, 0.5, 1.0 - 2.0 ** -24):
        r = run(oracle_lib, packed(tgt, dft, [1], [1], [1.0 - 2.0 ** -24, u]), 1.0)
        assert r.num_accepted[0] == 0
        assert r.residual_sum[0] == 0.0
        assert r.flagged[0] & 4 and r.flagged[0] & 2 and r.flagged[0] & 8
        assert np.isinf(r.final_err[0])
        assert r.out_tokens[0] == 0


def test_bound_flag_rule(oracle_lib):
    """Flag bit 3 is set exactly when E exceeds a tenth of the tie window:
    a residual of ~1e-22 of the mass (p and q agree on tokens 0 and 1 to
    ~1e-22) has E far above it; p = (1/2, 1/2) against q ~ (3/4, 1/4) has E
    at the level of double rounding."""
    r = run(oracle_lib, packed([[0.0, 0.0, -60.0], [0.0, 0.0, 0.0]], [[0.0, 0.0, -50.0]],
                               [1], [2], [0.5, 0.5]), 1.0)
    assert r.num_accepted[0] == 0 and r.final_err[0] > 1e-7 and r.flagged[0] & 8
    r = run(oracle_lib, packed([[0.0, 0.0], [0.0, 0.0]], [[np.log(3.0), 0.0]], [1], [0],
                               [0.99, 0.3]), 1.0)
    assert r.num_accepted[0] == 0
    # q = (e^l, 1) / (e^l + 1) with l = ln 3 rounded to f32: residual q_0 - p_0
    assert abs(r.residual_sum[0] - (special.expit(f32(np.log(3.0))) - 0.5)) < 1e-15
    assert r.final_err[0] < 1e-13 and not (r.flagged[0] & 8)


@pytest.mark.parametrize("dtype,T", [("f32", 1.0), ("bf16", 0.7), ("bf16", 3.0)])
def test_overlap_mass_matches_scipy(oracle_lib, dtype, T):
    """sum_k min(p_k, q_k) (the acceptance rate alpha that fixes the draft
    noise of the heavy-tailed workloads) against scipy softmax."""
    rng = np.random.default_rng(17)
    for V in (2, 100, 5000, 32000):
        tgt = W.to_dtype(rng.normal(0.0, 2.0, size=V), dtype)
        dft = W.to_dtype(W.to_f64(tgt, dtype) + rng.normal(0.0, 1.0, size=V), dtype)
        want = np.minimum(special.softmax(W.to_f64(tgt, dtype) / f32(T)),
                          special.softmax(W.to_f64(dft, dtype) / f32(T))).sum()
        got = oracle_lib.overlap_mass(tgt, dft, T, dtype)
        assert abs(got - want) <= 1e-12 * want, (V, got, want)
