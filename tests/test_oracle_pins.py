"""Pins of the float64 oracle against what the pages and the mathematics fix.

Nothing here re-types the oracle's procedure.  Each test checks the oracle as
a black box against one of:
  * a library routine (scipy softmax / expit, numpy searchsorted) on a special
    case that reduces to it;
  * a closed form (the truncated-geometric law of the accepted count, the
    expected emitted length (1 - a^(g+1)) / (1 - a) with the page's printed
    example, Σ max(0, p - q) = 1 - Σ min(p, q));
  * the pages' invariants: identical draft and target rows accept every draft,
    a one-hot target with the argmax as draft accepts every draft, and the
    output law equals the target's (losslessness);
  * hand-worked cases stored under tests/golden/;
  * deterministic quadrature and an exact enumeration over the 24-bit uniform
    grid that recovers the oracle's decision thresholds by bisection.
"""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def f32(x):
    return float(np.float32(x))


def softmax64(stored, dtype, T):
    return special.softmax(W.to_f64(stored, dtype) / f32(T))


def packed(target_rows, draft_rows, gammas, tokens, uniforms, dtype="f32"):
    """Host arrays of one packed batch from python lists of float64 rows."""
    V = len(target_rows[0])
    tgt = W.to_dtype(np.asarray(target_rows, dtype=np.float64), dtype)
    if len(draft_rows):
        dft = W.to_dtype(np.asarray(draft_rows, dtype=np.float64), dtype)
    else:
        dft = np.zeros((0, V), dtype=tgt.dtype)
    return dict(num_seqs=len(gammas), cu_draft=W.cu_from_gammas(gammas),
                target_logits=tgt, draft_logits=dft,
                draft_tokens=np.asarray(tokens, dtype=np.int32),
                uniforms=np.asarray(uniforms, dtype=np.float32))


def run(oracle_lib, batch, T, **kw):
    return oracle_lib.verify(batch["num_seqs"], batch["cu_draft"],
                             batch["target_logits"], batch["draft_logits"],
                             batch["draft_tokens"], batch["uniforms"], f32(T),
                             **kw)


# ------------------------------------------------------------ normalisers

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.7, 0.8, 1.0, 1.3])
def test_row_softmax_matches_scipy(oracle_lib, dtype, T):
    rng = np.random.default_rng(11)
    for V in (1, 2, 5, 8, 63, 1000, 32000):
        stored = W.to_dtype(rng.standard_normal(V) * 3.0, dtype)
        p = oracle_lib.row_softmax(stored, f32(T), dtype)
        np.testing.assert_allclose(p, softmax64(stored, dtype, T), rtol=1e-12,
                                   atol=0)


def test_row_softmax_closed_forms(oracle_lib):
    # V = 1: the single token has probability exactly 1.
    assert oracle_lib.row_softmax(np.array([3.5], np.float32), 1.0)[0] == 1.0
    # V = 2: p_0 is the logistic function of (l_0 - l_1) / T.
    for l0, l1, T in [(0.3, -1.2, 1.0), (4.0, 4.5, 0.7), (-2.0, 3.0, 1.3)]:
        row = np.array([l0, l1], np.float32)
        p = oracle_lib.row_softmax(row, f32(T))
        want = special.expit((float(row[0]) - float(row[1])) / f32(T))
        assert abs(p[0] - want) < 1e-15 and abs(p[1] - (1 - want)) < 1e-15
    # -inf logits get exactly zero mass; the rest renormalises.
    row = np.array([0.0, -np.inf, np.log(3.0), -np.inf], np.float32)
    p = oracle_lib.row_softmax(row, 1.0)
    assert p[1] == 0.0 and p[3] == 0.0
    assert abs(p[2] / p[0] - 3.0) < 1e-6


def test_p_q_at_draft_tokens_match_scipy(oracle_lib):
    inp = W.config(2, seed=21, num_seqs=4, vocab=3000)
    r = oracle_lib.verify_inputs(inp)
    for b in range(inp.num_seqs):
        for i in range(int(inp.gammas[b])):
            x = inp.draft_tokens[inp.draft_row(b, i)]
            p = softmax64(inp.target_logits[inp.target_row(b, i)], "bf16",
                          inp.temperature)[x]
            q = softmax64(inp.draft_logits[inp.draft_row(b, i)], "bf16",
                          inp.temperature)[x]
            assert abs(r.p_draft[inp.draft_row(b, i)] / p - 1) < 1e-12
            assert abs(r.q_draft[inp.draft_row(b, i)] / q - 1) < 1e-12


# ------------------------------------------------------------ invariants (i), (ii)

@pytest.mark.parametrize("seed", [0, 1, 2])
def test_identical_rows_accept_every_draft(oracle_lib, seed):
    """p == q bitwise: r = 1 > u for every u in [0, 1), so all gamma drafts
    are accepted and the bonus is a plain inverse-CDF draw from p_gamma."""
    rng = np.random.default_rng(seed)
    gammas = [0, 1, 3, 8, 2, 5]
    inp = W.build("identical", 100 + seed, gammas, 257, W.BF16, 0.8,
                  W.iid_normal_rows(2.0), 0.0, draft_copy=lambda b: True)
    u = inp.uniforms.copy()
    u[rng.integers(0, u.shape[0], 6)] = np.float32(1 - 2 ** -24)
    u[rng.integers(0, u.shape[0], 6)] = np.float32(0.0)
    r = oracle_lib.verify(inp.num_seqs, inp.cu_draft, inp.target_logits,
                          inp.draft_logits, inp.draft_tokens, u,
                          inp.temperature)
    np.testing.assert_array_equal(r.num_accepted, inp.gammas)
    assert (r.residual_sum == 0).all()
    for b in range(inp.num_seqs):
        g = int(inp.gammas[b])
        emitted = r.emitted(b, inp.cu_draft)
        np.testing.assert_array_equal(
            emitted[:g], inp.draft_tokens[inp.draft_row(b, 0):inp.draft_row(b, 0) + g])
        if r.flagged[b] & 2:
            continue
        p = softmax64(inp.target_logits[inp.target_row(b, g)], "bf16",
                      inp.temperature)
        want = np.searchsorted(np.cumsum(p), u[inp.target_row(b, g)], "right")
        assert emitted[g] == want


@pytest.mark.parametrize("neg", [-np.inf, -1.0e4])
def test_one_hot_target_accepts_its_argmax(oracle_lib, neg):
    """p one-hot at a_i and x_i = a_i: r = 1 / q(a_i) >= 1, so every draft is
    accepted and the bonus is the one-hot token of the last target row."""
    rng = np.random.default_rng(5)
    V = 50
    gammas = [0, 2, 6, 1]
    cu = W.cu_from_gammas(gammas)
    R_d = int(cu[-1])
    R_t = R_d + len(gammas)
    hot = rng.integers(0, V, R_t)
    tgt = np.full((R_t, V), neg)
    tgt[np.arange(R_t), hot] = rng.standard_normal(R_t)
    dft = rng.standard_normal((R_d, V)) * 2.0
    tokens = np.empty(R_d, np.int32)
    for b, g in enumerate(gammas):
        for i in range(g):
            tokens[cu[b] + i] = hot[cu[b] + b + i]
    u = W.uniform_grid24(rng, R_t)
    u[::3] = np.float32(1 - 2 ** -24)
    r = run(oracle_lib, packed(tgt, dft, gammas, tokens, u), 1.0)
    np.testing.assert_array_equal(r.num_accepted, gammas)
    for b, g in enumerate(gammas):
        np.testing.assert_array_equal(r.emitted(b, cu),
                                      hot[cu[b] + b:cu[b] + b + g + 1])


# ------------------------------------------------------------ hand cases

def test_golden_hand_cases(oracle_lib):
    spec = json.load(open(os.path.join(GOLDEN, "hand_cases.json")))
    for case in spec["cases"]:
        conv = lambda rows: [[float(v) for v in row] for row in rows]
        batch = packed(conv(case["target"]), conv(case["draft"]),
                       case["gammas"], case["tokens"], case["uniforms"])
        r = run(oracle_lib, batch, case["T"])
        assert r.out_tokens.tolist() == case["expect_tokens"], case["name"]
        assert r.num_accepted.tolist() == case["expect_accepted"], case["name"]
        want_flags = case.get("expect_flagged", [0] * len(case["gammas"]))
        assert r.flagged.tolist() == want_flags, case["name"]


def test_zero_weight_token_never_drawn(oracle_lib):
    """The smallest k with C_k > t: with w_0 = 0 and u = 0 the draw must skip
    token 0 (a >= comparison would return it)."""
    batch = packed([[-np.inf, 0.0, 0.0]], [], [0], [], [0.0])
    assert run(oracle_lib, batch, 1.0).out_tokens.tolist() == [1]
    batch = packed([[0.0, -np.inf, 0.0, -np.inf]], [], [0], [],
                   [np.float32(1 - 2 ** -24)])
    assert run(oracle_lib, batch, 1.0).out_tokens.tolist() == [2]


# ------------------------------------------------------------ library special cases

@pytest.mark.parametrize("dtype,T", [("f32", 1.0), ("bf16", 0.7), ("bf16", 1.3)])
def test_gamma_zero_is_textbook_inverse_cdf(oracle_lib, dtype, T):
    """gamma = 0 (plain decode): the output is searchsorted(cumsum(p), u)."""
    rng = np.random.default_rng(7)
    B, V = 400, 1000
    tgt = rng.standard_normal((B, V)) * 2.5
    u = W.uniform_grid24(rng, B)
    batch = packed(tgt, [], [0] * B, [], u, dtype)
    r = run(oracle_lib, batch, T)
    checked = 0
    for b in range(B):
        if r.flagged[b]:
            continue
        p = softmax64(batch["target_logits"][b], dtype, T)
        assert r.out_tokens[b] == np.searchsorted(np.cumsum(p), u[b], "right")
        checked += 1
    assert checked > 0.9 * B


def test_one_hot_draft_reduces_to_bernoulli_and_renormalised_p(oracle_lib):
    """q one-hot at x (a deterministic draft): r = p(x), so the draft passes
    iff u < p(x); a rejection draws from p with x removed, renormalised."""
    rng = np.random.default_rng(9)
    B, V = 300, 40
    tgt = rng.standard_normal((B, V)) * 1.5
    x = rng.integers(0, V, B)
    dft = np.full((B, V), -np.inf)
    dft[np.arange(B), x] = 0.0
    u = W.uniform_grid24(rng, 2 * B)
    tgt2 = np.concatenate([np.stack([tgt[b], tgt[(b + 1) % B]]) for b in range(B)])
    batch = packed(tgt2, dft, [1] * B, x, u)
    r = run(oracle_lib, batch, 1.0)
    for b in range(B):
        p = softmax64(batch["target_logits"][2 * b], "f32", 1.0)
        if abs(u[2 * b] - p[x[b]]) < 1e-9:
            continue
        accepted = bool(u[2 * b] < p[x[b]])
        assert r.num_accepted[b] == int(accepted)
        if not accepted and not r.flagged[b]:
            w = p.copy()
            w[x[b]] = 0.0
            want = np.searchsorted(np.cumsum(w), u[2 * b + 1] * w.sum(), "right")
            assert r.out_tokens[2 * b] == want


def test_residual_sum_is_total_variation(oracle_lib):
    """Σ_k max(0, p_k - q_k) = 1 - Σ_k min(p_k, q_k) for normalised p, q."""
    inp = W.config(2, seed=33, num_seqs=16, vocab=4000)
    r = oracle_lib.verify_inputs(inp)
    seen = 0
    for b in range(inp.num_seqs):
        j = int(r.num_accepted[b])
        if j == inp.gammas[b]:
            assert r.residual_sum[b] == 0.0
            continue
        p = softmax64(inp.target_logits[inp.target_row(b, j)], "bf16", inp.temperature)
        q = softmax64(inp.draft_logits[inp.draft_row(b, j)], "bf16", inp.temperature)
        assert abs(r.residual_sum[b] - (1.0 - np.minimum(p, q).sum())) < 1e-12
        seen += 1
    assert seen > 0


# ------------------------------------------------------------ statistics (iii), (iv)

def _replicate(oracle_lib, tgt_rows, dft_rows, N, seed, T=1.0):
    """N independent trials of one sequence whose target rows are tgt_rows
    (gamma+1 of them) and draft rows dft_rows, with draft tokens drawn from
    the draft distributions by numpy and fresh uniforms per trial."""
    rng = np.random.default_rng(seed)
    g = len(dft_rows)
    tgt = W.to_dtype(np.asarray(tgt_rows, np.float64), "f32")
    dft = W.to_dtype(np.asarray(dft_rows, np.float64), "f32") if g else \
        np.zeros((0, tgt.shape[1]), np.float32)
    V = tgt.shape[1]
    q = [softmax64(dft[i], "f32", T) for i in range(g)]
    tokens = np.empty((N, g), np.int32)
    for i in range(g):
        tokens[:, i] = rng.choice(V, size=N, p=q[i])
    u = W.uniform_grid24(rng, N * (g + 1))
    r = oracle_lib.verify(N, W.cu_from_gammas([g] * N),
                          np.tile(tgt, (N, 1)), np.tile(dft, (N, 1)),
                          tokens.reshape(-1), u, f32(T))
    return tgt, dft, r.out_tokens.reshape(N, g + 1), r.num_accepted


@pytest.mark.slow
def test_lossless_chi_square(oracle_lib):
    """Losslessness: among trials that reach position i, the token emitted
    there follows p_i (1e6 trials, V = 6, gamma = 3, Bonferroni over the
    positions); the pass rate at each position is sum_k min(p_i, q_i)."""
    rng = np.random.default_rng(2024)
    V, g, N = 6, 3, 1_000_000
    tgt_rows = rng.standard_normal((g + 1, V)) * 1.0
    dft_rows = tgt_rows[:g] + rng.standard_normal((g, V)) * 0.9
    tgt, dft, out, n = _replicate(oracle_lib, tgt_rows, dft_rows, N, 77)
    alpha_level = 1e-3 / (2 * g + 1)
    for i in range(g + 1):
        p = softmax64(tgt[i], "f32", 1.0)
        mask = n >= i
        counts = np.bincount(out[mask, i], minlength=V)
        assert counts.sum() == mask.sum()
        res = stats.chisquare(counts, mask.sum() * p)
        assert res.pvalue > alpha_level, (i, counts, mask.sum() * p)
        if i < g:
            a = np.minimum(p, softmax64(dft[i], "f32", 1.0)).sum()
            reached, passed = mask.sum(), (n >= i + 1).sum()
            z = (passed - reached * a) / np.sqrt(reached * a * (1 - a))
            assert abs(z) < stats.norm.isf(alpha_level / 2), (i, z)


def _geometric_case(oracle_lib, tgt_rows, dft_rows, g, N, seed):
    tgt, dft, out, n = _replicate(oracle_lib, tgt_rows, dft_rows, N, seed)
    alphas = [np.minimum(softmax64(tgt[i], "f32", 1.0),
                         softmax64(dft[i], "f32", 1.0)).sum() for i in range(g)]
    a = float(np.mean(alphas))
    assert max(alphas) - min(alphas) < 1e-6
    # P(n = k) = a^k (1 - a) for k < g, a^g for k = g.
    probs = np.array([a ** k * (1 - a) for k in range(g)] + [a ** g])
    counts = np.bincount(n, minlength=g + 1)
    assert stats.chisquare(counts, N * probs).pvalue > 1e-4
    emitted = n + 1.0
    want = (1 - a ** (g + 1)) / (1 - a)
    se = emitted.std() / np.sqrt(N)
    assert abs(emitted.mean() - want) < 4 * se, (emitted.mean(), want, se)
    return a, want


@pytest.mark.slow
def test_expected_emitted_length_page_example(oracle_lib):
    """(1 - a^(k+1)) / (1 - a) at the page's printed example a = 0.8, k = 5."""
    ex = json.load(open(os.path.join(GOLDEN, "expected_length_example.json")))
    a0, k = ex["alpha"], ex["k"]
    assert abs((1 - a0 ** (k + 1)) / (1 - a0) - ex["formula_value"]) < 1e-12
    assert round((1 - a0 ** (k + 1)) / (1 - a0)) in (ex["page_rounded_value"],
                                                      ex["page_rounded_value"] + 1)
    # V = 2: p = (0.9, 0.1), q = (0.7, 0.3) gives min-overlap 0.7 + 0.1 = 0.8
    # at every position.
    tgt = [np.log([0.9, 0.1])] * (k + 1)
    dft = [np.log([0.7, 0.3])] * k
    a, want = _geometric_case(oracle_lib, tgt, dft, k, 1_000_000, 5)
    assert abs(a - a0) < 1e-6
    assert abs(want - ex["formula_value"]) < 1e-4


@pytest.mark.slow
def test_expected_emitted_length_disjoint_support(oracle_lib):
    """a = 0.6, gamma = 8, V = 16: p lives on 8 ids (others -inf), q = a p +
    (1 - a) nu with nu on the other 8 ids, so Σ min(p, q) = a exactly; the
    ids are permuted differently at every position."""
    rng = np.random.default_rng(31)
    V, g, a = 16, 8, 0.6
    tgt_rows, dft_rows = [], []
    for i in range(g + 1):
        perm = rng.permutation(V)
        p = np.zeros(V)
        p[perm[:8]] = rng.dirichlet(np.ones(8) * 3)
        nu = np.zeros(V)
        nu[perm[8:]] = rng.dirichlet(np.ones(8) * 3)
        with np.errstate(divide="ignore"):
            tgt_rows.append(np.log(p))
            if i < g:
                dft_rows.append(np.log(a * p + (1 - a) * nu))
    got_a, _ = _geometric_case(oracle_lib, tgt_rows, dft_rows, g, 1_000_000, 6)
    assert abs(got_a - a) < 1e-6


# ------------------------------------------------------------ quadrature

def test_midpoint_quadrature_first_token_law(oracle_lib):
    """gamma = 1, V = 3: integrate the oracle over a 1000 x 1000 midpoint grid
    of (u_0, u_final) for every draft token x (weight q(x)).  The first
    emitted token must follow p_1, the accepted-and-x event must have mass
    min(p_1(x), q_1(x)), and the bonus must follow p_2."""
    G = 1000
    grid = ((np.arange(G) + 0.5) / G).astype(np.float32)
    l_p1 = np.array([0.4, -0.3, 1.1])
    l_q1 = np.array([-0.2, 0.7, 0.9])
    l_p2 = np.array([1.0, -1.0, 0.2])
    p1 = softmax64(W.to_dtype(l_p1, "f32"), "f32", 1.0)
    q1 = softmax64(W.to_dtype(l_q1, "f32"), "f32", 1.0)
    p2 = softmax64(W.to_dtype(l_p2, "f32"), "f32", 1.0)
    N = G * G
    u = np.empty((N, 2), np.float32)
    u[:, 0] = np.repeat(grid, G)
    u[:, 1] = np.tile(grid, G)
    law0 = np.zeros(3)
    acc = np.zeros(3)
    bonus = np.zeros(3)
    for x in range(3):
        batch = packed(np.tile(np.stack([l_p1, l_p2]), (N, 1)),
                       np.tile(l_q1[None, :], (N, 1)), [1] * N,
                       np.full(N, x), u.reshape(-1))
        r = run(oracle_lib, batch, 1.0)
        out = r.out_tokens.reshape(N, 2)
        law0 += q1[x] * np.bincount(out[:, 0], minlength=3) / N
        accepted = r.num_accepted == 1
        acc[x] += q1[x] * accepted.mean()
        bonus += q1[x] * np.bincount(out[accepted, 1], minlength=3) / N
    tol = 3.0 / G
    np.testing.assert_allclose(law0, p1, atol=tol)
    np.testing.assert_allclose(acc, np.minimum(p1, q1), atol=tol)
    np.testing.assert_allclose(bonus / bonus.sum(), p2, atol=tol)


# ------------------------------------------------------------ exact enumeration

class _Seq:
    """One gamma = 2 sequence evaluated by the oracle at chosen uniforms."""

    def __init__(self, oracle_lib, tgt, dft, tokens):
        self.o = oracle_lib
        self.batch = packed(tgt, dft, [2], tokens, [0.0, 0.0, 0.0])

    def __call__(self, u):
        self.batch["uniforms"] = np.asarray(u, np.float32)
        r = run(self.o, self.batch, 1.0)
        return int(r.num_accepted[0]), r.out_tokens.tolist()


def _first_true(pred, lo=0, hi=1 << 24):
    """Smallest m in [lo, hi] with pred(m) true; pred is monotone in m."""
    while lo < hi:
        mid = (lo + hi) // 2
        if pred(mid):
            hi = mid
        else:
            lo = mid + 1
    return lo


def _grid(m):
    return float(m) * 2.0 ** -24


def test_exact_enumeration_output_law(oracle_lib):
    """V = 3, gamma = 2: enumerate every draft pair (weight q_0 q_1), recover
    the oracle's accept thresholds and inverse-CDF boundaries on the 24-bit
    uniform grid by bisection, and integrate exactly.  The token emitted at
    each position, given that position is reached, must follow that
    position's target distribution to grid accuracy."""
    V = 3
    rng = np.random.default_rng(3)
    tgt = rng.standard_normal((3, V))
    dft = tgt[:2] + rng.standard_normal((2, V)) * 1.2
    p = [softmax64(W.to_dtype(t, "f32"), "f32", 1.0) for t in tgt]
    q = [softmax64(W.to_dtype(d, "f32"), "f32", 1.0) for d in dft]
    ONE = (1 << 24) - 1
    law = [np.zeros(V) for _ in range(3)]
    reach = np.zeros(3)

    def draw_law(seq, u_prefix, pos):
        # token at position pos as a function of the final uniform
        k_of = lambda m: seq(u_prefix + [_grid(m)])[1][pos]
        bounds = [0] + [_first_true(lambda m, k=k: k_of(m) >= k, 0, ONE + 1)
                        for k in range(1, V)] + [ONE + 1]
        return np.diff(bounds) / float(1 << 24)

    for x0 in range(V):
        for x1 in range(V):
            w = q[0][x0] * q[1][x1]
            seq = _Seq(oracle_lib, tgt, dft, [x0, x1])
            # accept probability of draft 0: smallest m rejecting at 0
            a0 = _first_true(lambda m: seq([_grid(m), 0.0, 0.0])[0] == 0, 0, ONE + 1)
            a0 /= float(1 << 24)
            reach[0] += w
            law[0][x0] += w * a0
            if a0 < 1.0:
                law[0] += w * (1 - a0) * draw_law(seq, [_grid(ONE), 0.0], 0)
            if a0 == 0.0:
                continue
            a1 = _first_true(lambda m: seq([0.0, _grid(m), 0.0])[0] == 1, 0, ONE + 1)
            a1 /= float(1 << 24)
            reach[1] += w * a0
            law[1][x1] += w * a0 * a1
            if a1 < 1.0:
                law[1] += w * a0 * (1 - a1) * draw_law(seq, [0.0, _grid(ONE)], 1)
            if a1 > 0.0:
                reach[2] += w * a0 * a1
                law[2] += w * a0 * a1 * draw_law(seq, [0.0, 0.0], 2)
    for i in range(3):
        np.testing.assert_allclose(law[i] / reach[i], p[i], atol=1e-6)
    assert abs(reach[1] - np.minimum(p[0], q[0]).sum()) < 1e-6
    assert abs(reach[2] / reach[1] - np.minimum(p[1], q[1]).sum()) < 1e-6


# ------------------------------------------------------------ edge cases and flags

def test_edge_cases(oracle_lib):
    # B = 0 is a no-op.
    r = oracle_lib.verify(0, np.zeros(1, np.int32), np.zeros((0, 4), np.float32),
                          np.zeros((0, 4), np.float32), np.zeros(0, np.int32),
                          np.zeros(0, np.float32), 1.0, vocab=4)
    assert r.out_tokens.size == 0
    # V = 1: p = q = 1, every draft (token 0) accepted, bonus token 0.
    batch = packed([[0.5]] * 4, [[2.0]] * 3, [3], [0, 0, 0], [0.9, 0.99, 0.5, 0.7])
    r = run(oracle_lib, batch, 1.0)
    assert r.out_tokens.tolist() == [0, 0, 0, 0] and r.num_accepted.tolist() == [3]
    # invalid arguments are rejected
    with pytest.raises(ValueError):
        run(oracle_lib, batch, 0.0)
    bad = dict(batch, draft_tokens=np.array([0, 5, 0], np.int32))
    with pytest.raises(ValueError):
        run(oracle_lib, bad, 1.0)


def test_tie_flags(oracle_lib):
    """A uniform within 1e-6 of r sets flag bit 0; far from it, no flag."""
    tgt = [[0.0, 0.0], [0.0, 0.0]]
    dft = [[np.log(3.0), 0.0]]
    p = softmax64(W.to_dtype(np.array(tgt[0]), "f32"), "f32", 1.0)
    q = softmax64(W.to_dtype(np.array(dft[0]), "f32"), "f32", 1.0)
    r0 = p[0] / q[0]               # about 2/3
    for du, flagged in [(3e-7, 1), (-3e-7, 1), (1e-3, 0), (-1e-3, 0)]:
        u = np.float32(r0 + du)
        r = run(oracle_lib, packed(tgt, dft, [1], [0], [u, 0.3]), 1.0)
        assert (r.flagged[0] & 1) == flagged, du
        assert r.num_accepted[0] == int(float(u) < r0)
        assert abs(r.tie_accept[0] - abs(float(u) - r0)) < 1e-12
    # final draw on a CDF boundary: uniform p = (1/2, 1/2), u = 0.5
    r = run(oracle_lib, packed([[0.0, 0.0]], [], [0], [], [0.5]), 1.0)
    assert r.flagged[0] & 2
