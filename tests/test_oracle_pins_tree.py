"""Pins of the oracle's tree verification (greedy and point-mass candidates):
chain-shaped trees reduce to the (separately pinned) chain verifiers, hand
cases under tests/golden/, numpy argmax along the greedy path, and the
output law p at each depth for point candidates (losslessness)."""
import json
import os

import numpy as np
import pytest
from scipy import special, stats

import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tree_cases.json")


def _rows(rows):
    return np.asarray([[float(v) for v in r] for r in rows], dtype=np.float64)


def _one(case):
    N = len(case["parent"])
    return (np.asarray([0, N], np.int32), np.asarray(case["parent"], np.int32),
            np.asarray([max(t, 0) for t in case["tokens"]], np.int32),
            _rows(case["target"]).astype(np.float32))


def test_tree_golden_cases(oracle_lib):
    spec = json.load(open(GOLDEN))
    assert "3.2" in spec["source"]
    for case in spec["greedy"]:
        cu, par, tok, tgt = _one(case)
        r = oracle_lib.verify_tree_greedy(1, cu, par, tok, tgt)
        assert r.out_tokens.tolist() == case["expect_tokens"], case["name"]
        assert r.out_path.tolist() == case["expect_path"], case["name"]
        assert int(r.num_accepted[0]) == case["expect_accepted"], case["name"]
    for case in spec["point"]:
        cu, par, tok, tgt = _one(case)
        r = oracle_lib.verify_tree_point(1, cu, par, tok, tgt,
                                         np.asarray(case["uniforms"], np.float32), 1.0)
        assert r.out_tokens.tolist() == case["expect_tokens"], case["name"]
        assert r.out_path.tolist() == case["expect_path"], case["name"]
        assert int(r.num_accepted[0]) == case["expect_accepted"], case["name"]
        assert r.flagged[0] == case.get("expect_flagged", 0), case["name"]


def _chain_as_tree(inp):
    """A chain batch (gamma_b drafts) as trees: node n+1 carries draft n and
    hangs under node n; node n's row is the chain's target row n; node n+1's
    uniform is the test of draft n and the root's slot the final draw."""
    B = inp.num_seqs
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(inp.gammas + 1)
    R = int(cu[-1])
    parent = np.empty(R, np.int32)
    tokens = np.zeros(R, np.int32)
    unif = np.empty(R, np.float32)
    for b in range(B):
        g, t0, d0 = int(inp.gammas[b]), int(cu[b]), int(inp.cu_draft[b])
        parent[t0] = -1
        parent[t0 + 1:t0 + g + 1] = np.arange(g)
        tokens[t0 + 1:t0 + g + 1] = inp.draft_tokens[d0:d0 + g]
        unif[t0 + 1:t0 + g + 1] = inp.uniforms[t0:t0 + g]
        unif[t0] = inp.uniforms[t0 + g]
    return cu, parent, tokens, unif


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chain_trees_reduce_to_chain_verifiers(oracle_lib, dtype):
    inp = W.build("chain", 77, [3, 0, 6, 2, 8, 1, 5], 700, dtype, 0.9,
                  W.boosted_top_rows(1.5, 3, 5.0), 0.4)
    inp = W.with_deterministic_drafts(inp)
    cu, parent, tokens, unif = _chain_as_tree(inp)
    # cu_nodes equals the chain's target-row layout (gamma_b + 1 rows each)
    tg = oracle_lib.verify_tree_greedy(inp.num_seqs, cu, parent, tokens, inp.target_logits,
                                       dtype=dtype)
    cg = oracle_lib.verify_greedy(inp.num_seqs, inp.cu_draft, inp.target_logits,
                                  inp.draft_tokens, dtype=dtype)
    np.testing.assert_array_equal(tg.out_tokens, cg.out_tokens)
    np.testing.assert_array_equal(tg.num_accepted, cg.num_accepted)
    tp = oracle_lib.verify_tree_point(inp.num_seqs, cu, parent, tokens, inp.target_logits, unif,
                                      inp.temperature, dtype=dtype)
    cp = oracle_lib.verify_onehot(inp.num_seqs, inp.cu_draft, inp.target_logits,
                                  inp.draft_tokens, inp.uniforms, inp.temperature, dtype=dtype)
    np.testing.assert_array_equal(tp.out_tokens, cp.out_tokens)
    np.testing.assert_array_equal(tp.num_accepted, cp.num_accepted)
    np.testing.assert_array_equal(tp.flagged != 0, cp.flagged != 0)
    assert 0 < tp.num_accepted.sum() and (tg.num_accepted > 0).any()


def test_greedy_path_follows_numpy_argmax(oracle_lib):
    tr = W.build_tree("t", 5, [W.tree_shape(W.TREE_17)] * 12 + [W.tree_shape([(1, 3)])] * 3 +
                      [np.asarray([-1], np.int32)], 900, "bf16", 1.0,
                      W.boosted_top_rows(1.0, 2, 6.0), 0.3)
    r = oracle_lib.verify_tree_greedy(tr.num_seqs, tr.cu_nodes, tr.parent, tr.tokens,
                                      tr.target_logits, dtype="bf16")
    vals = W.to_f64(tr.target_logits, "bf16")
    deep = 0
    for b in range(tr.num_seqs):
        g0, N = int(tr.cu_nodes[b]), int(tr.cu_nodes[b + 1] - tr.cu_nodes[b])
        n = int(r.num_accepted[b])
        cur = 0
        for i in range(n):
            nxt = int(r.out_path[g0 + i])
            a = int(np.argmax(vals[g0 + cur]))
            assert tr.parent[g0 + nxt] == cur and tr.tokens[g0 + nxt] == a
            assert r.out_tokens[g0 + i] == a
            cur = nxt
        a = int(np.argmax(vals[g0 + cur]))
        assert r.out_tokens[g0 + n] == a
        kids = [m for m in range(N) if tr.parent[g0 + m] == cur]
        assert all(tr.tokens[g0 + m] != a for m in kids)
        assert (r.out_tokens[g0 + n + 1:g0 + N] == -1).all()
        deep = max(deep, n)
    assert deep >= 2


def test_point_tree_output_law(oracle_lib):
    """10^6 trials of one root with three candidates (one repeated) whose
    nodes have their own children: the token emitted at depth 0 follows
    p_root, and among trials that accepted node c the next token follows
    p_c (chi-square, Bonferroni)."""
    rng = np.random.default_rng(31)
    V, N = 6, 200_000
    rows = (rng.standard_normal((6, V)) * 1.1).astype(np.float32)
    parent = np.asarray([-1, 0, 0, 0, 0, 1, 2], np.int32)
    tokens = np.asarray([0, 2, 4, 2, 1, 3, 5], np.int32)
    rows = np.vstack([rows, rows[:1]])          # 7 nodes
    p = [special.softmax(r.astype(np.float64)) for r in rows]
    tr_cu = np.arange(0, 7 * N + 1, 7, dtype=np.int32)
    res = oracle_lib.verify_tree_point(N, tr_cu, np.tile(parent, N), np.tile(tokens, N),
                                       np.tile(rows, (N, 1)), W.uniform_grid24(rng, 7 * N), 1.0)
    out = res.out_tokens.reshape(N, 7)
    path = res.out_path.reshape(N, 7)
    level = 1e-3 / 5
    c0 = np.bincount(out[:, 0], minlength=V)
    assert stats.chisquare(c0, N * p[0]).pvalue > level
    for node in (1, 2, 4):
        m = path[:, 0] == node
        c1 = np.bincount(out[m, 1], minlength=V)
        assert stats.chisquare(c1, m.sum() * p[node]).pvalue > level, node
    assert not (path[:, 0] == 3).any()           # the repeated token is never accepted
    assert (res.flagged & 4 == 0).all()


def test_tree_argument_errors(oracle_lib):
    tgt = np.zeros((3, 4), np.float32)
    cu = np.asarray([0, 3], np.int32)
    with pytest.raises(ValueError):              # parent not before the child
        oracle_lib.verify_tree_greedy(1, cu, np.asarray([-1, 2, 0], np.int32),
                                      np.asarray([0, 1, 1], np.int32), tgt)
    with pytest.raises(ValueError):              # token out of range
        oracle_lib.verify_tree_point(1, cu, np.asarray([-1, 0, 0], np.int32),
                                     np.asarray([0, 1, 4], np.int32), tgt,
                                     np.zeros(3, np.float32), 1.0)
    with pytest.raises(ValueError):              # empty tree
        oracle_lib.verify_tree_greedy(1, np.asarray([0, 0], np.int32), np.zeros(0, np.int32),
                                      np.zeros(0, np.int32), tgt[:0])
