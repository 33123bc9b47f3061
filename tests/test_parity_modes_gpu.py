"""Parity of greedy verification and point-mass-draft verification (through
the C ABI) with the float64 oracle.

Greedy verification is integer work and must match bit for bit.  Point-mass
drafts follow the sampled verify's parity rule (exact tokens and counts
outside flagged 1e-6 ties; probabilities within 1e-5 / 2e-3 relative for
f32 / bf16).  Every case prints its name before touching the GPU.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import (compare, compare_greedy, log, make_verifier, oracle_greedy, ties,
                               oracle_point, run_gpu, to_device)

torch = pytest.importorskip("torch")
pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _greedy(inp, label, **kw):
    log(f"[case] greedy {label}: B={inp.num_seqs} R_t={inp.target_rows} V={inp.vocab} {inp.dtype}")
    gpu = run_gpu(inp, mode="greedy", **kw)
    compare_greedy(inp, gpu, oracle_greedy(inp), label=f"greedy {label}")
    assert gpu.status == 0, f"{label}: status {gpu.status:#x}"
    return gpu


def _point(inp, label, **kw):
    log(f"[case] point {label}: B={inp.num_seqs} R_t={inp.target_rows} V={inp.vocab} "
        f"{inp.dtype} T={inp.temperature}")
    ora = oracle_point(inp)
    gpu = run_gpu(inp, mode="point", **kw)
    rep = compare(inp, gpu, ora, label=f"point {label}", point=True)
    assert gpu.status == 0, f"{label}: status {gpu.status:#x}"
    assert (gpu.q_draft == 1.0).all()
    return rep


def _argmax_drafts(inp, rng, match):
    """Test-side inputs: each draft token is its target row's first maximum
    with probability `match`, else a random other token (numpy argmax)."""
    tok = inp.draft_tokens.copy()
    for b in range(inp.num_seqs):
        for i in range(int(inp.gammas[b])):
            row = W.to_f64(inp.target_logits[inp.target_row(b, i)], inp.dtype)
            a = int(np.argmax(row))
            tok[inp.draft_row(b, i)] = a if rng.random() < match else \
                (a + 1 + int(rng.integers(0, inp.vocab - 1))) % inp.vocab if inp.vocab > 1 else 0
    import dataclasses
    return dataclasses.replace(inp, draft_tokens=tok)


# ------------------------------------------------------------ greedy

@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_greedy_named_workload_full_size(idx):
    inp = W.with_deterministic_drafts(W.config(idx))
    _greedy(inp, f"workload {idx} ({inp.name})")


@pytest.mark.parametrize("V", [1, 5, 8, 63, 1000, 4097, 32000, 128256, 152064])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_greedy_vocab_sizes_with_ties(V, dtype):
    """A narrow logit range makes tied maxima common in bf16; most drafts are
    the target argmax so prefixes run long."""
    rng = np.random.default_rng(V)
    inp = W.build(f"gV{V}", 8000 + V, [0, 1, 4, 8, 3, 6], V, dtype, 1.0,
                  W.iid_normal_rows(0.3), 0.5)
    inp = _argmax_drafts(inp, rng, 0.8)
    _greedy(inp, f"V={V} {dtype}")


def test_greedy_planted_ties_and_neg_inf():
    rng = np.random.default_rng(4)
    V = 9000
    inp = W.build("gties", 44, [3, 0, 5, 2, 7], V, W.BF16, 1.0, W.iid_normal_rows(1.0), 0.5)
    t = inp.target_logits
    hi = W.round_to_bf16_bits(np.asarray([20.0]))[0]
    neg = np.uint16(0xFF80)
    t[0, [4096, 100, 8999]] = hi           # lowest id is 100, across wave tasks
    t[1, :] = neg                          # all -inf: argmax 0
    t[2, :4096] = neg
    t[2, [4096 + 7, V - 1]] = hi
    t[3, [V - 1]] = hi                     # in the ragged last group
    t[4, 2048:6144] = neg
    inp = _argmax_drafts(inp, rng, 1.0)
    gpu = _greedy(inp, "planted ties, -inf rows")
    ora = oracle_greedy(inp)
    assert ora.argmax[0] == 100 and ora.argmax[1] == 0 and ora.argmax[2] == 4096 + 7
    assert (gpu.num_accepted == inp.gammas).all()


def test_greedy_long_drafts():
    rng = np.random.default_rng(9)
    gam = [70, 0, 3, 65, 64, 0, 1, 63, 128]
    inp = W.build("glong", 91, gam, 2000, W.BF16, 1.0, W.iid_normal_rows(1.0), 0.05)
    _greedy(_argmax_drafts(inp, rng, 1.0), "gamma up to 128, all match")
    _greedy(_argmax_drafts(inp, rng, 0.98), "gamma up to 128, 98% match")


@pytest.mark.parametrize("ld_extra,offset", [(8, 0), (1, 0), (0, 1), (3, 5)])
def test_greedy_row_pitch_and_alignment(ld_extra, offset):
    rng = np.random.default_rng(12)
    inp = W.build("gpitch", 12, [2, 5, 0, 3], 4003, W.BF16, 1.0, W.iid_normal_rows(0.3), 1.0)
    inp = _argmax_drafts(inp, rng, 0.8)
    _greedy(inp, f"ld=V+{ld_extra} offset={offset}", ld=inp.vocab + ld_extra, offset=offset)


def test_greedy_bad_tokens_and_offsets():
    inp = W.with_deterministic_drafts(W.config(2, seed=4, num_seqs=6, vocab=3000))
    d = to_device(inp)
    sv = make_verifier(inp, check=True)
    d.tokens[3] = 5000
    d.target[inp.target_row(3, 0), 17] = float("nan")
    out = sv.greedy(d.cu, d.target, d.tokens)
    torch.cuda.synchronize()
    st = int(out.status.item()) & 0xFFFFFFFF
    assert st & 2 and st & 8, hex(st)
    toks = out.out_tokens.cpu().numpy()
    assert (toks[inp.target_row(0, 0):inp.target_row(0, 5) + 1] == -1).all()
    cu_bad = d.cu.clone()
    cu_bad[2] = 10 ** 6
    out2 = sv.greedy(cu_bad, d.target, d.tokens)
    torch.cuda.synchronize()
    assert int(out2.status.item()) & 1


def test_greedy_ignores_uniforms_temperature_and_draft_logits():
    """Same outputs whatever the fields greedy verification ignores hold."""
    inp = W.with_deterministic_drafts(W.config(2, seed=5, num_seqs=8))
    a = run_gpu(inp, mode="greedy")
    d = to_device(inp)
    sv = make_verifier(inp)
    out = sv._run("spec_verify_run_greedy", d.cu, d.target, d.draft, d.tokens,
                  torch.full_like(d.uniforms, 7.0), -3.0, None, inp.draft_rows, None, None, None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.out_tokens.cpu().numpy(), a.out_tokens)
    np.testing.assert_array_equal(out.num_accepted.cpu().numpy(), a.num_accepted)


# ------------------------------------------------------------ point-mass drafts

@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_point_named_workload_full_size(idx):
    inp = W.with_deterministic_drafts(W.config(idx))
    rep = _point(inp, f"workload {idx} ({inp.name})")
    assert rep.flagged <= max(3, inp.num_seqs // 10)


@pytest.mark.parametrize("idx", [2, 3, 4, 5])
def test_point_sampled_drafts_reduced(idx):
    """Drafts sampled from q (as in the sampled workloads), verified as if
    they were point proposals: many more accepts at the heavy-tail rows."""
    inp = W.config(idx, seed=31, num_seqs=24)
    _point(inp, f"workload {idx} sampled drafts B=24")


@pytest.mark.parametrize("V", [1, 5, 8, 63, 1000, 4097, 32000, 128256, 152064])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_point_vocab_sizes(V, dtype):
    T = {1: 1.3, 5: 0.7, 8: 1.0, 63: 0.8}.get(V, 1.0)
    inp = W.build(f"pV{V}", 9000 + V, [0, 1, 4, 8, 3], V, dtype, T,
                  W.boosted_top_rows(2.0, 5, 4.0), 1.0)
    _point(inp, f"V={V} {dtype}")


@pytest.mark.parametrize("T", [0.05, 0.2, 0.7, 0.8, 1.0, 1.3, 5.0, 20.0])
def test_point_temperatures(T):
    inp = W.build(f"pT{T}", 56, [2, 6, 0, 8, 5, 1], 32000, W.BF16, T,
                  W.boosted_random_ids_rows(3.0, 20, 8.0), 1.0)
    _point(inp, f"T={T}")


def test_point_long_drafts_and_extreme_uniforms():
    rng = np.random.default_rng(2)
    gam = [70, 0, 3, 65, 64, 0, 1, 63]
    inp = W.build("plong", 93, gam, 2000, W.BF16, 1.0, W.boosted_top_rows(1.0, 1, 12.0), 0.05)
    inp = _argmax_drafts(inp, rng, 1.0)
    _point(inp, "gamma up to 70, drafts on a dominant token")
    u = inp.uniforms
    u[0::3] = np.float32(0.0)
    u[1::3] = np.float32(1 - 2 ** -24)
    _point(inp, "gamma up to 70, u in {0, 1-2^-24}")


def test_point_minus_inf_logits():
    inp = W.build("pneginf", 18, [3, 0, 5, 2], 5000, W.BF16, 0.8, W.iid_normal_rows(2.0), 0.7)
    rng = np.random.default_rng(1)
    neg = np.uint16(0xFF80)
    mask = rng.random(inp.target_logits.shape) < 0.3
    inp.target_logits[mask] = neg
    inp.target_logits[1, :2048 * 2] = neg
    inp.target_logits[1, 3000] = np.uint16(0x4000)
    _point(inp, "-inf logits (some drafts have p(x) = 0)")


@pytest.mark.parametrize("ld_extra,offset", [(8, 0), (1, 0), (0, 1), (3, 5)])
def test_point_row_pitch_and_alignment(ld_extra, offset):
    inp = W.build("ppitch", 13, [2, 5, 0, 3], 4003, W.BF16, 1.0,
                  W.boosted_top_rows(2.0, 20, 5.0), 1.0)
    ora = oracle_point(inp)
    gpu = run_gpu(inp, mode="point", ld=inp.vocab + ld_extra, offset=offset)
    compare(inp, gpu, ora, label=f"point ld=V+{ld_extra} offset={offset}", point=True)
    base = run_gpu(inp, mode="point")
    np.testing.assert_array_equal(gpu.out_tokens, base.out_tokens)


def test_point_lossless_on_gpu_one_launch():
    """Losslessness on the GPU path: 10^6 sequences in one launch, V = 8,
    gamma = 3, fixed draft tokens, fresh uniforms.  Among sequences reaching
    position i the emitted token follows p_i (chi-square, Bonferroni) and
    the pass rate at i is p_i(x_i); outputs equal the oracle's bit for bit
    outside flagged ties."""
    from scipy import special, stats
    rng = np.random.default_rng(707)
    V, g, N = 8, 3, 1_000_000
    tgt_rows = (rng.standard_normal((g + 1, V)) * 1.2).astype(np.float32)
    p = [special.softmax(tgt_rows[i].astype(np.float64)) for i in range(g + 1)]
    xs = [int(np.argsort(p[i])[-1 - i]) for i in range(g)]
    inp = W.VerifyInputs(
        name="point lossless", vocab=V, dtype=W.F32, temperature=1.0,
        gammas=np.full(N, g, np.int32), cu_draft=W.cu_from_gammas([g] * N),
        target_logits=np.tile(tgt_rows, (N, 1)), draft_logits=np.zeros((0, V), np.float32),
        draft_tokens=np.tile(np.asarray(xs, np.int32), N),
        uniforms=W.uniform_grid24(rng, N * (g + 1)))
    log(f"[case] point lossless one launch: B={N} V={V} gamma={g} drafts={xs}")
    gpu = run_gpu(inp, mode="point")
    out = gpu.out_tokens.reshape(N, g + 1)
    n = gpu.num_accepted
    alpha_level = 1e-3 / (2 * g + 1)
    for i in range(g + 1):
        mask = n >= i
        counts = np.bincount(out[mask, i], minlength=V)
        assert stats.chisquare(counts, mask.sum() * p[i]).pvalue > alpha_level, (i, counts)
        if i < g:
            a = p[i][xs[i]]
            reached, passed = mask.sum(), (n >= i + 1).sum()
            z = (passed - reached * a) / np.sqrt(reached * a * (1 - a))
            assert abs(z) < stats.norm.isf(alpha_level / 2), (i, z)
    ora = oracle_point(inp)
    flagged = ties(ora.flagged)
    same = (gpu.num_accepted == ora.num_accepted) & \
        (out == ora.out_tokens.reshape(N, g + 1)).all(axis=1)
    log(f"[parity] point lossless one launch: seqs={N} flagged={int(flagged.sum())} "
        f"differing={int((~same).sum())}")
    assert (same | flagged).all()


def test_modes_share_one_context_and_workspace():
    """The three entry points alternate on one context and workspace; each
    call's results equal a fresh call's."""
    inp = W.with_deterministic_drafts(W.config(2, seed=77, num_seqs=32))
    sv = make_verifier(inp)
    d = to_device(inp)
    ref = {m: run_gpu(inp, mode=m) for m in ("sampled", "point", "greedy")}
    for m in ("greedy", "sampled", "point", "sampled", "greedy", "point"):
        got = run_gpu(inp, sv=sv, dev_inputs=d, mode=m)
        np.testing.assert_array_equal(got.out_tokens, ref[m].out_tokens, err_msg=m)
        np.testing.assert_array_equal(got.num_accepted, ref[m].num_accepted, err_msg=m)


@pytest.mark.parametrize("V", [300000, 1 << 21])
def test_greedy_and_point_largest_vocabularies(V):
    inp = W.with_deterministic_drafts(W.build(f"modes V{V}", 61, [3, 0, 5, 2, 8], V, W.BF16,
                                              1.0, W.boosted_random_ids_rows(2.0, 30, 7.0), 0.8))
    g = run_gpu(inp, mode="greedy")
    og = oracle_greedy(inp)
    np.testing.assert_array_equal(g.out_tokens, og.out_tokens)
    np.testing.assert_array_equal(g.num_accepted, og.num_accepted)
    _point(inp, f"V={V}")


def test_concurrent_streams_with_separate_workspaces():
    """One context, two workspaces, calls on two streams that overlap (the
    header allows it): every result equals the same call made alone."""
    import torch
    from rejection_sampling_verify_08_amd import SpecVerifier
    inps = [W.config(2, seed=300 + k, num_seqs=48) for k in range(2)]
    dets = [W.with_deterministic_drafts(x) for x in inps]
    refs = [(run_gpu(inps[k]), run_gpu(dets[k], mode="point"), run_gpu(dets[k], mode="greedy"))
            for k in range(2)]
    sv = SpecVerifier(inps[0].vocab, inps[0].dtype, max_seqs=48,
                      max_draft_rows=max(x.draft_rows for x in inps))
    # a second workspace for the same context
    ws2 = torch.empty_like(sv.workspace)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    devs = [to_device(inps[k]) for k in range(2)]
    toks = [torch.from_numpy(dets[k].draft_tokens).cuda() for k in range(2)]
    outs = [[sv.allocate_outputs(48, inps[k].draft_rows) for _ in range(3)] for k in range(2)]
    torch.cuda.synchronize()
    ws1 = sv.workspace
    for rep in range(3):
        for k in range(2):
            sv.workspace = ws1 if k == 0 else ws2
            d = devs[k]
            with torch.cuda.stream(streams[k]):
                sv(d.cu, d.target, d.draft, d.tokens, d.uniforms, inps[k].temperature,
                   out=outs[k][0], stream=streams[k])
                sv.point_drafts(d.cu, d.target, toks[k], d.uniforms, inps[k].temperature,
                                out=outs[k][1], stream=streams[k])
                sv.greedy(d.cu, d.target, toks[k], out=outs[k][2], stream=streams[k])
        sv.workspace = ws1
        torch.cuda.synchronize()
        for k in range(2):
            for j in range(3):
                got, ref = outs[k][j], refs[k][j]
                np.testing.assert_array_equal(got.out_tokens.cpu().numpy(), ref.out_tokens,
                                              err_msg=f"rep {rep} stream {k} call {j}")
                np.testing.assert_array_equal(got.num_accepted.cpu().numpy(), ref.num_accepted,
                                              err_msg=f"rep {rep} stream {k} call {j}")


@pytest.mark.parametrize("seed", range(12))
def test_random_configurations_greedy_and_point(seed):
    rng = np.random.default_rng(30_000 + seed)
    V = int(rng.integers(1, 40000))
    B = int(rng.integers(1, 40))
    gam = rng.integers(0, 21, size=B)
    dtype = W.BF16 if rng.random() < 0.6 else W.F32
    T = float(rng.uniform(0.5, 1.5))
    inp = W.with_deterministic_drafts(
        W.build(f"random {seed}", 40_000 + seed, gam, V, dtype, T,
                W.boosted_top_rows(1.0, max(1, min(5, V)), 5.0), float(rng.uniform(0.0, 1.0))))
    _greedy(inp, f"random {seed} V={V} {dtype}")
    _point(inp, f"random {seed} V={V} {dtype} T={T:.3f}")
