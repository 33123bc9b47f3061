"""Seeded synthetic inputs for the batched speculative-decoding verify step.

This module is shared by the tests, the benchmark and the oracle's test
harness. It produces *inputs only*: logits, draft tokens, uniforms and the
ragged per-sequence draft lengths. It holds none of the verify step's
arithmetic (no softmax, no acceptance ratio, no residual, no inverse CDF).

Draft tokens must be samples from the draft distribution q = softmax(l_q / T)
(the draft model proposes gamma tokens autoregressively and the verify step's
losslessness assumes they were drawn from q; see "推测解码与连续批处理深度实战"
section 1.2 step 1 and "大模型推理加速新范式" section 2.1).  They are drawn here
with the Gumbel-max construction, argmax_k(l_k / T + G_k) with G_k iid standard
Gumbel, which samples exactly from softmax(l / T) without normalising it.

Packed ragged layout (no padding), shared by every consumer:
    cu_draft[b]   = sum of gamma_{b'} for b' < b        (int32, B+1 entries)
    target row of (b, i), i in [0, gamma_b]  : cu_draft[b] + b + i
    draft  row of (b, i), i in [0, gamma_b)  : cu_draft[b] + i
    uniforms[target row of (b, i)], i < gamma_b : accept test of draft i
    uniforms[target row of (b, gamma_b)]        : the final draw (residual or bonus)

bf16 logits are stored as their raw uint16 bit patterns; the float64 draws are
rounded once, to nearest with ties to even, directly to 8 significant bits.
Uniforms lie on the 24-bit grid m * 2**-24, m in [0, 2**24), so float32 holds
them exactly.

The five named workloads follow the shapes and value distributions of the
verify step in a continuous-batching server: per-request draft lengths of a
few tokens ("大模型推理加速新范式" section 2.3 gives K of 4-8 as the useful
range), acceptance rates around 0.5-0.7 (same section and section 3.3), and
mixed speculative / plain-decode requests in one batch (the dynamic-batching
post, "结合使用").  No public benchmark or dataset is involved; these synthetic
logits stand in for model outputs.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Callable, Optional

import numpy as np

F32 = "f32"
BF16 = "bf16"

# Draft-noise standard deviation for the heavy-tailed 128K-vocabulary
# workloads, chosen by bisection so that the mean overlap mass
# sum_k min(p_k, q_k) over the calibration seed is 0.60 (written by
# oracle/calibrate_sigma.py with its defaults: seed 1003, 32 sequences of
# 8 positions, bisection with the overlap measured by the oracle).
HEAVY_TAIL_DRAFT_SIGMA = 1.0935

# Stream order of SeedSequence(seed).spawn(6).
_S_TARGET, _S_BOOST, _S_DRAFT, _S_TOKENS, _S_UNIF, _S_GAMMA = range(6)


@dataclasses.dataclass
class VerifyInputs:
    """One batch of verify-step inputs in the packed ragged layout."""

    name: str
    vocab: int
    dtype: str                 # "f32" or "bf16"
    temperature: float         # a float32 value (both sides use exactly this)
    gammas: np.ndarray         # int32 [B]
    cu_draft: np.ndarray       # int32 [B+1]
    target_logits: np.ndarray  # [R_t, V] float32, or uint16 bf16 bits
    draft_logits: np.ndarray   # [R_d, V] same dtype as target_logits
    draft_tokens: np.ndarray   # int32 [R_d]
    uniforms: np.ndarray       # float32 [R_t]

    @property
    def num_seqs(self) -> int:
        return int(self.gammas.shape[0])

    @property
    def target_rows(self) -> int:
        return int(self.target_logits.shape[0])

    @property
    def draft_rows(self) -> int:
        """R_d = cu_draft[B] (also when no draft logits are stored)."""
        return int(self.cu_draft[-1])

    def target_row(self, b: int, i: int) -> int:
        return int(self.cu_draft[b]) + b + i

    def draft_row(self, b: int, i: int) -> int:
        return int(self.cu_draft[b]) + i

    def logit_bytes(self) -> int:
        return int(self.target_logits.nbytes + self.draft_logits.nbytes)


# ---------------------------------------------------------------- rounding

def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns, one rounding to nearest, ties to even.

    Works on the float64 bit pattern: the 52-bit mantissa is rounded to the 7
    bits bf16 keeps (a carry into the exponent is the correct result), the
    value is then exact in float32 and its top 16 bits are the bf16 pattern.
    Normal range only (|x| far inside float32's range, no NaN), which holds
    for every generator here; -inf maps to the bf16 -inf pattern.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    b = x.view(np.uint64)
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = (b + np.uint64((1 << 44) - 1) + lsb) & ~np.uint64((1 << 45) - 1)
    f = r.view(np.float64).astype(np.float32)
    out = (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out[np.isneginf(x)] = 0xFF80
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == BF16:
        return round_to_bf16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """The exact float64 value of stored logits."""
    if dtype == F32:
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    if dtype == BF16:
        return bf16_bits_to_f64(stored)
    raise ValueError(f"unknown dtype {dtype!r}")


def uniform_grid24(rng: np.random.Generator, n: int) -> np.ndarray:
    """n uniforms on the 24-bit grid m * 2**-24, m in [0, 2**24)."""
    m = rng.integers(0, 1 << 24, size=n, dtype=np.int64)
    return (m.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def cu_from_gammas(gammas) -> np.ndarray:
    g = np.asarray(gammas, dtype=np.int64)
    cu = np.zeros(g.shape[0] + 1, dtype=np.int64)
    np.cumsum(g, out=cu[1:])
    return cu.astype(np.int32)


# ---------------------------------------------------------------- sampling

def gumbel_max_token(logits_f64: np.ndarray, temperature: float,
                     rng: np.random.Generator) -> int:
    """One sample from softmax(logits / T) by the Gumbel-max construction.

    -log(E) with E ~ Exp(1) is a standard Gumbel variable."""
    e = rng.standard_exponential(logits_f64.shape[0])
    return int(np.argmax(logits_f64 / float(temperature) - np.log(e)))


# ---------------------------------------------------------------- builders

RowFn = Callable[[np.random.Generator, np.random.Generator, int], np.ndarray]


def iid_normal_rows(sd: float) -> RowFn:
    """Target row generator: iid N(0, sd^2)."""
    def gen(rng, _boost_rng, vocab):
        return rng.standard_normal(vocab) * sd
    return gen


def boosted_random_ids_rows(sd: float, n_boost: int, boost: float) -> RowFn:
    """N(0, sd^2) with `n_boost` distinct uniformly random ids raised by `boost`."""
    def gen(rng, boost_rng, vocab):
        row = rng.standard_normal(vocab) * sd
        ids = boost_rng.choice(vocab, size=min(n_boost, vocab), replace=False)
        row[ids] += boost
        return row
    return gen


def boosted_top_rows(sd: float, n_top: int, boost: float) -> RowFn:
    """N(0, sd^2) with the `n_top` largest draws of the row raised by `boost`
    (a heavy upper tail, like an LM head whose mass sits on a few dozen ids)."""
    def gen(rng, _boost_rng, vocab):
        row = rng.standard_normal(vocab) * sd
        k = min(n_top, vocab)
        if k > 0:
            top = np.argpartition(row, vocab - k)[vocab - k:]
            row[top] += boost
        return row
    return gen


def _child(ss: np.random.SeedSequence, n: int):
    return [np.random.Generator(np.random.PCG64(c)) for c in ss.spawn(n)]


def build(name: str, seed: int, gammas, vocab: int, dtype: str,
          temperature: float, target_row: RowFn,
          draft_sd, draft_copy: Optional[Callable[[int], bool]] = None,
          workers: Optional[int] = None) -> VerifyInputs:
    """Generic packed-batch builder.

    target_row(rng, boost_rng, V) -> float64 row.  The draft row at position i
    of sequence b is the float64 target row of (b, i) plus iid N(0, sd^2)
    noise, where sd = draft_sd (a float) or draft_sd(b); when draft_copy(b) is
    true the draft rows of b are bitwise copies of its rounded target rows.

    Seeding: SeedSequence(seed).spawn(6) gives the streams [target, boost ids,
    draft noise, draft-token Gumbel noise, verify uniforms, gammas]; the first
    four spawn one child per row (target streams per target row, the others
    per draft row), so every row depends only on the seed and its packed
    position, and rows are generated in parallel threads.
    """
    ss = np.random.SeedSequence(seed).spawn(6)
    gammas = np.asarray(gammas, dtype=np.int32)
    if gammas.ndim != 1 or (gammas < 0).any():
        raise ValueError("gammas must be a 1-D array of non-negative ints")
    cu = cu_from_gammas(gammas)
    B = gammas.shape[0]
    R_d = int(cu[-1])
    R_t = R_d + B
    T = float(np.float32(temperature))
    store = np.float32 if dtype == F32 else np.uint16
    tgt = np.empty((R_t, vocab), dtype=store)
    dft = np.empty((R_d, vocab), dtype=store)
    tokens = np.empty(R_d, dtype=np.int32)

    r_tgt = _child(ss[_S_TARGET], R_t)
    r_boost = _child(ss[_S_BOOST], R_t)
    r_draft = _child(ss[_S_DRAFT], R_d)
    r_tok = _child(ss[_S_TOKENS], R_d)

    def one_seq(b: int) -> None:
        g = int(gammas[b])
        sd = draft_sd(b) if callable(draft_sd) else draft_sd
        copy = bool(draft_copy(b)) if draft_copy is not None else False
        for i in range(g + 1):
            trow = int(cu[b]) + b + i
            t64 = target_row(r_tgt[trow], r_boost[trow], vocab)
            tgt[trow] = to_dtype(t64, dtype)
            if i == g:
                break
            drow = int(cu[b]) + i
            if copy:
                dft[drow] = tgt[trow]
            else:
                noise = r_draft[drow].standard_normal(vocab) * sd
                dft[drow] = to_dtype(t64 + noise, dtype)
            tokens[drow] = gumbel_max_token(to_f64(dft[drow], dtype), T,
                                            r_tok[drow])

    n_work = workers or min(16, os.cpu_count() or 1)
    if B * vocab < (1 << 18) or n_work <= 1:
        for b in range(B):
            one_seq(b)
    else:
        with concurrent.futures.ThreadPoolExecutor(n_work) as ex:
            list(ex.map(one_seq, range(B)))

    r_unif = np.random.Generator(np.random.PCG64(ss[_S_UNIF]))
    uniforms = uniform_grid24(r_unif, R_t)
    return VerifyInputs(name=name, vocab=vocab, dtype=dtype, temperature=T,
                        gammas=gammas, cu_draft=cu, target_logits=tgt,
                        draft_logits=dft, draft_tokens=tokens,
                        uniforms=uniforms)


def with_deterministic_drafts(inp: VerifyInputs, name: Optional[str] = None) -> VerifyInputs:
    """A copy of `inp` whose draft tokens are proposed without sampling.

    Each draft token becomes the first maximum of its draft row: the draft
    model decoding greedily, which is the temperature -> 0 limit of the
    Gumbel-max draw above.  These are the inputs of greedy verification and
    stand in for drafts that carry no distribution at all (n-gram /
    prompt-lookup proposals, "推测解码与连续批处理深度实战" sections 1.4 and
    3.3).  Target rows, draft rows and uniforms are shared with `inp`.
    """
    tokens = np.empty(inp.draft_rows, dtype=np.int32)
    for r0 in range(0, inp.draft_rows, 64):
        rows = to_f64(inp.draft_logits[r0:r0 + 64], inp.dtype)
        tokens[r0:r0 + 64] = np.argmax(rows, axis=1)
    return dataclasses.replace(inp, name=name or inp.name + " deterministic drafts",
                               draft_tokens=tokens)


# ---------------------------------------------------------------- candidate trees

@dataclasses.dataclass
class TreeInputs:
    """One batch of candidate trees in the packed layout.

    Sequence b owns nodes g = cu_nodes[b] + n, n in [0, N_b); node 0 is the
    root (the last committed token).  parent[g] is the parent's local index
    (0 <= parent < n), tokens[g] the node's token (root: -1), target row g
    the target's logits for the token after node n, uniforms[g] node n's
    accept test (n >= 1) and, at the root, the final draw."""

    name: str
    vocab: int
    dtype: str
    temperature: float
    cu_nodes: np.ndarray       # int32 [B+1]
    parent: np.ndarray         # int32 [R]
    tokens: np.ndarray         # int32 [R]
    target_logits: np.ndarray  # [R, V]
    uniforms: np.ndarray       # float32 [R]

    @property
    def num_seqs(self) -> int:
        return int(self.cu_nodes.shape[0]) - 1

    @property
    def rows(self) -> int:
        return int(self.target_logits.shape[0])


def tree_shape(levels) -> np.ndarray:
    """Local parent indices of a tree in breadth-first order.  levels is a
    list of (parents, children): the first `parents` nodes of the previous
    level each get `children` children.  [(1, 4), (2, 3), (2, 2), (1, 2)]
    gives 1 + 4 + 6 + 4 + 2 = 17 nodes."""
    parent = [-1]
    prev = [0]
    for n_par, n_ch in levels:
        cur = []
        for pnode in prev[:n_par]:
            for _ in range(n_ch):
                parent.append(pnode)
                cur.append(len(parent) - 1)
        prev = cur
    return np.asarray(parent, dtype=np.int32)


def build_tree(name: str, seed: int, shapes, vocab: int, dtype: str, temperature: float,
               target_row: RowFn, draft_sd: float, workers: Optional[int] = None) -> TreeInputs:
    """Candidate trees: sequence b has the local parent array shapes[b].  A
    node's children carry the top tokens (largest first, distinct while the
    vocabulary allows) of a draft row made of the node's float64 target row
    plus N(0, draft_sd^2) noise -- a drafter proposing its top-k at each
    expanded node.  Seeding as in
    build(): SeedSequence(seed).spawn(6), one child per row for the target,
    boost and draft-noise streams."""
    ss = np.random.SeedSequence(seed).spawn(6)
    sizes = np.asarray([len(sh) for sh in shapes], dtype=np.int64)
    cu = np.zeros(len(shapes) + 1, dtype=np.int64)
    np.cumsum(sizes, out=cu[1:])
    R = int(cu[-1])
    store = np.float32 if dtype == F32 else np.uint16
    tgt = np.empty((R, vocab), dtype=store)
    parent = np.empty(R, dtype=np.int32)
    tokens = np.full(R, -1, dtype=np.int32)
    r_tgt = _child(ss[_S_TARGET], R)
    r_boost = _child(ss[_S_BOOST], R)
    r_draft = _child(ss[_S_DRAFT], R)

    def one_seq(b: int) -> None:
        sh = np.asarray(shapes[b], dtype=np.int32)
        g0 = int(cu[b])
        parent[g0:g0 + len(sh)] = sh
        for n in range(len(sh)):
            t64 = target_row(r_tgt[g0 + n], r_boost[g0 + n], vocab)
            tgt[g0 + n] = to_dtype(t64, dtype)
            kids = np.nonzero(sh == n)[0]
            if kids.size:
                d = t64 + r_draft[g0 + n].standard_normal(vocab) * draft_sd
                top = np.argsort(-d, kind="stable")[:kids.size]
                # fewer tokens than children (tiny vocabularies): repeat them
                tokens[g0 + kids] = np.resize(top, kids.size).astype(np.int32)

    n_work = workers or min(16, os.cpu_count() or 1)
    if R * vocab < (1 << 18) or n_work <= 1:
        for b in range(len(shapes)):
            one_seq(b)
    else:
        with concurrent.futures.ThreadPoolExecutor(n_work) as ex:
            list(ex.map(one_seq, range(len(shapes))))
    r_unif = np.random.Generator(np.random.PCG64(ss[_S_UNIF]))
    return TreeInputs(name=name, vocab=vocab, dtype=dtype,
                      temperature=float(np.float32(temperature)),
                      cu_nodes=cu.astype(np.int32), parent=parent, tokens=tokens,
                      target_logits=tgt, uniforms=uniform_grid24(r_unif, R))


TREE_17 = [(1, 4), (2, 3), (2, 2), (1, 2)]   # 17 nodes, depth 4


def tree_config(seed: int = 6, num_seqs: int = 128, vocab: int = 128256) -> TreeInputs:
    """The named tree workload: 128 sequences with 17-node candidate trees
    (top-4 at the root, top-3 under the two best, top-2 below; 2176 rows,
    as many as the headline chain batch), V = 128256 bf16, T = 1.0,
    heavy-tailed target rows and draft noise as in the headline workload."""
    shape = tree_shape(TREE_17)
    return build_tree(f"trees B={num_seqs} 17 nodes V={vocab} bf16 T=1.0", seed,
                      [shape] * num_seqs, vocab, BF16, 1.0, boosted_top_rows(2.0, 50, 6.0),
                      HEAVY_TAIL_DRAFT_SIGMA)


# ---------------------------------------------------------------- named workloads

def _gamma_stream(seed: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed).spawn(6)[_S_GAMMA]))


def config(index: int, seed: Optional[int] = None, *,
           num_seqs: Optional[int] = None,
           vocab: Optional[int] = None) -> VerifyInputs:
    """The five named workloads (index 1..5); seed defaults to the index.

    num_seqs / vocab override the batch size or vocabulary (same recipe) for
    reduced-size variants used where a full-size batch is not needed.
    """
    s = index if seed is None else seed
    heavy = boosted_top_rows(2.0, 50, 6.0)
    if index == 1:
        B = num_seqs or 1
        return build("B=1 gamma=4 V=1000 f32 T=1.0", s, [4] * B,
                     vocab or 1000, F32, 1.0, iid_normal_rows(2.0), 0.5)
    if index == 2:
        B = num_seqs or 64
        return build("B=64 gamma=5 V=32000 bf16 T=0.7", s, [5] * B,
                     vocab or 32000, BF16, 0.7,
                     boosted_random_ids_rows(3.0, 20, 8.0), 1.0)
    if index == 3:
        B = num_seqs or 128
        return build("B=128 gamma=8 V=128256 bf16 T=1.0", s, [8] * B,
                     vocab or 128256, BF16, 1.0, heavy, HEAVY_TAIL_DRAFT_SIGMA)
    if index == 4:
        B = num_seqs or 256
        gam = _gamma_stream(s).integers(0, 9, size=B)
        return build("ragged 256 seqs gamma~U{0..8} V=128256 bf16 T=0.8", s,
                     gam, vocab or 128256, BF16, 0.8, heavy,
                     HEAVY_TAIL_DRAFT_SIGMA)
    if index == 5:
        B = num_seqs or 512
        half = B // 2
        return build("B=512 gamma=4 V=152064 bf16 T=1.0 half draft==target",
                     s, [4] * B, vocab or 152064, BF16, 1.0, heavy,
                     lambda b: 2.0, draft_copy=lambda b: b < half)
    raise ValueError("config index must be 1..5")


CONFIG_SHAPES = {
    1: dict(B=1, gamma=4, V=1000, dtype=F32, T=1.0),
    2: dict(B=64, gamma=5, V=32000, dtype=BF16, T=0.7),
    3: dict(B=128, gamma=8, V=128256, dtype=BF16, T=1.0),
    4: dict(B=256, gamma="U{0..8}", V=128256, dtype=BF16, T=0.8),
    5: dict(B=512, gamma=4, V=152064, dtype=BF16, T=1.0),
}
