"""Randomized parity sweep over fixed seed ranges (GPU, marked slow).

Three families of seeded batches, each case drawn from its seed alone and
checked against the oracle under the same parity rule as every other GPU
test (tests/gpu_helpers.py):

* masked: -inf over 0-99% of every row, temperatures from ~0.04 to ~25,
  drafted tokens hit by the mask restored at logit 1 (so q(x) is tiny) and
  gamma up to 63: rejections whose residual is a difference of near-equal
  distributions, down to and below fp32 resolution;
* near: draft rows within 0-0.02 logits of the target rows (a residual
  ~1e-3 of the mass or less), fp32 and bf16, through spec_verify_run and
  spec_verify_run_point_drafts;
* shapes: vocabulary, batch, ragged gamma (up to 20), dtype, temperature,
  generator, draft noise and row pitch, as test_random_configurations but
  over further seeds;
* large: vocabularies of 131073 to 700000 logits (rows of more than 64
  residual tiles, and above 262144 of more than 64 row-pass tasks: the
  workgroup-wide scans instead of the one-wave ones), B <= 5, near-identical
  to distant draft rows, through spec_verify_run and
  spec_verify_run_point_drafts.

Sizes are capped (V < 9000 and B < 25, or B <= 5 for the large family) so
that the oracle finishes each case in well under a second; each case prints
its family, seed and shape first.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import compare, log, oracle_point, run_gpu, status_ok

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

BLOCK = 20   # seeds per test


def _gens(rng, V):
    return [W.iid_normal_rows(float(rng.uniform(0.3, 3.0))),
            W.boosted_top_rows(2.0, max(1, min(50, V // 3)), 6.0),
            W.boosted_random_ids_rows(3.0, max(1, min(20, V)), 8.0)]


def _masked(seed):
    rng = np.random.default_rng(500_000 + seed)
    V = int(rng.choice([int(rng.integers(2, 300)), int(rng.integers(300, 9000))]))
    B = int(rng.integers(1, 25))
    gam = rng.integers(0, int(rng.choice([8, 20, 63])) + 1, size=B)
    dtype = W.BF16 if rng.random() < 0.6 else W.F32
    T = float(rng.choice([0.05, 0.2, 1.0, 3.0, 20.0])) * float(rng.uniform(0.8, 1.25))
    gen = _gens(rng, V)[int(rng.integers(0, 3))]
    noise = float(rng.uniform(0.0, 2.0))
    frac = float(rng.choice([0.0, 0.3, 0.9, 0.99]))
    inp = W.build(f"sweep masked {seed}", 510_000 + seed, gam, V, dtype, T, gen, noise)
    neg = np.uint16(0xFF80) if dtype == W.BF16 else np.float32(-np.inf)
    one = np.uint16(0x3F80) if dtype == W.BF16 else np.float32(1.0)
    for arr in (inp.target_logits, inp.draft_logits):
        if arr.shape[0] == 0 or frac == 0.0:
            continue
        arr[rng.random(arr.shape) < frac] = neg
        for r in range(arr.shape[0]):
            if (arr[r] == neg).all():
                arr[r, int(rng.integers(0, V))] = one
    for r, x in enumerate(inp.draft_tokens):
        if inp.draft_logits[r, x] == neg:
            inp.draft_logits[r, x] = one
    return inp


def _near(seed):
    rng = np.random.default_rng(600_000 + seed)
    V = int(rng.integers(2, 9000))
    B = int(rng.integers(1, 25))
    gam = rng.integers(0, 13, size=B)
    dtype = W.BF16 if seed % 2 else W.F32
    T = float(rng.uniform(0.3, 2.0))
    gen = _gens(rng, V)[int(rng.integers(0, 3))]
    return W.build(f"sweep near {seed}", 610_000 + seed, gam, V, dtype, T, gen,
                   float(rng.uniform(0.0, 0.02)))


def _shapes(seed):
    rng = np.random.default_rng(700_000 + seed)
    V = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 9000))]))
    B = int(rng.integers(1, 25))
    gam = rng.integers(0, 21, size=B)
    dtype = W.BF16 if rng.random() < 0.6 else W.F32
    T = float(rng.uniform(0.5, 1.5))
    gen = _gens(rng, V)[int(rng.integers(0, 3))]
    inp = W.build(f"sweep shapes {seed}", 710_000 + seed, gam, V, dtype, T, gen,
                  float(rng.uniform(0.0, 2.0)))
    return inp, V + int(rng.integers(0, 3)) * 8


def _large(seed):
    rng = np.random.default_rng(900_000 + seed)
    V = int(rng.integers(131_073, 700_000))
    B = int(rng.integers(1, 6))
    gam = rng.integers(0, 9, size=B)
    dtype = W.BF16 if seed % 2 else W.F32
    T = float(rng.choice([0.2, 0.7, 1.0, 2.0]))
    gen = _gens(rng, V)[int(rng.integers(0, 3))]
    return W.build(f"sweep large {seed}", 910_000 + seed, gam, V, dtype, T, gen,
                   float(rng.choice([0.005, 0.5, 1.5])))


def _run(inp, label, point=False, ld=None):
    log(f"[case] {label}: B={inp.num_seqs} R_d={inp.draft_rows} V={inp.vocab} {inp.dtype} "
        f"T={inp.temperature:.4f}")
    ora = oracle_point(inp) if point else oracle.verify_inputs(inp)
    gpu = run_gpu(inp, mode="point" if point else "sampled", ld=ld)
    compare(inp, gpu, ora, label=label, point=point)
    assert status_ok(gpu.status, ora), f"{label}: status {gpu.status:#x}"


@pytest.mark.parametrize("block", range(15))
def test_sweep_masked(block):
    for seed in range(block * BLOCK, (block + 1) * BLOCK):
        _run(_masked(seed), f"sweep masked {seed}")


@pytest.mark.parametrize("block", range(6))
def test_sweep_near_identical(block):
    for seed in range(block * BLOCK, (block + 1) * BLOCK):
        inp = _near(seed)
        _run(inp, f"sweep near {seed}")
        _run(inp, f"sweep near {seed} point", point=True)


@pytest.mark.parametrize("block", range(6))
def test_sweep_shapes(block):
    for seed in range(block * BLOCK, (block + 1) * BLOCK):
        inp, ld = _shapes(seed)
        _run(inp, f"sweep shapes {seed} ld={ld}", ld=ld)


@pytest.mark.parametrize("block", range(3))
def test_sweep_large_vocabulary(block):
    for seed in range(block * BLOCK, (block + 1) * BLOCK):
        inp = _large(seed)
        _run(inp, f"sweep large {seed}")
        _run(inp, f"sweep large {seed} point", point=True)
