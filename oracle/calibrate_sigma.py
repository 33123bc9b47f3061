"""Calibrate the draft-noise sigma of the heavy-tailed 128K-vocabulary workload.

The workload asks for draft = target + N(0, sigma^2) with sigma chosen so the
mean overlap mass sum_k min(p_k, q_k) (the per-position acceptance probability
alpha) is about 0.6, the middle of the 0.5-0.7 range "大模型推理加速新范式"
gives in sections 2.3 and 3.3.  This script bisects sigma on the calibration
seed, measuring the overlap with the oracle, and prints the value that
`workloads.HEAVY_TAIL_DRAFT_SIGMA` holds.

Run:  python -m oracle.calibrate_sigma
"""
from __future__ import annotations

import argparse

import numpy as np

import oracle
import workloads as W


def mean_overlap(sigma: float, seed: int, num_seqs: int, vocab: int,
                 temperature: float) -> float:
    inp = W.build("calibration", seed, [8] * num_seqs, vocab, W.BF16,
                  temperature, W.boosted_top_rows(2.0, 50, 6.0), sigma)
    vals = []
    for b in range(inp.num_seqs):
        for i in range(int(inp.gammas[b])):
            vals.append(oracle.overlap_mass(
                inp.target_logits[inp.target_row(b, i)],
                inp.draft_logits[inp.draft_row(b, i)], inp.temperature,
                dtype="bf16"))
    return float(np.mean(vals))


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--seed", type=int, default=1003)
    ap.add_argument("--num-seqs", type=int, default=32)
    ap.add_argument("--vocab", type=int, default=128256)
    ap.add_argument("--target", type=float, default=0.60)
    ap.add_argument("--iters", type=int, default=16)
    a = ap.parse_args()
    lo, hi = 0.5, 2.0
    for _ in range(a.iters):
        mid = 0.5 * (lo + hi)
        alpha = mean_overlap(mid, a.seed, a.num_seqs, a.vocab, 1.0)
        print(f"sigma={mid:.5f} mean alpha={alpha:.5f}", flush=True)
        if alpha > a.target:
            lo = mid          # too similar: more noise
        else:
            hi = mid
    sigma = round(0.5 * (lo + hi), 4)
    print(f"HEAVY_TAIL_DRAFT_SIGMA = {sigma}")


if __name__ == "__main__":
    main()
