"""A seeded serving trace for the draft-length controller: request slots come
and go, each step verifies a random subset of the active slots with the
draft length their controller chose, and the accepted counts are binomial
with a per-request acceptance rate that drifts (chat-like, code-like
phases, the regime change [D] 4.3 motivates the controller with).

The trace is driven by the oracle (oracle/adaptive.py): its outputs decide
the next step's draft lengths, and they are recorded as the expected values
the library must reproduce on the same inputs."""
from __future__ import annotations

import dataclasses

import numpy as np

from oracle import adaptive as A


@dataclasses.dataclass
class Step:
    resets: np.ndarray      # int32 slots reset before the step
    slots: np.ndarray       # int32 [B]
    cu: np.ndarray          # int32 [B+1]
    accepted: np.ndarray    # int32 [B]
    next_k: np.ndarray      # expected int32 [B]
    next_cu: np.ndarray     # expected int32 [B+1]
    totals: tuple           # expected running (sequences, accepted, drafted, emitted)
    k_all: np.ndarray       # expected k of every slot after the step


def make_trace(params: A.Params, num_slots: int, steps: int, seed: int,
               max_batch: int | None = None) -> list[Step]:
    rng = np.random.default_rng(seed)
    bank = A.Bank(params, num_slots)
    rate = rng.uniform(0.1, 0.95, size=num_slots)
    active = rng.random(num_slots) < 0.7
    out = []
    for _ in range(steps):
        # requests finish and new ones take their slots
        ends = np.nonzero(active & (rng.random(num_slots) < 0.03))[0]
        starts = np.nonzero(~active & (rng.random(num_slots) < 0.2))[0]
        active[ends] = False
        active[starts] = True
        resets = starts.astype(np.int32)
        bank.reset(resets)
        rate[starts] = rng.uniform(0.1, 0.95, size=starts.size)
        drift = rng.random(num_slots) < 0.02               # a regime change
        rate[drift] = rng.uniform(0.05, 0.98, size=int(drift.sum()))
        cand = np.nonzero(active)[0]
        take = cand[rng.random(cand.size) < 0.8]
        if max_batch is not None:
            take = take[:max_batch]
        slots = rng.permutation(take).astype(np.int32)
        gam = np.array([bank.k_of(int(s)) for s in slots], dtype=np.int32)
        cu = np.concatenate([[0], np.cumsum(gam)]).astype(np.int32)
        acc = rng.binomial(gam, rate[slots]).astype(np.int32)
        nk, ncu = bank.step(slots, cu, acc)
        st = bank.stats
        out.append(Step(resets, slots, cu, acc, np.asarray(nk, np.int32),
                        np.asarray(ncu, np.int32),
                        (st.sequences, st.accepted, st.drafted, st.emitted),
                        np.asarray(bank.k, np.int32).copy()))
    return out
