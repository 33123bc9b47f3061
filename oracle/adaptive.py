"""Plain-Python oracle of the adaptive draft-length controller and the
acceptance statistics.

TEST INFRASTRUCTURE ONLY (like the rest of `oracle/`): imported by the tests,
never by the product path, and sharing no code with it.

Pages cited (by title and section):
  [D] "大模型推理加速新范式：推测解码（Speculative Decoding）原理剖析与
      vLLM生产级实现", section 4.3 (a sliding-window acceptance-rate feedback
      rule for the draft length K) and section 4.2 (the accept-rate metric
      spec_token_accept_rate as the core indicator).
  [B] the blog.hotdry.top post on speculative decoding and dynamic batching,
      延迟权衡与自适应策略 (adjust the candidate length from the recent pass
      rate) and its 工程落地参数清单 (start at 4-8; over the last 10 rounds,
      a pass rate above 80% adds one, below 50% removes one).

What one controller does, in the order of [D] 4.3:
  * it starts at k = k_init ([D] starts at k_min);
  * after each verify step of its sequence it takes the step's acceptance
    ratio alpha = accepted / max(drafted, 1) and appends it to a history of
    the last `window` values (the oldest value drops out);
  * with fewer than `min_history` values it changes nothing;
  * otherwise avg = (sum of the history, oldest first) / its length, and
    k <- min(k + 1, k_max) if avg > up, k <- max(k - 1, k_min) if avg < down.
[D]'s preset: k_min 2, k_max 8, k_init 2, window 50, min_history 10,
up = 0.6 + 0.1, down = 0.6 - 0.1 (computed in float64 as printed).
[B]'s preset (a reading: its list gives the thresholds, a 10-round window
and a 4-8 start; the lower bound 1 and the use of the same mean-of-ratios
rule are this reading's): k_min 1, k_max 8, k_init 4, window 10,
min_history 10, up 0.8, down 0.5.

Statistics: running totals of sequences verified, drafts accepted, drafts
proposed and tokens emitted (accepted + 1 per sequence); the accept rate of
[D] 4.2 is accepted / drafted.
"""
from __future__ import annotations

import dataclasses


@dataclasses.dataclass(frozen=True)
class Params:
    k_min: int
    k_max: int
    k_init: int
    window: int
    min_history: int
    up: float
    down: float


def preset_vllm_page() -> Params:
    """[D] 4.3 defaults: k_min=2, k_max=8, window=50, target 0.6 +- 0.1."""
    target = 0.6
    return Params(k_min=2, k_max=8, k_init=2, window=50, min_history=10,
                  up=target + 0.1, down=target - 0.1)


def preset_checklist() -> Params:
    """[B] 工程落地参数清单: last 10 rounds, > 80% adds one, < 50% removes one."""
    return Params(k_min=1, k_max=8, k_init=4, window=10, min_history=10, up=0.8, down=0.5)


def next_length(p: Params, k: int, alphas) -> int:
    """The draft length after a step, from the length k before it and every
    acceptance ratio of the sequence so far (`alphas`, oldest first; the
    step's own ratio is the last): the mean of the last `window` ratios moves
    k by one step towards the band [down, up], within [k_min, k_max]."""
    recent = alphas[-p.window:]
    if len(recent) < p.min_history:
        return k
    total = 0.0
    for a in recent:                          # sequential, oldest first
        total += a
    avg = total / len(recent)
    if avg > p.up:
        return min(k + 1, p.k_max)
    if avg < p.down:
        return max(k - 1, p.k_min)
    return k


def trace(p: Params, steps):
    """Draft length after each of `steps` = [(accepted, drafted), ...] for
    one sequence that starts at k_init."""
    k, alphas, out = p.k_init, [], []
    for accepted, drafted in steps:
        alphas.append(accepted / max(drafted, 1))
        k = next_length(p, k, alphas)
        out.append(k)
    return out


@dataclasses.dataclass
class Stats:
    sequences: int = 0
    accepted: int = 0
    drafted: int = 0
    emitted: int = 0

    def accept_rate(self) -> float:
        return self.accepted / self.drafted if self.drafted else 0.0


class Bank:
    """Controllers for `num_slots` request slots plus the running totals.

    step() takes one verify step's batch: slot of each sequence, the packed
    offsets cu (gamma_b = cu[b+1] - cu[b] drafts) and the accepted counts, and
    returns each sequence's next draft length and the next step's packed
    offsets (exclusive prefix of the next lengths)."""

    def __init__(self, p: Params, num_slots: int):
        self.p = p
        self.k = [p.k_init] * num_slots
        self.alphas = [[] for _ in range(num_slots)]
        self.stats = Stats()

    def reset(self, slots) -> None:
        for s in slots:
            self.k[int(s)] = self.p.k_init
            self.alphas[int(s)] = []

    def k_of(self, slot: int) -> int:
        return self.k[slot]

    def step(self, slots, cu, accepted):
        next_k, next_cu = [], [0]
        for b, s in enumerate(slots):
            s = int(s)
            drafted = int(cu[b + 1]) - int(cu[b])
            acc = int(accepted[b])
            self.alphas[s].append(acc / max(drafted, 1))
            self.k[s] = next_length(self.p, self.k[s], self.alphas[s])
            next_k.append(self.k[s])
            next_cu.append(next_cu[-1] + self.k[s])
            self.stats.sequences += 1
            self.stats.accepted += acc
            self.stats.drafted += drafted
            self.stats.emitted += acc + 1
        return next_k, next_cu
