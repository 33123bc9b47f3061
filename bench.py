#!/usr/bin/env python3
"""Benchmark of the batched speculative-decoding verify step on one MI355X.

One step = one spec_verify_run call (row statistics of every target and draft
row, accept tests, first-rejection stop, residual / bonus draw) over one batch
of a named workload.  The headline is B=128 sequences, gamma=8, V=128256,
bf16 logits, T=1.0, heavy-tailed target logits with draft noise giving
alpha ~ 0.6.  Inputs are resident in HBM before timing; three rotating device
copies keep a step from reading logits the previous step left in the 256 MB
Infinity Cache.

Every named workload (1-5) is measured the same way: W untimed steps (and
at least --min-warmup-s seconds of them, for the GPU's clocks), then K
timed steps, each between an event pair of its own (the per-step GPU
span: median, p10, p90; the value comes from the median); then, outside the
timed region, K steps with the library's per-kernel dispatch events (each
kernel's median duration: those events put ~5 us between the two kernels,
so they are kept out of the step figures) and K steps with no per-step
events (the plain mean, reported for reference); the two small
latency-bound workloads also get the device time per step of a replayed HIP
graph of calls.  For each workload the float64 CPU oracle runs on the same
batch: its rate is the CPU baseline and its outputs give the parity status
(sequences whose outputs match, tie-flagged ones, tie differences, widened
ones, and violations of the parity rule).  The headline is measured last, so
the others also bring the GPU to its steady clocks.

Prints one JSON line: the headline's verified rows/s (value, from the
median step), whole-step HBM GB/s, the roofline of the dominant kernel (the
row-statistics pass, HBM-bound; its duration from HIP events that are its
dispatch's own start and stop), the practical read ceiling measured by a
streaming-read probe over 1 GiB with the row pass's load pattern, the
oracle timed on this host, and under "configs" the same figures for every
named workload.  Under "modes" it carries the other entry points on the
headline rows: greedy, point-mass drafts and trees, and the draft-length
controller.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
HEADLINE = 3
METRIC = "verified rows/s + achieved HBM GB/s (% peak), B=128 γ=8 V=128256 bf16"
PMC_FILE = os.path.join(ROOT, "profiles", "verify_kernels_B128_g8_V128256_bf16.pmc.json")
KERNEL_SOURCES = [os.path.join(ROOT, "rejection_sampling_verify_08_amd", "csrc", f)
                  for f in ("spec_verify_kernels.hpp", "greedy_kernels.hpp", "tree_kernels.hpp",
                           "spec_verify.hip")]


def kernel_source_hash() -> str:
    """Identity of the kernel code: a hash of the kernel sources with comments
    and blank lines removed (an edit to a comment leaves it unchanged)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        src = re.sub(r"//[^\n]*", "", open(f).read())
        h.update("\n".join(l.rstrip() for l in src.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def traffic_from_profile(src_hash: str, mode: str = "sampled"):
    """HBM bytes per launch of a mode's dominant kernel from the committed
    rocprofv3 counter summary, or None when it is missing or the kernels
    changed since."""
    try:
        rec = json.load(open(PMC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != src_hash:
        return None
    return (rec.get("hbm_bytes_per_launch") or {}).get(mode)


def algorithmic_bytes(inp, num_accepted, mode="sampled"):
    """Minimum bytes one step must move.

    sampled: every target and draft row once, the final-draw row(s) once more
      (2 rows after a rejection, 1 for the bonus), tokens, uniforms, offsets,
      outputs (tokens, counts, p/q at the drafts, residual sums).
    point:   every target row once, one final-draw target row per sequence
      once more, tokens, uniforms, offsets, the same outputs.
    greedy:  every target row once, tokens, offsets, tokens and counts out.
    Returns (first-pass logit bytes, re-read logit bytes, other bytes)."""
    e = 2 if inp.dtype == "bf16" else 4
    V = inp.vocab
    B, R_t, R_d = inp.num_seqs, inp.target_rows, inp.draft_rows
    io = R_d * 4 + (B + 1) * 4 + R_t * 4 + B * 4          # tokens, cu, out tokens, counts
    if mode == "greedy":
        return R_t * V * e, 0, io
    io += R_t * 4 + R_d * 8 + B * 4                        # uniforms, p/q, residual sums
    if mode == "point":
        return R_t * V * e, B * V * e, io
    rejected = int((num_accepted < inp.gammas).sum())
    return (R_t + R_d) * V * e, (2 * rejected + (B - rejected)) * V * e, io


def host_cpu():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return model


def pct(xs):
    import numpy as np
    return {"p10": round(float(np.percentile(xs, 10)), 2),
            "p50": round(float(np.percentile(xs, 50)), 2),
            "p90": round(float(np.percentile(xs, 90)), 2)}


def run_oracle(inp, runs: int = 1, budget_s: float = 0.0):
    """The float64 oracle on the whole batch: `runs` runs at least, more
    while under `budget_s` seconds.  Returns (result, seconds per run)."""
    import oracle
    oracle._load()
    times = []
    res = None
    while True:
        t0 = time.perf_counter()
        res = oracle.verify_inputs(inp)
        times.append(time.perf_counter() - t0)
        if len(times) >= runs and sum(times) >= budget_s:
            break
    return res, times


def parity_status(inp, out, ora):
    """The parity rule of the GPU tests on this batch, counted, not asserted."""
    import numpy as np
    from tests.gpu_helpers import HostOutput, parity_check
    gpu = HostOutput(out.out_tokens.cpu().numpy(), out.num_accepted.cpu().numpy(),
                     out.p_draft.cpu().numpy().astype(np.float64),
                     out.q_draft.cpu().numpy().astype(np.float64),
                     out.residual_sum.cpu().numpy().astype(np.float64),
                     int(out.status.cpu().item()) & 0xFFFFFFFF)
    rep = parity_check(inp, gpu, ora)
    same = int(((gpu.num_accepted == ora.num_accepted) &
                np.array([np.array_equal(gpu.out_tokens[int(inp.cu_draft[b]) + b:
                                                         int(inp.cu_draft[b + 1]) + b + 1],
                                         ora.out_tokens[int(inp.cu_draft[b]) + b:
                                                        int(inp.cu_draft[b + 1]) + b + 1])
                          for b in range(inp.num_seqs)])).sum())
    return {"status": "green" if not rep.failures else "red",
            "sequences": rep.sequences, "identical": same,
            "tie_flagged": rep.flagged, "tie_differences": rep.tie_differences,
            "widened": rep.widened, "violations": len(rep.failures),
            "max_prob_rel": float(f"{rep.max_prob_rel:.3g}"),
            "max_residual_rel": float(f"{rep.max_residual_rel:.3g}"),
            "device_status": gpu.status}


class Bench:
    def __init__(self, a):
        import torch
        self.a = a
        self.torch = torch
        torch.cuda.set_device(0)
        self.dev = torch.device("cuda", 0)
        # every call goes to a stream of its own (default priority), which
        # is also torch's current stream from here on
        self.stream = torch.cuda.Stream(self.dev)
        torch.cuda.set_stream(self.stream)

    def events(self, n):
        evs = [self.torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(self.stream)          # creates the underlying hipEvent
        return evs

    def rows(self, arr, dtype):
        import numpy as np
        torch = self.torch
        if dtype == "bf16":
            return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(self.dev)
        return torch.from_numpy(arr).to(self.dev)

    def spans(self, call):
        """K steps, each between an event pair of its own on the stream:
        per-step spans (us) and the wall-clock mean per step (us)."""
        a = self.a
        torch = self.torch
        pairs = [self.events(2) for _ in range(a.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(a.steps):
            pairs[i][0].record(self.stream)
            call(i, None)
            pairs[i][1].record(self.stream)
        torch.cuda.synchronize()
        wall_us = (time.perf_counter() - t0) * 1e6 / a.steps
        return [e0.elapsed_time(e1) * 1e3 for e0, e1 in pairs], wall_us

    def timed(self, call, nk):
        """W untimed steps, then the K timed steps, each between an event
        pair of its own on the stream (the per-step span: median, p10, p90;
        and the wall clock over the K steps, synchronised on both sides).
        Then, outside the timed region, K steps with the library's
        per-kernel dispatch events for each kernel's duration (those events
        put ~5 us between the two kernels, so they stay out of the step
        figures) and K steps with no per-step events at all (the plain
        throughput).  Returns spans, per-kernel durations, wall-clock and
        plain means per step (us)."""
        a = self.a
        torch = self.torch
        # at least W untimed steps, and at least --min-warmup-s seconds of
        # them: the GPU's clocks settle only after ~0.2 s of this load (with
        # 5 steps the headline measured ~3% slower, both kernels alike)
        self.warmup_run = 0
        t_w = time.perf_counter()
        while (self.warmup_run < a.warmup or
               time.perf_counter() - t_w < a.min_warmup_s):
            call(self.warmup_run, None)
            self.warmup_run += 1
            if self.warmup_run % 64 == 0:
                torch.cuda.synchronize()
        spans, wall_us = self.spans(call)
        ev = [self.events(2 * nk) for _ in range(a.steps)]
        torch.cuda.synchronize()
        for i in range(a.steps):
            call(i, ev[i])
        torch.cuda.synchronize()
        kern = [[e[2 * k].elapsed_time(e[2 * k + 1]) * 1e3 for e in ev] for k in range(nk)]
        e0, e1 = self.events(2)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for i in range(a.steps):
            call(i, None)
        e1.record(self.stream)
        torch.cuda.synchronize()
        plain_us = e0.elapsed_time(e1) * 1e3 / a.steps
        return spans, kern, wall_us, plain_us

    def graph_step_us(self, call, per_graph=64, replays=10):
        """Device time per step of a captured HIP graph of `per_graph` calls
        (rotating inputs), over `replays` timed replays."""
        torch = self.torch
        for i in range(per_graph):
            call(i, None)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per_graph):
                call(i, None)
        g.replay()
        torch.cuda.synchronize()
        per = []
        for _ in range(replays):
            e0, e1 = self.events(2)
            e0.record(self.stream)
            g.replay()
            e1.record(self.stream)
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / per_graph)
        del g
        return pct(per)

    def config(self, idx, keep=False):
        """Measure named workload `idx`; returns its record (and, with keep,
        the device inputs for the mode measurements)."""
        import numpy as np
        import workloads as W
        from rejection_sampling_verify_08_amd import SpecVerifier
        torch = self.torch
        a = self.a
        t_gen = time.perf_counter()
        inp = W.config(idx)
        print(f"[bench] config {idx}: generated {inp.name} in {time.perf_counter() - t_gen:.1f} s",
              file=sys.stderr, flush=True)
        host_t, host_d = self.rows(inp.target_logits, inp.dtype), self.rows(inp.draft_logits,
                                                                           inp.dtype)
        sets = []
        for _ in range(max(1, a.sets)):
            t, d = torch.empty_like(host_t), torch.empty_like(host_d)
            t.copy_(host_t)
            d.copy_(host_d)
            sets.append((t, d))
        del host_t, host_d
        cu = torch.from_numpy(inp.cu_draft).to(self.dev)
        tok = torch.from_numpy(inp.draft_tokens).to(self.dev)
        uni = torch.from_numpy(inp.uniforms).to(self.dev)
        tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
        sv = SpecVerifier(inp.vocab, tdt, max_seqs=inp.num_seqs, max_draft_rows=inp.draft_rows)
        outs = [sv.allocate_outputs(inp.num_seqs, inp.draft_rows) for _ in sets]
        nk = sv.num_kernels

        def step(i, events):
            # torch's current stream: the bench's stream, or the capture
            # stream inside graph_step_us
            t, d = sets[i % len(sets)]
            sv(cu, t, d, tok, uni, inp.temperature, out=outs[i % len(sets)],
               stream=torch.cuda.current_stream(self.dev), timing_events=events)

        spans, kern, wall_us, plain_us = self.timed(step, nk)
        # unflushed: the same input set every step, so part of a step's rows
        # may still be in the Infinity Cache from the step before
        same, _ = self.spans(lambda i, ev: step(0, ev))
        graph = self.graph_step_us(step) if idx in (1, 2) else None
        torch.cuda.synchronize()
        num_acc = outs[0].num_accepted.cpu().numpy()
        first, reread, small = algorithmic_bytes(inp, num_acc)
        step_bytes = first + reread + small
        step_p = pct(spans)
        med_s = step_p["p50"] / 1e6
        k_med = [float(np.median(k)) for k in kern]
        achieved = first / (k_med[0] / 1e6) / 1e9
        # the oracle's rate is a median over --oracle-runs runs (the headline
        # repeats until the CPU budget is spent); --cpu-budget 0 times the
        # other workloads once, from their parity run
        ora, o_times = run_oracle(inp, runs=a.oracle_runs if (idx == HEADLINE or a.cpu_budget > 0)
                                  else 1, budget_s=a.cpu_budget if idx == HEADLINE else 0.0)
        o_med = float(np.median(o_times))
        rec = {
            "workload": inp.name, "B": inp.num_seqs,
            "gamma": "U{0..8}" if idx == 4 else int(inp.gammas[0]), "V": inp.vocab,
            "dtype": inp.dtype, "temperature": inp.temperature,
            "target_rows": inp.target_rows, "draft_rows": inp.draft_rows,
            "step_us": step_p, "wall_us_per_step": round(wall_us, 2),
            "unevented_us_per_step": round(plain_us, 2), "warmup_steps_run": self.warmup_run,
            "unflushed_step_us": pct(same),
            "graph_step_us": graph,
            "verified_rows_per_s": round(inp.target_rows / med_s, 1),
            "hbm_gbps": round(step_bytes / med_s / 1e9, 1),
            "hbm_frac": round(step_bytes / med_s / 1e9 / PEAK_HBM_GBPS, 4),
            "step_algorithmic_bytes": step_bytes,
            "kernel_names": ["row_stats_kernel", "finish_kernel"][:nk],
            "kernel_us": {"p50": [round(x, 2) for x in k_med],
                          "p10": [round(float(np.percentile(k, 10)), 2) for k in kern],
                          "p90": [round(float(np.percentile(k, 90)), 2) for k in kern]},
            "roofline": {"bound": "hbm", "kernel": "row_stats_kernel",
                         "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(achieved / PEAK_HBM_GBPS, 4),
                         "kernel_us": round(k_med[0], 2), "algorithmic_bytes_per_launch": first},
            "mean_accepted": round(float(num_acc.mean()), 4),
            "parity": parity_status(inp, outs[0], ora),
            "oracle": {"verified_rows_per_s": round(inp.target_rows / o_med, 1),
                       "runs": len(o_times), "median_s": round(o_med, 3), "cores": 1},
        }
        print(f"[bench] config {idx}: step p50 {step_p['p50']:.1f} us, "
              f"kernels {rec['kernel_us']['p50']}, parity {rec['parity']['status']}",
              file=sys.stderr, flush=True)
        if keep:
            return rec, dict(inp=inp, sets=sets, cu=cu, tok=tok, uni=uni, sv=sv, outs=outs,
                             step=step)
        del sets, outs, sv
        torch.cuda.empty_cache()
        return rec, None


def read_probe(b, mib):
    """The practical read ceiling: one streaming read of a buffer far larger
    than the Infinity Cache, with the row pass's load pattern."""
    import numpy as np
    torch = b.torch
    from rejection_sampling_verify_08_amd.binding import read_probe as probe_call
    nb = mib << 20
    buf = torch.empty(nb, dtype=torch.uint8, device=b.dev).fill_(7)
    sink = torch.zeros(1, dtype=torch.int32, device=b.dev)
    probe = {"bytes": nb, "kernel": "read_probe_kernel",
             "loads": "16-byte, one 1 KB span per wave instruction (the row pass's pattern)"}
    for nt, key in ((True, "nontemporal_gbps"), (False, "plain_gbps")):
        for _ in range(3):
            probe_call(buf, sink, nontemporal=nt, stream=b.stream)
        runs = [b.events(2) for _ in range(10)]
        torch.cuda.synchronize()
        for e in runs:
            probe_call(buf, sink, nontemporal=nt, stream=b.stream, events=e)
        torch.cuda.synchronize()
        gbps = sorted(nb / (e[0].elapsed_time(e[1]) / 1e3) / 1e9 for e in runs)
        probe[key] = round(float(np.median(gbps)), 1)
        probe[key.replace("gbps", "best_gbps")] = round(gbps[-1], 1)
    del buf
    torch.cuda.empty_cache()
    return probe


def modes(b, h, src_hash):
    """The other entry points on the headline rows (deterministic drafts for
    greedy and point-mass drafts), tree verification on the named tree
    workload, and the draft-length controller."""
    import numpy as np
    import workloads as W
    torch = b.torch
    inp, sets, cu, uni, sv, outs = h["inp"], h["sets"], h["cu"], h["uni"], h["sv"], h["outs"]
    det = W.with_deterministic_drafts(inp)
    tok_det = torch.from_numpy(det.draft_tokens).to(b.dev)
    res = {}

    def greedy_step(i, events):
        t, _ = sets[i % len(sets)]
        sv.greedy(cu, t, tok_det, out=outs[i % len(sets)], stream=b.stream, timing_events=events)

    def point_step(i, events):
        t, _ = sets[i % len(sets)]
        sv.point_drafts(cu, t, tok_det, uni, inp.temperature, out=outs[i % len(sets)],
                        stream=b.stream, timing_events=events)

    for name, step, kname in (("greedy", greedy_step, "argmax_kernel"),
                              ("point_drafts", point_step, "row_stats_kernel")):
        spans, kern, wall_us, plain_us = b.timed(step, sv.num_kernels)
        acc = outs[0].num_accepted.cpu().numpy()
        first, reread, small = algorithmic_bytes(det, acc, "greedy" if name == "greedy" else "point")
        med_s = float(np.median(spans)) / 1e6
        k_med = [float(np.median(k)) for k in kern]
        ach = first / (k_med[0] / 1e6) / 1e9
        res[name] = {
            "value": round(inp.target_rows / med_s, 1), "unit": "verified rows/s",
            "step_us": pct(spans), "hbm_gbps": round((first + reread + small) / med_s / 1e9, 1),
            "kernel_us": [round(x, 2) for x in k_med],
            "kernel_names": [kname, "greedy_finish_kernel" if name == "greedy" else "finish_kernel"],
            "mean_accepted": round(float(acc.mean()), 4),
            "status": int(outs[0].status.cpu().item()),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4),
                         "traffic": traffic_from_profile(src_hash, name), "kernel": kname,
                         "kernel_us": round(k_med[0], 2), "algorithmic_bytes_per_launch": first}}

    # tree verification on the named tree workload (128 trees of 17 nodes,
    # 2176 rows: as many as the chain batch)
    tr = W.tree_config()
    t_tree = b.rows(tr.target_logits, inp.dtype)
    tsets = [t_tree] + [t_tree.clone() for _ in range(len(sets) - 1)]
    dvc = lambda arr: torch.from_numpy(np.ascontiguousarray(arr)).to(b.dev)
    tcu, tpar, ttok, tuni = dvc(tr.cu_nodes), dvc(tr.parent), dvc(tr.tokens), dvc(tr.uniforms)
    tree_out = [None] * len(tsets)

    def tree_step(kind):
        def step(i, events):
            j = i % len(tsets)
            if kind == "tree_greedy":
                tree_out[j] = sv.tree_greedy(tcu, tpar, ttok, tsets[j], out=tree_out[j],
                                             timing_events=events, stream=b.stream)
            else:
                tree_out[j] = sv.tree_point(tcu, tpar, ttok, tsets[j], tuni, tr.temperature,
                                            out=tree_out[j], timing_events=events, stream=b.stream)
        return step

    for kind, kname, fname in (("tree_greedy", "argmax_kernel", "tree_greedy_kernel"),
                               ("tree_point", "row_stats_kernel", "tree_point_kernel")):
        spans, kern, wall_us, plain_us = b.timed(tree_step(kind), 2)
        depth = tree_out[0].num_accepted.cpu().numpy()
        first = tr.rows * tr.vocab * (2 if tr.dtype == "bf16" else 4)
        k_med = [float(np.median(k)) for k in kern]
        ach = first / (k_med[0] / 1e6) / 1e9
        res[kind] = {
            "workload": tr.name, "value": round(tr.rows / (float(np.median(spans)) / 1e6), 1),
            "unit": "verified node rows/s", "step_us": pct(spans),
            "kernel_us": [round(x, 2) for x in k_med], "kernel_names": [kname, fname],
            "mean_accepted_depth": round(float(depth.mean()), 4),
            "status": int(tree_out[0].status.cpu().item()),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBPS, 4),
                         "traffic": traffic_from_profile(src_hash, kind), "kernel": kname,
                         "kernel_us": round(k_med[0], 2), "algorithmic_bytes_per_launch": first}}
    del tsets

    # the adaptive draft-length controller after each verify call: one update
    # of B controllers (window 50) from a call's accepted counts, on the same
    # stream; latency-bound (one workgroup).  Its GPU time comes from a
    # replayed graph of updates; the Python call rate is reported too.
    from rejection_sampling_verify_08_amd import DraftLengthController, adapt_params
    h["step"](0, None)                 # outs[0] holds a sampled call's counts again
    ctl = DraftLengthController(inp.num_seqs, adapt_params("window50"), device=b.dev)
    next_k = torch.empty(inp.num_seqs, dtype=torch.int32, device=b.dev)
    next_cu = torch.empty(inp.num_seqs + 1, dtype=torch.int32, device=b.dev)
    for _ in range(20):
        ctl.update(cu, outs[0].num_accepted, next_k=next_k, next_cu=next_cu, stream=b.stream)
    e0, e1 = b.events(2)
    torch.cuda.synchronize()
    e0.record(b.stream)
    n_upd = 200
    for _ in range(n_upd):
        ctl.update(cu, outs[0].num_accepted, next_k=next_k, next_cu=next_cu, stream=b.stream)
    e1.record(b.stream)
    torch.cuda.synchronize()
    launch_us = e0.elapsed_time(e1) * 1e3 / n_upd
    graph, per_graph = torch.cuda.CUDAGraph(), 50
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            ctl.update(cu, outs[0].num_accepted, next_k=next_k, next_cu=next_cu)
    graph.replay()
    torch.cuda.synchronize()
    e0.record(b.stream)
    for _ in range(4):
        graph.replay()
    e1.record(b.stream)
    torch.cuda.synchronize()
    dev_us = e0.elapsed_time(e1) * 1e3 / (4 * per_graph)
    hctl = DraftLengthController(inp.num_seqs, adapt_params("window50"), device="host")
    hcu, hacc = inp.cu_draft, outs[0].num_accepted.cpu().numpy()
    t0 = time.perf_counter()
    for _ in range(n_upd):
        hctl.update(hcu, hacc)
    host_us = (time.perf_counter() - t0) * 1e6 / n_upd
    adapt = {"sequences": inp.num_seqs, "window": 50, "device_us_per_update": round(dev_us, 2),
             "python_launch_us_per_update": round(launch_us, 2),
             "host_us_per_update": round(host_us, 2), "bound": "latency",
             "accept_rate": round(ctl.accept_rate(), 4)}
    return res, adapt


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # the GPU reaches its steady clocks only after ~0.1-0.2 s of this load
    ap.add_argument("--min-warmup-s", type=float, default=0.25,
                    help="warm-up lasts at least this long as well (GPU clocks)")
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--configs", default="1,2,4,5,3",
                    help="named workloads to measure, in order (the headline, 3, last)")
    ap.add_argument("--sets", type=int, default=3, help="rotating device input copies")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle runs on the headline batch (at least --oracle-runs)")
    ap.add_argument("--oracle-runs", type=int, default=3)
    ap.add_argument("--skip-modes", action="store_true",
                    help="time only spec_verify_run (not greedy, point-mass drafts, trees, "
                         "the controller)")
    ap.add_argument("--read-probe-mib", type=int, default=1024,
                    help="size of the streaming-read probe (the practical read ceiling, "
                         "0 = skip)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after timing, run three plain device-to-device copies of this "
                         "many MiB (a known-size reference for HBM byte counters)")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the verify step shards by sequence with "
              "no exchange, and this build runs on a single MI355X (use --gpus 1).",
              file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    b = Bench(a)
    probe = read_probe(b, a.read_probe_mib) if a.read_probe_mib > 0 else None

    order = [int(x) for x in a.configs.split(",") if x.strip()]
    head_idx = HEADLINE if HEADLINE in order else order[-1]
    configs, head = {}, None
    for idx in order:
        rec, keep = b.config(idx, keep=(idx == head_idx))
        configs[str(idx)] = rec
        if keep is not None:
            head = keep

    if a.copy_probe_mib > 0:
        n = a.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=b.dev).fill_(7)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    src_hash = kernel_source_hash()
    hr = configs[str(head_idx)]
    roof = dict(hr["roofline"])
    roof["traffic"] = traffic_from_profile(src_hash) if head_idx == HEADLINE else None
    if probe:
        roof["frac_of_read_probe"] = round(roof["achieved"] / probe["nontemporal_gbps"], 4)
    # the whole step next to the dominant kernel: all of its algorithmic bytes
    # (first pass, re-read, small terms) over the median step
    roof["whole_step_gbps"] = hr["hbm_gbps"]
    roof["whole_step_frac"] = hr["hbm_frac"]
    modes_rec, adapt = (None, None) if a.skip_modes else modes(b, head, src_hash)
    inp = head["inp"]
    hc = hr["oracle"]
    cpu = {"value": hc["verified_rows_per_s"], "unit": "verified rows/s", "cores": hc["cores"],
           "kind": "oracle", "host_cpu": host_cpu(), "host_nproc": os.cpu_count(),
           "sample": f"the full {inp.name} batch ({inp.num_seqs} sequences, {inp.target_rows} "
                     f"target rows), median of {hc['runs']} single-threaded float64 runs "
                     f"({hc['median_s']} s each)"}
    med_ms = hr["step_us"]["p50"] / 1e3
    line = {
        "metric": METRIC, "value": hr["verified_rows_per_s"], "unit": "verified rows/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(med_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": hr["dtype"], "data": "synthetic",
        "config": {"workload": hr["workload"], "B": hr["B"], "gamma": hr["gamma"], "V": hr["V"],
                   "logits": hr["dtype"], "temperature": hr["temperature"],
                   "accumulate": "f64", "input_sets": a.sets,
                   "target_rows": hr["target_rows"], "draft_rows": hr["draft_rows"]},
        "step_us": hr["step_us"], "wall_ms_per_step": round(hr["wall_us_per_step"] / 1e3, 5),
        "unevented_ms_per_step": round(hr["unevented_us_per_step"] / 1e3, 5),
        "unflushed_step_us": hr["unflushed_step_us"],
        "warmup_steps_run": hr["warmup_steps_run"],
        "sequences_per_s": round(hr["B"] / (med_ms / 1e3), 1),
        "all_rows_per_s": round((hr["target_rows"] + hr["draft_rows"]) / (med_ms / 1e3), 1),
        "hbm_gbps": hr["hbm_gbps"], "hbm_frac": hr["hbm_frac"],
        "step_algorithmic_bytes": hr["step_algorithmic_bytes"],
        "kernel_names": hr["kernel_names"], "kernel_us": hr["kernel_us"],
        "mean_accepted": hr["mean_accepted"], "parity": hr["parity"],
        "roofline": roof, "read_probe": probe, "cpu_baseline": cpu,
        "configs": configs, "modes": modes_rec, "adaptive_draft_length": adapt,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(line, ensure_ascii=False), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
