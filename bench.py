#!/usr/bin/env python3
"""Benchmark of the batched speculative-decoding verify step on one MI355X.

One step = one spec_verify_run call (row statistics of every target and draft
row, accept tests, first-rejection stop, residual / bonus draw) over one batch
of the headline workload: B=128 sequences, gamma=8, V=128256, bf16 logits,
T=1.0, heavy-tailed target logits with draft noise giving alpha ~ 0.6.
Inputs are resident in HBM before timing; `--sets` copies rotate so no step
reads logits the previous step left in the 256 MB Infinity Cache.

Prints one JSON line: verified rows/s (value), whole-step HBM GB/s, the
roofline of the dominant kernel (the row-statistics pass, HBM-bound; its
duration from HIP events that are its dispatch's own start and stop), the
per-step GPU time's p10/p50/p90, the step time without rotating the inputs
("unflushed"), the practical read ceiling measured by a streaming-read probe
over 1 GiB with the row pass's load pattern, and the float64 CPU oracle
timed on this host as a reported baseline.

The same line carries, under "modes", the same measurement for the two other
entry points on the same batch with deterministic drafts (each draft token
the first maximum of its draft row): greedy verification
(spec_verify_run_greedy) and point-mass-draft verification
(spec_verify_run_point_drafts).
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
    rocprofv3 counter summary, or None when it is missing, was taken on
    another workload, or the kernels changed since."""
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


def cpu_baseline(inp, budget_s: float):
    import oracle
    oracle._load()
    t0 = time.perf_counter()
    runs = 0
    while True:
        oracle.verify_inputs(inp)
        runs += 1
        el = time.perf_counter() - t0
        if el >= budget_s or runs >= 50:
            break
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": inp.target_rows * runs / el, "unit": "verified rows/s", "cores": 1,
            "kind": "oracle", "host_cpu": model, "host_nproc": os.cpu_count(),
            "sample": f"the full headline batch ({inp.num_seqs} sequences, {inp.target_rows} "
                      f"target rows), {runs} run(s) in {el:.1f} s, single-threaded float64 C"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    # the GPU reaches its steady clocks only after ~0.1-0.2 s of this load
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--config", type=int, default=3, help="named workload 1..5")
    ap.add_argument("--sets", type=int, default=3, help="rotating device input copies")
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--event-every", type=int, default=10,
                    help="record per-kernel timing events on every n-th timed step")
    ap.add_argument("--skip-modes", action="store_true",
                    help="time only spec_verify_run (not the greedy and point-draft entry points)")
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

    import numpy as np
    import torch
    import workloads as W
    from rejection_sampling_verify_08_amd import SpecVerifier
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)

    t_gen = time.perf_counter()
    inp = W.config(a.config)
    print(f"[bench] generated {inp.name} in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr,
          flush=True)
    tdt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32

    def torch_rows(arr, dtype):
        if dtype == "bf16":
            return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(arr).to(dev)

    def up(arr):
        return torch_rows(arr, inp.dtype)

    host_t, host_d = up(inp.target_logits), up(inp.draft_logits)
    sets = []
    for s in range(max(1, a.sets)):
        t = torch.empty_like(host_t)
        d = torch.empty_like(host_d)
        t.copy_(host_t)
        d.copy_(host_d)
        sets.append((t, d))
    del host_t, host_d
    cu = torch.from_numpy(inp.cu_draft).to(dev)
    tok = torch.from_numpy(inp.draft_tokens).to(dev)
    uni = torch.from_numpy(inp.uniforms).to(dev)
    sv = SpecVerifier(inp.vocab, tdt, max_seqs=inp.num_seqs, max_draft_rows=inp.draft_rows)
    outs = [sv.allocate_outputs(inp.num_seqs, inp.draft_rows) for _ in sets]
    nk = sv.num_kernels
    stream = torch.cuda.current_stream(dev)

    def make_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)          # creates the underlying hipEvent
        return evs

    def timed(call):
        """Warm up, then time a.steps calls.  Every `event_every`-th timed
        step passes timing events to the library, which uses them as the
        start / stop events of each kernel's own dispatch."""
        for i in range(a.warmup):
            call(i, None)
        steps_ev = list(range(0, a.steps, a.event_every))
        ev = {i: make_events(2 * nk) for i in steps_ev}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(a.steps):
            call(i, ev.get(i))
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        ms = (t1 - t0) * 1e3 / a.steps
        k_ms = [[ev[i][2 * k].elapsed_time(ev[i][2 * k + 1]) for i in steps_ev]
                for k in range(nk)]
        # per-step GPU span: first kernel's start to the last kernel's stop
        span = [ev[i][0].elapsed_time(ev[i][2 * nk - 1]) for i in steps_ev]
        pct = {"p10": float(np.percentile(span, 10)), "p50": float(np.percentile(span, 50)),
               "p90": float(np.percentile(span, 90))}
        timed.last_pct = {k: round(v * 1e3, 2) for k, v in pct.items()}
        timed.last_kernel_p50 = [round(float(np.percentile(x, 50)) * 1e3, 2) for x in k_ms]
        return ms, [sum(x) / len(x) for x in k_ms]

    def sampled_step(i, events):
        t, d = sets[i % len(sets)]
        sv(cu, t, d, tok, uni, inp.temperature, out=outs[i % len(sets)], stream=stream,
           timing_events=events)

    ms_step, k_avg = timed(sampled_step)
    step_pct, k_p50 = timed.last_pct, timed.last_kernel_p50

    # the same call without rotating the inputs: part of each step's rows can
    # then still be in the 256 MB Infinity Cache from the step before
    def unflushed_step(i, events):
        t, d = sets[0]
        sv(cu, t, d, tok, uni, inp.temperature, out=outs[0], stream=stream, timing_events=events)

    ms_unflushed, _ = timed(unflushed_step)

    # the practical read ceiling: one streaming read of a buffer far larger
    # than the Infinity Cache, with the row pass's load pattern
    probe = None
    if a.read_probe_mib > 0:
        from rejection_sampling_verify_08_amd.binding import read_probe
        nb = a.read_probe_mib << 20
        buf = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(7)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        probe = {"bytes": nb, "kernel": "read_probe_kernel",
                 "loads": "16-byte, one 1 KB span per wave instruction (the row pass's pattern)"}
        for nt, key in ((True, "nontemporal_gbps"), (False, "plain_gbps")):
            for _ in range(3):
                read_probe(buf, sink, nontemporal=nt, stream=stream)
            runs = [make_events(2) for _ in range(10)]
            torch.cuda.synchronize()
            for e in runs:
                read_probe(buf, sink, nontemporal=nt, stream=stream, events=e)
            torch.cuda.synchronize()
            gbps = sorted(nb / (e[0].elapsed_time(e[1]) / 1e3) / 1e9 for e in runs)
            probe[key] = round(float(np.median(gbps)), 1)
            probe[key.replace("gbps", "best_gbps")] = round(gbps[-1], 1)
        del buf

    if a.copy_probe_mib > 0:
        n = a.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(7)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    num_acc = outs[0].num_accepted.cpu().numpy()
    status = int(outs[0].status.cpu().item())
    first, reread, small = algorithmic_bytes(inp, num_acc)
    step_bytes = first + reread + small
    value = inp.target_rows / (ms_step / 1e3)
    hbm = step_bytes / (ms_step / 1e3) / 1e9
    # the dominant kernel is the row-statistics pass: one read of every row
    achieved = first / (k_avg[0] / 1e3) / 1e9
    src_hash = kernel_source_hash()
    traffic = traffic_from_profile(src_hash) if a.config == 3 else None
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
            "traffic": traffic, "kernel": "row_stats_kernel",
            "kernel_avg_us": round(k_avg[0] * 1e3, 2),
            "algorithmic_bytes_per_launch": first}
    if probe:
        roof["frac_of_read_probe"] = round(achieved / probe["nontemporal_gbps"], 4)

    # the other two entry points on the same target rows, deterministic drafts
    modes = {}
    if not a.skip_modes:
        det = W.with_deterministic_drafts(inp)
        tok_det = torch.from_numpy(det.draft_tokens).to(dev)

        def greedy_step(i, events):
            t, _ = sets[i % len(sets)]
            sv.greedy(cu, t, tok_det, out=outs[i % len(sets)], stream=stream,
                      timing_events=events)

        def point_step(i, events):
            t, _ = sets[i % len(sets)]
            sv.point_drafts(cu, t, tok_det, uni, inp.temperature, out=outs[i % len(sets)],
                            stream=stream, timing_events=events)

        for name, step, kname in (("greedy", greedy_step, "argmax_kernel"),
                                  ("point_drafts", point_step, "row_stats_kernel")):
            m_ms, m_k = timed(step)
            m_acc = outs[0].num_accepted.cpu().numpy()
            m_first, m_reread, m_small = algorithmic_bytes(
                det, m_acc, "greedy" if name == "greedy" else "point")
            m_bytes = m_first + m_reread + m_small
            m_ach = m_first / (m_k[0] / 1e3) / 1e9
            modes[name] = {
                "value": round(inp.target_rows / (m_ms / 1e3), 1), "unit": "verified rows/s",
                "ms_per_step": round(m_ms, 5),
                "hbm_gbps": round(m_bytes / (m_ms / 1e3) / 1e9, 1),
                "step_algorithmic_bytes": m_bytes,
                "kernel_avg_us": [round(x * 1e3, 2) for x in m_k],
                "kernel_names": [kname, "greedy_finish_kernel" if name == "greedy"
                                 else "finish_kernel"],
                "mean_accepted": round(float(m_acc.mean()), 4),
                "status": int(outs[0].status.cpu().item()),
                "roofline": {"bound": "hbm", "achieved": round(m_ach, 1),
                             "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                             "frac": round(m_ach / PEAK_HBM_GBPS, 4),
                             "traffic": traffic_from_profile(src_hash, name) if a.config == 3 else None,
                             "kernel": kname, "kernel_avg_us": round(m_k[0] * 1e3, 2),
                             "algorithmic_bytes_per_launch": m_first},
            }

    # tree verification on the named tree workload (128 trees of 17 nodes,
    # 2176 rows: as many as the chain batch above)
    if not a.skip_modes and a.config == 3:
        tr = W.tree_config()
        t_tree = torch_rows(tr.target_logits, inp.dtype)
        tsets = [t_tree] + [t_tree.clone() for _ in range(max(1, a.sets) - 1)]
        dvc = lambda arr: torch.from_numpy(np.ascontiguousarray(arr)).to(dev)
        tcu, tpar, ttok, tuni = dvc(tr.cu_nodes), dvc(tr.parent), dvc(tr.tokens), dvc(tr.uniforms)
        tree_out = [None] * len(tsets)

        def tree_step(kind):
            def step(i, events):
                j = i % len(tsets)
                if kind == "tree_greedy":
                    tree_out[j] = sv.tree_greedy(tcu, tpar, ttok, tsets[j], out=tree_out[j],
                                                 timing_events=events, stream=stream)
                else:
                    tree_out[j] = sv.tree_point(tcu, tpar, ttok, tsets[j], tuni, tr.temperature,
                                                out=tree_out[j], timing_events=events,
                                                stream=stream)
            return step

        for kind, kname, fname in (("tree_greedy", "argmax_kernel", "tree_greedy_kernel"),
                                   ("tree_point", "row_stats_kernel", "tree_point_kernel")):
            m_ms, m_k = timed(tree_step(kind))
            depth = tree_out[0].num_accepted.cpu().numpy()
            m_first = tr.rows * tr.vocab * (2 if tr.dtype == "bf16" else 4)
            m_ach = m_first / (m_k[0] / 1e3) / 1e9
            modes[kind] = {
                "workload": tr.name,
                "value": round(tr.rows / (m_ms / 1e3), 1), "unit": "verified node rows/s",
                "ms_per_step": round(m_ms, 5),
                "kernel_avg_us": [round(x * 1e3, 2) for x in m_k],
                "kernel_names": [kname, fname],
                "mean_accepted_depth": round(float(depth.mean()), 4),
                "status": int(tree_out[0].status.cpu().item()),
                "roofline": {"bound": "hbm", "achieved": round(m_ach, 1), "peak": PEAK_HBM_GBPS,
                             "unit": "GB/s", "frac": round(m_ach / PEAK_HBM_GBPS, 4),
                             "traffic": traffic_from_profile(src_hash, kind),
                             "kernel": kname, "kernel_avg_us": round(m_k[0] * 1e3, 2),
                             "algorithmic_bytes_per_launch": m_first},
            }
        del tsets

    # the adaptive draft-length controller after each verify call: one
    # update of B controllers (window 50) from the call's accepted counts,
    # enqueued on the same stream; latency-bound (one workgroup).  Its GPU
    # time comes from replaying a captured graph of updates (a Python call
    # per update costs more than the kernel); the Python rate is reported too.
    adapt = None
    if not a.skip_modes:
        from rejection_sampling_verify_08_amd import DraftLengthController, adapt_params
        sampled_step(0, None)          # outs[0] holds a sampled call's counts again
        ctl = DraftLengthController(inp.num_seqs, adapt_params("window50"), device=dev)
        next_k = torch.empty(inp.num_seqs, dtype=torch.int32, device=dev)
        next_cu = torch.empty(inp.num_seqs + 1, dtype=torch.int32, device=dev)
        for _ in range(20):
            ctl.update(cu, outs[0].num_accepted, next_k=next_k, next_cu=next_cu, stream=stream)
        e0, e1 = make_events(2)
        torch.cuda.synchronize()
        e0.record(stream)
        n_upd = 200
        for _ in range(n_upd):
            ctl.update(cu, outs[0].num_accepted, next_k=next_k, next_cu=next_cu, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        launch_us = e0.elapsed_time(e1) * 1e3 / n_upd
        graph, per_graph = torch.cuda.CUDAGraph(), 50
        with torch.cuda.graph(graph):
            for _ in range(per_graph):
                ctl.update(cu, outs[0].num_accepted, next_k=next_k, next_cu=next_cu)
        graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(4):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        dev_us = e0.elapsed_time(e1) * 1e3 / (4 * per_graph)
        hctl = DraftLengthController(inp.num_seqs, adapt_params("window50"), device="host")
        hcu, hacc = inp.cu_draft, outs[0].num_accepted.cpu().numpy()
        t0 = time.perf_counter()
        for _ in range(n_upd):
            hctl.update(hcu, hacc)
        host_us = (time.perf_counter() - t0) * 1e6 / n_upd
        adapt = {"sequences": inp.num_seqs, "window": 50,
                 "device_us_per_update": round(dev_us, 2),
                 "python_launch_us_per_update": round(launch_us, 2),
                 "host_us_per_update": round(host_us, 2),
                 "bound": "latency", "accept_rate": round(ctl.accept_rate(), 4)}

    cpu = None
    if a.cpu_budget > 0:
        cpu = cpu_baseline(inp, a.cpu_budget)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "verified rows/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": inp.name, "B": inp.num_seqs, "gamma": 8 if a.config == 3 else None,
                   "V": inp.vocab, "logits": inp.dtype, "temperature": inp.temperature,
                   "accumulate": "f64", "input_sets": len(sets),
                   "target_rows": inp.target_rows, "draft_rows": inp.draft_rows},
        "sequences_per_s": round(inp.num_seqs / (ms_step / 1e3), 1),
        "all_rows_per_s": round((inp.target_rows + inp.draft_rows) / (ms_step / 1e3), 1),
        "hbm_gbps": round(hbm, 1), "hbm_frac": round(hbm / PEAK_HBM_GBPS, 4),
        "step_algorithmic_bytes": step_bytes,
        "kernel_avg_us": [round(x * 1e3, 2) for x in k_avg],
        "kernel_p50_us": k_p50,
        "kernel_names": ["row_stats_kernel", "finish_kernel"][:nk],
        "step_gpu_us": step_pct,
        "unflushed_ms_per_step": round(ms_unflushed, 5),
        "mean_accepted": round(float(num_acc.mean()), 4), "status": status,
        "roofline": roof, "read_probe": probe, "cpu_baseline": cpu,
        "modes": modes or None,
        "adaptive_draft_length": adapt,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(line, ensure_ascii=False), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
