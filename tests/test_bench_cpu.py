"""bench.py's host-side contract, without a GPU: the refusal of more than one
GPU, the kernel-source identity that gates the stored HBM counters, and the
algorithmic byte count the roofline divides by."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line


def test_kernel_hash_ignores_comments_only(tmp_path, monkeypatch):
    code = "__global__ void k(float* x) {\n  x[0] = 1.0f;   // store\n}\n"
    a, b, c = tmp_path / "a.hpp", tmp_path / "b.hpp", tmp_path / "c.hpp"
    a.write_text("// version one\n" + code)
    b.write_text("// version two, reworded\n\n" + code.replace("// store", "// the store"))
    c.write_text("// version one\n" + code.replace("1.0f", "2.0f"))
    hashes = []
    for f in (a, b, c):
        monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(f)])
        hashes.append(bench.kernel_source_hash())
    assert hashes[0] == hashes[1]
    assert hashes[0] != hashes[2]


def test_stored_traffic_needs_the_matching_kernel_hash(tmp_path, monkeypatch):
    f = tmp_path / "pmc.json"
    f.write_text(json.dumps({"kernel_source_hash": "0123456789abcdef",
                             "hbm_bytes_per_launch": {"sampled": 558282410, "greedy": 295583148}}))
    monkeypatch.setattr(bench, "PMC_FILE", str(f))
    assert bench.traffic_from_profile("0123456789abcdef") == 558282410
    assert bench.traffic_from_profile("0123456789abcdef", "greedy") == 295583148
    assert bench.traffic_from_profile("fedcba9876543210") is None
    monkeypatch.setattr(bench, "PMC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_from_profile("0123456789abcdef") is None


def test_committed_counters_carry_a_kernel_hash():
    rec = json.load(open(bench.PMC_FILE))
    assert len(rec["kernel_source_hash"]) == 16
    assert rec["hbm_bytes_per_launch"]["sampled"] > 0


@pytest.mark.parametrize("mode", ["sampled", "point", "greedy"])
def test_algorithmic_bytes(mode):
    """The counts from the inputs' own arrays: every logit row once, then per
    sequence the rows its final draw reads again."""
    inp = W.config(3, num_seqs=6, vocab=4096)
    B = inp.num_seqs
    acc = np.minimum(np.arange(B), inp.gammas)           # sequence b accepts b drafts
    first, again, io = bench.algorithmic_bytes(inp, acc, mode)
    row = inp.target_logits.nbytes // inp.target_rows    # bytes of one logit row
    ints_in = inp.draft_tokens.nbytes + inp.cu_draft.nbytes
    ints_out = 4 * inp.target_rows + 4 * B                # output tokens, accepted counts
    if mode == "greedy":
        assert first == inp.target_logits.nbytes and again == 0
        assert io == ints_in + ints_out
        return
    probs_out = 8 * inp.draft_rows + 4 * B               # p(x), q(x) per draft; residual sums
    assert io == ints_in + ints_out + inp.uniforms.nbytes + probs_out
    if mode == "point":
        assert first == inp.target_logits.nbytes
        assert again == B * row                          # one target row per final draw
        return
    assert first == inp.target_logits.nbytes + inp.draft_logits.nbytes
    reread = sum(2 if acc[b] < inp.gammas[b] else 1 for b in range(B))
    assert again == reread * row                         # a rejection's pair, or a bonus row
