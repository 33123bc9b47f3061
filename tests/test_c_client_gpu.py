"""The C ABI from a plain C program (tests/c_client/verify_client.c: HIP
runtime allocations, spec_verify_create / run / destroy, no Python or
PyTorch), run as a child process; its outputs meet the parity rule against
the oracle."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import HostOutput, compare, log

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "verify_client")


def _write_input(path, inp):
    B, R_d, V = inp.num_seqs, inp.draft_rows, inp.vocab
    dt = 1 if inp.dtype == W.BF16 else 0
    with open(path, "wb") as f:
        f.write(b"SVC1")
        f.write(np.int32(B).tobytes() + np.int64(R_d).tobytes() + np.int64(V).tobytes())
        f.write(np.int32(dt).tobytes() + np.float32(inp.temperature).tobytes())
        f.write(np.ascontiguousarray(inp.cu_draft, np.int32).tobytes())
        f.write(np.ascontiguousarray(inp.target_logits).tobytes())
        f.write(np.ascontiguousarray(inp.draft_logits).tobytes())
        f.write(np.ascontiguousarray(inp.draft_tokens, np.int32).tobytes())
        f.write(np.ascontiguousarray(inp.uniforms, np.float32).tobytes())


def _read_output(path, inp) -> HostOutput:
    B, R_d, R_t = inp.num_seqs, inp.draft_rows, inp.target_rows
    raw = open(path, "rb").read()
    assert raw[:4] == b"SVO1"
    off = 4

    def take(n, dt):
        nonlocal off
        a = np.frombuffer(raw, dtype=dt, count=n, offset=off)
        off += n * np.dtype(dt).itemsize
        return a.copy()

    tok, n = take(R_t, np.int32), take(B, np.int32)
    p, q, r = take(R_d, np.float32), take(R_d, np.float32), take(B, np.float32)
    st = int(take(1, np.uint32)[0])
    assert off == len(raw)
    return HostOutput(tok, n, p.astype(np.float64), q.astype(np.float64), r.astype(np.float64), st)


@pytest.mark.parametrize("cfg", [1, 2])
def test_c_client_matches_the_oracle(cfg, tmp_path):
    assert os.path.exists(CLIENT), "tests/c_client/verify_client is built by __graft_entry__.build()"
    inp = W.config(cfg, seed=70 + cfg) if cfg == 1 else W.config(2, seed=72, num_seqs=24)
    fin, fout = tmp_path / "in.bin", tmp_path / "out.bin"
    _write_input(fin, inp)
    log(f"[c client] {inp.name}")
    res = subprocess.run([CLIENT, str(fin), str(fout)], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 0, res.stderr
    gpu = _read_output(fout, inp)
    compare(inp, gpu, oracle.verify_inputs(inp), label=f"C client cfg {cfg}")
    assert gpu.status == 0
