"""ctypes wrapper of the float64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the GPU library; the only common module is the seeded input generator
(`workloads`), which carries no verify-step arithmetic.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "lib", "liboracle.so")
TIE_TOL = 1e-6

F32, BF16 = 0, 1
_DTYPE_CODES = {"f32": F32, "bf16": BF16}


def build(verbose: bool = False) -> str:
    """Compile oracle.c with gcc: -O2, strict IEEE (no contraction, no
    fast-math), no SIMD intrinsics, no threads."""
    os.makedirs(os.path.dirname(LIB_PATH), exist_ok=True)
    cmd = ["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB_PATH, _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.oracle_verify.restype = ctypes.c_int
        lib.oracle_verify.argtypes = [
            ctypes.c_int32, P, P, P, ctypes.c_int64, ctypes.c_int64,
            ctypes.c_int, P, P, ctypes.c_float, ctypes.c_double,
            P, P, P, P, P, P, P, P, P]
        lib.oracle_row_softmax.restype = ctypes.c_int
        lib.oracle_row_softmax.argtypes = [P, ctypes.c_int, ctypes.c_int64,
                                           ctypes.c_float, P]
        lib.oracle_verify_greedy.restype = ctypes.c_int
        lib.oracle_verify_greedy.argtypes = [ctypes.c_int32, P, P, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_int, P, P, P, P]
        lib.oracle_verify_onehot.restype = ctypes.c_int
        lib.oracle_verify_onehot.argtypes = [
            ctypes.c_int32, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, P, P,
            ctypes.c_float, ctypes.c_double, P, P, P, P, P, P, P, P]
        lib.oracle_verify_tree_greedy.restype = ctypes.c_int
        lib.oracle_verify_tree_greedy.argtypes = [ctypes.c_int32, P, P, P, P, ctypes.c_int64,
                                                  ctypes.c_int64, ctypes.c_int, P, P, P]
        lib.oracle_verify_tree_point.restype = ctypes.c_int
        lib.oracle_verify_tree_point.argtypes = [
            ctypes.c_int32, P, P, P, P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, P,
            ctypes.c_float, ctypes.c_double, P, P, P, P, P]
        lib.oracle_overlap_mass.restype = ctypes.c_double
        lib.oracle_overlap_mass.argtypes = [P, P, ctypes.c_int, ctypes.c_int64,
                                            ctypes.c_float]
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(logits: np.ndarray, dtype) -> int:
    if dtype is None:
        dtype = "bf16" if logits.dtype == np.uint16 else "f32"
    code = _DTYPE_CODES[dtype] if isinstance(dtype, str) else int(dtype)
    want = np.float32 if code == F32 else np.uint16
    if logits.dtype != want:
        raise TypeError(f"logits dtype {logits.dtype} does not match {dtype}")
    return code


@dataclasses.dataclass
class OracleResult:
    out_tokens: np.ndarray        # int32 [R_t]
    num_accepted: np.ndarray      # int32 [B]
    p_draft: np.ndarray           # float64 [R_d]
    q_draft: np.ndarray           # float64 [R_d]
    residual_sum: np.ndarray      # float64 [B]
    tie_accept: np.ndarray        # float64 [R_d], |u - r| less r's error bound (>= 0),
                                  # NaN where not evaluated
    tie_final: np.ndarray         # float64 [B], final-draw boundary distance less E (>= 0)
    final_err: np.ndarray         # float64 [B], E: bound on the error of every C_k / S
    flagged: np.ndarray           # int32 [B], nonzero = a decision within the tie window
                                  # widened by its error bound (bit0 accept test, bit1
                                  # final draw, bit2 empty residual, bit3 E > tie / 10)

    def emitted(self, b: int, cu: np.ndarray) -> np.ndarray:
        t0 = int(cu[b]) + b
        return self.out_tokens[t0:t0 + int(self.num_accepted[b]) + 1]


def verify(num_seqs: int, cu_draft, target_logits, draft_logits, draft_tokens,
           uniforms, temperature: float, *, vocab: int | None = None,
           dtype=None, tie_tol: float = TIE_TOL) -> OracleResult:
    """Run the oracle on host arrays in the packed ragged layout.

    target_logits [R_t, ld] / draft_logits [R_d, ld]: float32 or uint16 (bf16
    bits).  `vocab` defaults to the row length."""
    lib = _load()
    tgt = np.ascontiguousarray(target_logits)
    code = _dtype_code(tgt, dtype)
    ld = tgt.shape[1]
    V = ld if vocab is None else int(vocab)
    dft = np.ascontiguousarray(draft_logits)
    if dft.size == 0:
        dft = np.zeros((1, ld), dtype=tgt.dtype)
    cu = np.ascontiguousarray(cu_draft, dtype=np.int32)
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    if tok.size == 0:
        tok = np.zeros(1, dtype=np.int32)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    B = int(num_seqs)
    R_t = tgt.shape[0]
    R_d = max(int(cu[-1]) if B > 0 else 0, 0)
    res = OracleResult(
        out_tokens=np.full(R_t, -7, dtype=np.int32),
        num_accepted=np.zeros(B, dtype=np.int32),
        p_draft=np.zeros(R_d, dtype=np.float64),
        q_draft=np.zeros(R_d, dtype=np.float64),
        residual_sum=np.zeros(B, dtype=np.float64),
        tie_accept=np.full(R_d, np.nan, dtype=np.float64),
        tie_final=np.zeros(B, dtype=np.float64),
        final_err=np.zeros(B, dtype=np.float64),
        flagged=np.zeros(B, dtype=np.int32))
    rc = lib.oracle_verify(
        B, _ptr(cu), _ptr(tgt), _ptr(dft), ld, V, code, _ptr(tok), _ptr(u),
        float(temperature), float(tie_tol), _ptr(res.out_tokens),
        _ptr(res.num_accepted), _ptr(res.p_draft) if R_d else None,
        _ptr(res.q_draft) if R_d else None, _ptr(res.residual_sum),
        _ptr(res.tie_accept) if R_d else None, _ptr(res.tie_final),
        _ptr(res.final_err), _ptr(res.flagged))
    if rc != 0:
        raise ValueError(f"oracle_verify returned {rc}")
    return res


def verify_inputs(inp, **kw) -> OracleResult:
    """Run the oracle on a workloads.VerifyInputs batch."""
    return verify(inp.num_seqs, inp.cu_draft, inp.target_logits,
                  inp.draft_logits, inp.draft_tokens, inp.uniforms,
                  inp.temperature, vocab=inp.vocab, dtype=inp.dtype, **kw)


def row_softmax(logits_row, temperature: float, dtype=None) -> np.ndarray:
    """The oracle's step-1 distribution softmax(l / T) of one row."""
    lib = _load()
    row = np.ascontiguousarray(logits_row)
    code = _dtype_code(row, dtype)
    p = np.empty(row.shape[0], dtype=np.float64)
    rc = lib.oracle_row_softmax(_ptr(row), code, row.shape[0],
                                float(temperature), _ptr(p))
    if rc != 0:
        raise ValueError(f"oracle_row_softmax returned {rc}")
    return p


def overlap_mass(target_row, draft_row, temperature: float, dtype=None) -> float:
    """sum_k min(p_k, q_k) for one target / draft row pair."""
    lib = _load()
    t = np.ascontiguousarray(target_row)
    d = np.ascontiguousarray(draft_row)
    code = _dtype_code(t, dtype)
    return float(lib.oracle_overlap_mass(_ptr(t), _ptr(d), code, t.shape[0],
                                         float(temperature)))


@dataclasses.dataclass
class GreedyResult:
    out_tokens: np.ndarray       # int32 [R_t]
    num_accepted: np.ndarray     # int32 [B]
    argmax: np.ndarray           # int32 [R_t], each target row's argmax

    def emitted(self, b: int, cu: np.ndarray) -> np.ndarray:
        t0 = int(cu[b]) + b
        return self.out_tokens[t0:t0 + int(self.num_accepted[b]) + 1]


def verify_greedy(num_seqs: int, cu_draft, target_logits, draft_tokens, *,
                  vocab: int | None = None, dtype=None) -> GreedyResult:
    """Greedy verification (argmax of each target row, lowest id on ties)."""
    lib = _load()
    tgt = np.ascontiguousarray(target_logits)
    code = _dtype_code(tgt, dtype)
    ld = tgt.shape[1]
    V = ld if vocab is None else int(vocab)
    cu = np.ascontiguousarray(cu_draft, dtype=np.int32)
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    if tok.size == 0:
        tok = np.zeros(1, dtype=np.int32)
    B = int(num_seqs)
    R_t = tgt.shape[0]
    res = GreedyResult(out_tokens=np.full(R_t, -7, np.int32),
                       num_accepted=np.zeros(B, np.int32),
                       argmax=np.full(R_t, -7, np.int32))
    rc = lib.oracle_verify_greedy(B, _ptr(cu), _ptr(tgt), ld, V, code, _ptr(tok),
                                  _ptr(res.out_tokens), _ptr(res.num_accepted),
                                  _ptr(res.argmax))
    if rc != 0:
        raise ValueError(f"oracle_verify_greedy returned {rc}")
    return res


def verify_onehot(num_seqs: int, cu_draft, target_logits, draft_tokens, uniforms,
                  temperature: float, *, vocab: int | None = None, dtype=None,
                  tie_tol: float = TIE_TOL) -> OracleResult:
    """Verification of a deterministic draft (q is the point mass at x)."""
    lib = _load()
    tgt = np.ascontiguousarray(target_logits)
    code = _dtype_code(tgt, dtype)
    ld = tgt.shape[1]
    V = ld if vocab is None else int(vocab)
    cu = np.ascontiguousarray(cu_draft, dtype=np.int32)
    tok = np.ascontiguousarray(draft_tokens, dtype=np.int32)
    if tok.size == 0:
        tok = np.zeros(1, dtype=np.int32)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    B = int(num_seqs)
    R_t = tgt.shape[0]
    R_d = max(int(cu[-1]) if B > 0 else 0, 0)
    res = OracleResult(
        out_tokens=np.full(R_t, -7, dtype=np.int32),
        num_accepted=np.zeros(B, dtype=np.int32),
        p_draft=np.zeros(R_d, dtype=np.float64),
        q_draft=np.ones(R_d, dtype=np.float64),
        residual_sum=np.zeros(B, dtype=np.float64),
        tie_accept=np.full(R_d, np.nan, dtype=np.float64),
        tie_final=np.zeros(B, dtype=np.float64),
        final_err=np.zeros(B, dtype=np.float64),
        flagged=np.zeros(B, dtype=np.int32))
    rc = lib.oracle_verify_onehot(
        B, _ptr(cu), _ptr(tgt), ld, V, code, _ptr(tok), _ptr(u), float(temperature),
        float(tie_tol), _ptr(res.out_tokens), _ptr(res.num_accepted),
        _ptr(res.p_draft) if R_d else None, _ptr(res.residual_sum),
        _ptr(res.tie_accept) if R_d else None, _ptr(res.tie_final), _ptr(res.final_err),
        _ptr(res.flagged))
    if rc != 0:
        raise ValueError(f"oracle_verify_onehot returned {rc}")
    return res


@dataclasses.dataclass
class TreeResult:
    out_tokens: np.ndarray       # int32 [R]: accepted tokens, final token, then -1
    out_path: np.ndarray         # int32 [R]: accepted nodes' local indices, then -1
    num_accepted: np.ndarray     # int32 [B]: accepted depth
    tie: np.ndarray              # float64 [B]: smallest distance of a decision to its threshold
    flagged: np.ndarray          # int32 [B]: 1 accept tie, 2 final-draw tie, 4 empty residual


def _tree_common(cu_nodes, parent, tokens, target_logits, vocab, dtype):
    tgt = np.ascontiguousarray(target_logits)
    code = _dtype_code(tgt, dtype)
    ld = tgt.shape[1]
    V = ld if vocab is None else int(vocab)
    return (tgt, code, ld, V, np.ascontiguousarray(cu_nodes, dtype=np.int32),
            np.ascontiguousarray(parent, dtype=np.int32),
            np.ascontiguousarray(tokens, dtype=np.int32))


def verify_tree_greedy(num_seqs: int, cu_nodes, parent, tokens, target_logits, *,
                       vocab=None, dtype=None) -> TreeResult:
    """Greedy tree verification (see oracle.c)."""
    lib = _load()
    tgt, code, ld, V, cu, par, tok = _tree_common(cu_nodes, parent, tokens, target_logits,
                                                  vocab, dtype)
    B, R = int(num_seqs), tgt.shape[0]
    res = TreeResult(np.full(R, -7, np.int32), np.full(R, -7, np.int32),
                     np.zeros(B, np.int32), np.full(B, np.inf), np.zeros(B, np.int32))
    rc = lib.oracle_verify_tree_greedy(B, _ptr(cu), _ptr(par), _ptr(tok), _ptr(tgt), ld, V,
                                       code, _ptr(res.out_tokens), _ptr(res.out_path),
                                       _ptr(res.num_accepted))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree_greedy returned {rc}")
    return res


def verify_tree_point(num_seqs: int, cu_nodes, parent, tokens, target_logits, uniforms,
                      temperature: float, *, vocab=None, dtype=None,
                      tie_tol: float = TIE_TOL) -> TreeResult:
    """Tree verification of point-mass candidates (see oracle.c)."""
    lib = _load()
    tgt, code, ld, V, cu, par, tok = _tree_common(cu_nodes, parent, tokens, target_logits,
                                                  vocab, dtype)
    u = np.ascontiguousarray(uniforms, dtype=np.float32)
    B, R = int(num_seqs), tgt.shape[0]
    res = TreeResult(np.full(R, -7, np.int32), np.full(R, -7, np.int32),
                     np.zeros(B, np.int32), np.full(B, np.inf), np.zeros(B, np.int32))
    rc = lib.oracle_verify_tree_point(B, _ptr(cu), _ptr(par), _ptr(tok), _ptr(tgt), ld, V,
                                      code, _ptr(u), float(temperature), float(tie_tol),
                                      _ptr(res.out_tokens), _ptr(res.out_path),
                                      _ptr(res.num_accepted), _ptr(res.tie), _ptr(res.flagged))
    if rc != 0:
        raise ValueError(f"oracle_verify_tree_point returned {rc}")
    return res
