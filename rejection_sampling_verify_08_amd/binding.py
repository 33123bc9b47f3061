"""ctypes binding of libspec_verify.so (include/spec_verify.h).

Argument marshalling only: torch tensors supply device memory and the HIP
stream, their raw pointers go through the C ABI, and every step of the verify
runs in the library's gfx950 kernels.  There is no fallback path: without the
built library every entry point raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "lib", "libspec_verify.so")

# keep in step with include/spec_verify.h
OK, EINVAL, EUNSUPPORTED, ECAPACITY, EHIP = 0, -1, -2, -3, -4
F32, BF16 = 0, 1
FLAG_CHECK = 1
DEV_BAD_OFFSETS = 1
DEV_BAD_TOKEN = 2
DEV_BAD_UNIFORM = 4
DEV_BAD_LOGIT = 8
DEV_EMPTY_ROW = 16
DEV_ZERO_Q = 32
DEV_EMPTY_RESIDUAL = 64

EXPORTED = ("spec_verify_create", "spec_verify_query_workspace",
            "spec_verify_workspace_size",
            "spec_verify_num_kernels", "spec_verify_run",
            "spec_verify_run_greedy", "spec_verify_run_point_drafts",
            "spec_verify_destroy", "spec_verify_status_string",
            "spec_verify_last_hip_error")


class SpecVerifyError(RuntimeError):
    def __init__(self, where: str, status: int, hip_error: int = 0):
        lib = _lib if _lib is not None else None
        text = lib.spec_verify_status_string(status).decode() if lib else str(status)
        msg = f"{where}: {text} (status {status})"
        if status == EHIP:
            msg += f", hipError {hip_error}"
        super().__init__(msg)
        self.status = status
        self.hip_error = hip_error


class Args(ctypes.Structure):
    """spec_verify_args, field for field."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_draft_rows", ctypes.c_int64),
        ("cu_draft", ctypes.c_void_p),
        ("target_logits", ctypes.c_void_p),
        ("draft_logits", ctypes.c_void_p),
        ("ld", ctypes.c_int64),
        ("draft_tokens", ctypes.c_void_p),
        ("uniforms", ctypes.c_void_p),
        ("temperature", ctypes.c_float),
        ("out_tokens", ctypes.c_void_p),
        ("out_num_accepted", ctypes.c_void_p),
        ("out_p_draft", ctypes.c_void_p),
        ("out_q_draft", ctypes.c_void_p),
        ("out_residual_sum", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("status", ctypes.c_void_p),
        ("timing_events", ctypes.c_void_p),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libspec_verify.so; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with "
            "`python -m rejection_sampling_verify_08_amd.build` (hipcc, gfx950); "
            "there is no fallback implementation")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.spec_verify_create.restype = ctypes.c_int
    lib.spec_verify_create.argtypes = [ctypes.POINTER(P), ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_int32, ctypes.c_int64,
                                       ctypes.c_uint32, ctypes.POINTER(ctypes.c_size_t)]
    lib.spec_verify_query_workspace.restype = ctypes.c_int
    lib.spec_verify_query_workspace.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.POINTER(ctypes.c_size_t)]
    lib.spec_verify_workspace_size.restype = ctypes.c_size_t
    lib.spec_verify_workspace_size.argtypes = [P]
    lib.spec_verify_num_kernels.restype = ctypes.c_int
    lib.spec_verify_num_kernels.argtypes = [P]
    for name in ("spec_verify_run", "spec_verify_run_greedy", "spec_verify_run_point_drafts"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P, ctypes.POINTER(Args), P]
    lib.spec_verify_destroy.restype = ctypes.c_int
    lib.spec_verify_destroy.argtypes = [P]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_status_string.argtypes = [ctypes.c_int]
    lib.spec_verify_last_hip_error.restype = ctypes.c_int
    lib.spec_verify_last_hip_error.argtypes = []
    _lib = lib
    return lib


@dataclasses.dataclass
class VerifyOutput:
    out_tokens: "torch.Tensor"          # int32 [R_t]
    num_accepted: "torch.Tensor"        # int32 [B]
    p_draft: Optional["torch.Tensor"]   # float32 [R_d]
    q_draft: Optional["torch.Tensor"]   # float32 [R_d]
    residual_sum: Optional["torch.Tensor"]  # float32 [B]
    status: Optional["torch.Tensor"]    # uint32-as-int32 [1]


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


class SpecVerifier:
    """One context of the verify step for a vocabulary size and logit dtype.

    Owns the context (host state) and a workspace tensor on `device`.
    """

    def __init__(self, vocab: int, dtype="bf16", max_seqs: int = 1,
                 max_draft_rows: int = 0, device=None, check: bool = False):
        import torch
        self._torch = torch
        lib = load_library()
        if isinstance(dtype, str):
            code = {"f32": F32, "float32": F32, "bf16": BF16, "bfloat16": BF16}[dtype]
        elif dtype in (torch.float32,):
            code = F32
        elif dtype in (torch.bfloat16,):
            code = BF16
        else:
            code = int(dtype)
        self.dtype_code = code
        self.torch_dtype = torch.bfloat16 if code == BF16 else torch.float32
        self.vocab = int(vocab)
        dev = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        self.device = dev
        ctx = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        with torch.cuda.device(dev):
            st = lib.spec_verify_create(ctypes.byref(ctx), dev.index or 0, self.vocab,
                                        code, int(max_seqs), int(max_draft_rows),
                                        FLAG_CHECK if check else 0, ctypes.byref(ws))
        if st != OK:
            raise SpecVerifyError("spec_verify_create", st, lib.spec_verify_last_hip_error())
        self._ctx = ctx
        self.max_seqs = int(max_seqs)
        self.max_draft_rows = int(max_draft_rows)
        self.workspace = torch.empty(max(int(ws.value), 256), dtype=torch.uint8, device=dev)
        self.num_kernels = lib.spec_verify_num_kernels(ctx)

    def close(self):
        if getattr(self, "_ctx", None):
            load_library().spec_verify_destroy(self._ctx)
            self._ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def allocate_outputs(self, num_seqs: int, draft_rows: int, *, probs: bool = True,
                         residual: bool = True, status: bool = True) -> VerifyOutput:
        torch = self._torch
        dev = self.device
        R_t = draft_rows + num_seqs
        return VerifyOutput(
            out_tokens=torch.empty(R_t, dtype=torch.int32, device=dev),
            num_accepted=torch.empty(num_seqs, dtype=torch.int32, device=dev),
            p_draft=torch.empty(draft_rows, dtype=torch.float32, device=dev) if probs else None,
            q_draft=torch.empty(draft_rows, dtype=torch.float32, device=dev) if probs else None,
            residual_sum=torch.empty(num_seqs, dtype=torch.float32, device=dev) if residual else None,
            status=torch.zeros(1, dtype=torch.int32, device=dev) if status else None)

    def __call__(self, cu_draft, target_logits, draft_logits, draft_tokens, uniforms,
                 temperature: float, *, num_seqs: Optional[int] = None,
                 total_draft_rows: Optional[int] = None, out: Optional[VerifyOutput] = None,
                 timing_events: Optional[Sequence] = None, stream=None) -> VerifyOutput:
        """Enqueue one verify step (spec_verify_run) on `stream` (default:
        torch's current stream).

        num_seqs / total_draft_rows default to the tensor shapes
        (cu_draft has B+1 entries, draft_logits has R_d rows).  Nothing is
        synchronised; `out` (see allocate_outputs) is filled asynchronously.
        """
        return self._run("spec_verify_run", cu_draft, target_logits, draft_logits,
                         draft_tokens, uniforms, temperature, num_seqs, total_draft_rows,
                         out, timing_events, stream)

    def point_drafts(self, cu_draft, target_logits, draft_tokens, uniforms,
                     temperature: float, *, num_seqs: Optional[int] = None,
                     out: Optional[VerifyOutput] = None,
                     timing_events: Optional[Sequence] = None, stream=None) -> VerifyOutput:
        """Verify deterministic drafts (spec_verify_run_point_drafts): the
        draft distribution is the point mass at each proposed token; no draft
        logits.  R_d = draft_tokens.numel()."""
        return self._run("spec_verify_run_point_drafts", cu_draft, target_logits, None,
                         draft_tokens, uniforms, temperature, num_seqs,
                         int(draft_tokens.numel()), out, timing_events, stream)

    def greedy(self, cu_draft, target_logits, draft_tokens, *,
               num_seqs: Optional[int] = None, out: Optional[VerifyOutput] = None,
               timing_events: Optional[Sequence] = None, stream=None) -> VerifyOutput:
        """Greedy verification (spec_verify_run_greedy): argmax of each
        target row, lowest id on ties.  Only out_tokens, num_accepted and
        status are written.  R_d = draft_tokens.numel()."""
        return self._run("spec_verify_run_greedy", cu_draft, target_logits, None,
                         draft_tokens, None, 1.0, num_seqs, int(draft_tokens.numel()),
                         out, timing_events, stream)

    def _run(self, entry, cu_draft, target_logits, draft_logits, draft_tokens, uniforms,
             temperature, num_seqs, total_draft_rows, out, timing_events, stream):
        torch = self._torch
        B = int(cu_draft.shape[0]) - 1 if num_seqs is None else int(num_seqs)
        R_d = int(draft_logits.shape[0]) if (total_draft_rows is None and draft_logits is not None) \
            else int(total_draft_rows or 0)
        if out is None:
            out = self.allocate_outputs(B, R_d)
        for name, t in (("target_logits", target_logits), ("draft_logits", draft_logits)):
            if t is not None and (t.dtype != self.torch_dtype or t.stride(-1) != 1):
                raise ValueError(f"{name} must be {self.torch_dtype} with unit column stride")
        ld = int(target_logits.stride(0)) if target_logits.dim() == 2 else self.vocab
        if draft_logits is not None and draft_logits.dim() == 2 and draft_logits.shape[0] > 0 \
                and int(draft_logits.stride(0)) != ld:
            raise ValueError("target and draft logits must share one row pitch")
        for name, t, dt in (("cu_draft", cu_draft, torch.int32),
                            ("draft_tokens", draft_tokens, torch.int32),
                            ("uniforms", uniforms, torch.float32)):
            if t is not None and (t.dtype != dt or not t.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous {dt} tensor")
        events = None
        if timing_events is not None:
            arr = (ctypes.c_void_p * len(timing_events))(
                *[ctypes.c_void_p(int(e.cuda_event)) if hasattr(e, "cuda_event") else e
                  for e in timing_events])
            events = arr
        a = Args(
            num_seqs=B, total_draft_rows=R_d, cu_draft=_ptr(cu_draft),
            target_logits=_ptr(target_logits),
            draft_logits=_ptr(draft_logits) if (draft_logits is not None and R_d > 0) else None,
            ld=ld, draft_tokens=_ptr(draft_tokens) if R_d > 0 else None,
            uniforms=_ptr(uniforms), temperature=float(temperature),
            out_tokens=_ptr(out.out_tokens), out_num_accepted=_ptr(out.num_accepted),
            out_p_draft=_ptr(out.p_draft), out_q_draft=_ptr(out.q_draft),
            out_residual_sum=_ptr(out.residual_sum), workspace=_ptr(self.workspace),
            workspace_bytes=int(self.workspace.numel()), status=_ptr(out.status),
            timing_events=ctypes.cast(events, ctypes.c_void_p) if events is not None else None)
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        lib = load_library()
        st = getattr(lib, entry)(self._ctx, ctypes.byref(a), ctypes.c_void_p(handle))
        if st != OK:
            raise SpecVerifyError(entry, st, lib.spec_verify_last_hip_error())
        self._keepalive = events
        return out


def verify(cu_draft, target_logits, draft_logits, draft_tokens, uniforms,
           temperature: float, *, vocab: Optional[int] = None, check: bool = False):
    """One-shot convenience wrapper: builds a context sized for these tensors."""
    V = int(target_logits.shape[1]) if vocab is None else int(vocab)
    B = int(cu_draft.shape[0]) - 1
    R_d = int(draft_logits.shape[0]) if draft_logits is not None else 0
    sv = SpecVerifier(V, target_logits.dtype, max_seqs=max(B, 1),
                      max_draft_rows=R_d, device=target_logits.device, check=check)
    return sv(cu_draft, target_logits, draft_logits, draft_tokens, uniforms, temperature)
