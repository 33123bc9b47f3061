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
DEV_BAD_TREE = 128
MAX_TREE_NODES, MAX_TREE_CHILDREN = 1024, 64

EXPORTED = ("spec_verify_create", "spec_verify_query_workspace",
            "spec_verify_workspace_size",
            "spec_verify_num_kernels", "spec_verify_run", "spec_verify_run_static",
            "spec_verify_run_greedy", "spec_verify_run_point_drafts",
            "spec_verify_tree_run_greedy", "spec_verify_tree_run_point",
            "spec_verify_destroy", "spec_verify_status_string",
            "spec_verify_last_hip_error", "spec_verify_read_probe",
            "spec_verify_adapt_preset", "spec_verify_adapt_state_bytes",
            "spec_verify_adapt_reset", "spec_verify_adapt_update")

# keep in step with include/spec_verify_adapt.h
ADAPT_HOST = -1
ADAPT_PRESETS = {"window50": 0, "last10": 1}
ADAPT_BAD_SLOT, ADAPT_BAD_COUNTS = 1, 2


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


class TreeArgs(ctypes.Structure):
    """spec_verify_tree_args, field for field."""
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_nodes", ctypes.c_int64),
        ("cu_nodes", ctypes.c_void_p),
        ("parent", ctypes.c_void_p),
        ("tokens", ctypes.c_void_p),
        ("target_logits", ctypes.c_void_p),
        ("ld", ctypes.c_int64),
        ("uniforms", ctypes.c_void_p),
        ("temperature", ctypes.c_float),
        ("out_tokens", ctypes.c_void_p),
        ("out_path", ctypes.c_void_p),
        ("out_num_accepted", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("status", ctypes.c_void_p),
        ("timing_events", ctypes.c_void_p),
    ]


class AdaptParams(ctypes.Structure):
    """spec_verify_adapt_params, field for field."""
    _fields_ = [
        ("k_min", ctypes.c_int32),
        ("k_max", ctypes.c_int32),
        ("k_init", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("min_history", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("up", ctypes.c_double),
        ("down", ctypes.c_double),
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
    for name in ("spec_verify_run", "spec_verify_run_static", "spec_verify_run_greedy",
                 "spec_verify_run_point_drafts"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P, ctypes.POINTER(Args), P]
    for name in ("spec_verify_tree_run_greedy", "spec_verify_tree_run_point"):
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [P, ctypes.POINTER(TreeArgs), P]
    AP = ctypes.POINTER(AdaptParams)
    lib.spec_verify_adapt_preset.restype = ctypes.c_int
    lib.spec_verify_adapt_preset.argtypes = [ctypes.c_int, AP]
    lib.spec_verify_adapt_state_bytes.restype = ctypes.c_int
    lib.spec_verify_adapt_state_bytes.argtypes = [AP, ctypes.c_int64,
                                                  ctypes.POINTER(ctypes.c_size_t)]
    lib.spec_verify_adapt_reset.restype = ctypes.c_int
    lib.spec_verify_adapt_reset.argtypes = [AP, ctypes.c_int64, P, ctypes.c_size_t,
                                            ctypes.c_int64, P, ctypes.c_int, P]
    lib.spec_verify_adapt_update.restype = ctypes.c_int
    lib.spec_verify_adapt_update.argtypes = [AP, ctypes.c_int64, P, ctypes.c_size_t,
                                             ctypes.c_int32, P, P, P, P, P, P, P,
                                             ctypes.c_int, P]
    lib.spec_verify_destroy.restype = ctypes.c_int
    lib.spec_verify_destroy.argtypes = [P]
    lib.spec_verify_status_string.restype = ctypes.c_char_p
    lib.spec_verify_status_string.argtypes = [ctypes.c_int]
    lib.spec_verify_last_hip_error.restype = ctypes.c_int
    lib.spec_verify_last_hip_error.argtypes = []
    lib.spec_verify_read_probe.restype = ctypes.c_int
    lib.spec_verify_read_probe.argtypes = [P, ctypes.c_size_t, ctypes.c_int, P, P, P, P]
    _lib = lib
    return lib


@dataclasses.dataclass
class TreeOutput:
    out_tokens: "torch.Tensor"          # int32 [R]
    out_path: "torch.Tensor"            # int32 [R]
    num_accepted: "torch.Tensor"        # int32 [B]
    status: Optional["torch.Tensor"]    # int32 [1]


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

    def run_static(self, cu_draft, target_logits, draft_logits, draft_tokens, uniforms,
                   temperature: float, *, num_seqs: Optional[int] = None,
                   total_draft_rows: Optional[int] = None, out: Optional[VerifyOutput] = None,
                   stream=None) -> VerifyOutput:
        """spec_verify_run_static: the same verify step with the library's
        own device workspace (no workspace argument, nothing allocated by
        the library; `out` is still the caller's)."""
        return self._run("spec_verify_run_static", cu_draft, target_logits, draft_logits,
                         draft_tokens, uniforms, temperature, num_seqs, total_draft_rows,
                         out, None, stream)

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

    def tree_greedy(self, cu_nodes, parent, tokens, target_logits, **kw) -> TreeOutput:
        """Greedy tree verification (spec_verify_tree_run_greedy)."""
        return self._run_tree("spec_verify_tree_run_greedy", cu_nodes, parent, tokens,
                              target_logits, None, 1.0, **kw)

    def tree_point(self, cu_nodes, parent, tokens, target_logits, uniforms, temperature: float,
                   **kw) -> TreeOutput:
        """Tree verification of point-mass candidates (spec_verify_tree_run_point)."""
        return self._run_tree("spec_verify_tree_run_point", cu_nodes, parent, tokens,
                              target_logits, uniforms, temperature, **kw)

    def _run_tree(self, entry, cu_nodes, parent, tokens, target_logits, uniforms, temperature,
                  out: Optional[TreeOutput] = None, timing_events=None, stream=None):
        torch = self._torch
        B = int(cu_nodes.shape[0]) - 1
        R = int(target_logits.shape[0])
        dev = self.device
        if out is None:
            out = TreeOutput(torch.empty(R, dtype=torch.int32, device=dev),
                             torch.empty(R, dtype=torch.int32, device=dev),
                             torch.empty(B, dtype=torch.int32, device=dev),
                             torch.zeros(1, dtype=torch.int32, device=dev))
        if target_logits.dtype != self.torch_dtype or target_logits.stride(-1) != 1:
            raise ValueError(f"target_logits must be {self.torch_dtype} with unit column stride")
        for name, t, dt in (("cu_nodes", cu_nodes, torch.int32), ("parent", parent, torch.int32),
                            ("tokens", tokens, torch.int32), ("uniforms", uniforms, torch.float32)):
            if t is not None and (t.dtype != dt or not t.is_contiguous()):
                raise ValueError(f"{name} must be a contiguous {dt} tensor")
        events = None
        if timing_events is not None:
            events = (ctypes.c_void_p * len(timing_events))(
                *[ctypes.c_void_p(int(e.cuda_event)) if hasattr(e, "cuda_event") else e
                  for e in timing_events])
        a = TreeArgs(num_seqs=B, total_nodes=R, cu_nodes=_ptr(cu_nodes), parent=_ptr(parent),
                     tokens=_ptr(tokens), target_logits=_ptr(target_logits),
                     ld=int(target_logits.stride(0)), uniforms=_ptr(uniforms),
                     temperature=float(temperature), out_tokens=_ptr(out.out_tokens),
                     out_path=_ptr(out.out_path), out_num_accepted=_ptr(out.num_accepted),
                     workspace=_ptr(self.workspace), workspace_bytes=int(self.workspace.numel()),
                     status=_ptr(out.status),
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
        static = entry == "spec_verify_run_static"   # the library's own workspace
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
            out_residual_sum=_ptr(out.residual_sum),
            workspace=None if static else _ptr(self.workspace),
            workspace_bytes=0 if static else int(self.workspace.numel()), status=_ptr(out.status),
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


def read_probe(src, sink, *, nontemporal: bool = True, stream=None, events=None) -> None:
    """Enqueue spec_verify_read_probe over the bytes of the CUDA tensor `src`
    (measurement only).  `sink` is a one-element int32 CUDA tensor; `events`
    an optional (start, stop) pair of timing-enabled torch.cuda.Event that
    have been recorded once (so the HIP events exist)."""
    import torch
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    handle = (stream or torch.cuda.current_stream()).cuda_stream
    ev = (None, None)
    if events is not None:
        ev = tuple(int(e.cuda_event) for e in events)
    st = lib.spec_verify_read_probe(ctypes.c_void_p(src.data_ptr()), nbytes, int(nontemporal),
                                    ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(handle),
                                    ctypes.c_void_p(ev[0]), ctypes.c_void_p(ev[1]))
    if st != OK:
        raise SpecVerifyError("spec_verify_read_probe", st, lib.spec_verify_last_hip_error())


def adapt_params(preset: str = "window50", **overrides) -> AdaptParams:
    """A preset of spec_verify_adapt_preset, with fields overridden."""
    lib = load_library()
    p = AdaptParams()
    st = lib.spec_verify_adapt_preset(ADAPT_PRESETS[preset], ctypes.byref(p))
    if st != OK:
        raise SpecVerifyError("spec_verify_adapt_preset", st)
    for k, v in overrides.items():
        setattr(p, k, v)
    return p


class DraftLengthController:
    """Adaptive draft lengths for `num_slots` request slots plus acceptance
    statistics (include/spec_verify_adapt.h).

    device "host": state and arrays are numpy (the library computes on the
    calling thread); otherwise a torch device: state and arrays are device
    tensors and every call is enqueued on the stream.  Marshalling only."""

    def __init__(self, num_slots: int, params: Optional[AdaptParams] = None,
                 device="host"):
        import numpy as np
        self._np = np
        self.lib = load_library()
        self.params = params if params is not None else adapt_params()
        self.num_slots = int(num_slots)
        nbytes = ctypes.c_size_t()
        st = self.lib.spec_verify_adapt_state_bytes(ctypes.byref(self.params), self.num_slots,
                                                    ctypes.byref(nbytes))
        if st != OK:
            raise SpecVerifyError("spec_verify_adapt_state_bytes", st)
        self.state_bytes = int(nbytes.value)
        self.host = device == "host"
        if self.host:
            raw = np.zeros(self.state_bytes + 256, dtype=np.uint8)
            off = (-raw.ctypes.data) % 256
            self._raw = raw
            self.state = raw[off:off + self.state_bytes]
            self.stats = np.zeros(4, dtype=np.uint64)
            self.status = np.zeros(1, dtype=np.uint32)
            self.device_index = ADAPT_HOST
        else:
            import torch
            self._torch = torch
            dev = torch.device(device)
            self.state = torch.zeros(max(self.state_bytes, 256), dtype=torch.uint8, device=dev)
            self.stats = torch.zeros(4, dtype=torch.int64, device=dev)
            self.status = torch.zeros(1, dtype=torch.int32, device=dev)
            self.device_index = dev.index or 0
        self.reset()

    def _p(self, a):
        if a is None:
            return None
        return a.ctypes.data if self.host else int(a.data_ptr())

    def _stream(self, stream):
        if self.host:
            return None
        torch = self._torch
        if stream is None:
            stream = torch.cuda.current_stream(self.state.device)
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream")
                               else int(stream))

    def reset(self, slots=None, stream=None):
        """Reset slots (all when None) to k_init with an empty history."""
        n = self.num_slots if slots is None else int(slots.shape[0])
        st = self.lib.spec_verify_adapt_reset(
            ctypes.byref(self.params), self.num_slots, self._p(self.state), self.state_bytes, n,
            self._p(slots), self.device_index, self._stream(stream))
        if st != OK:
            raise SpecVerifyError("spec_verify_adapt_reset", st, self.lib.spec_verify_last_hip_error())

    def update(self, cu_draft, num_accepted, slots=None, next_k=None, next_cu=None,
               stream=None):
        """One step: returns (next_k [B], next_cu [B+1]) for the batch."""
        B = int(cu_draft.shape[0]) - 1
        if self.host:
            np = self._np
            next_k = np.empty(B, np.int32) if next_k is None else next_k
            next_cu = np.empty(B + 1, np.int32) if next_cu is None else next_cu
        else:
            torch = self._torch
            dev = self.state.device
            next_k = torch.empty(B, dtype=torch.int32, device=dev) if next_k is None else next_k
            next_cu = torch.empty(B + 1, dtype=torch.int32, device=dev) if next_cu is None else next_cu
        st = self.lib.spec_verify_adapt_update(
            ctypes.byref(self.params), self.num_slots, self._p(self.state), self.state_bytes, B,
            self._p(slots), self._p(cu_draft), self._p(num_accepted), self._p(next_k),
            self._p(next_cu), self._p(self.stats), self._p(self.status), self.device_index,
            self._stream(stream))
        if st != OK:
            raise SpecVerifyError("spec_verify_adapt_update", st,
                                  self.lib.spec_verify_last_hip_error())
        return next_k, next_cu

    def totals(self):
        """(sequences, accepted, drafted, emitted) so far (synchronises)."""
        v = self.stats if self.host else self.stats.cpu().numpy()
        return tuple(int(x) for x in v.astype("uint64"))

    def accept_rate(self) -> float:
        _, acc, drafted, _ = self.totals()
        return acc / drafted if drafted else 0.0
