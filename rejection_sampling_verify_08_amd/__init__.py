"""Batched speculative-decoding verify step for AMD Instinct MI355X (gfx950).

The computation runs in the hand-written HIP kernels of libspec_verify.so,
reached through its C ABI (include/spec_verify.h, include/spec_verify_adapt.h);
this package is the thin Python binding over it.  See `SpecVerifier` (sampled,
greedy and point-mass-draft verification) and `DraftLengthController` (the
adaptive draft length and acceptance statistics).
"""
from .binding import (  # noqa: F401
    BF16, EXPORTED, F32, FLAG_CHECK, LIB_PATH, AdaptParams, DraftLengthController,
    SpecVerifier, SpecVerifyError, VerifyOutput, adapt_params, load_library, verify,
)

__all__ = ["SpecVerifier", "SpecVerifyError", "VerifyOutput", "load_library",
           "verify", "LIB_PATH", "EXPORTED", "F32", "BF16", "FLAG_CHECK",
           "AdaptParams", "DraftLengthController", "adapt_params"]
