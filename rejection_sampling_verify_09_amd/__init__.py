"""MI355X (gfx950) speculative-sampling verification.

The computation runs in libspecverify.so (hand-written HIP kernels behind the
C ABI of include/specverify.h); this package is its Python binding.
"""
from ._lib import (  # noqa: F401
    SV_BF16,
    SV_F32,
    SV_MAX_K,
    DraftLengthController,
    SpecVerifyError,
    filtered_probs,
    init,
    lib,
    lm_logits,
    profile_start,
    profile_stop,
    read_floor,
    release,
    scratch_bytes,
    stream_release,
    sample,
    spec_verify,
    spec_verify_noalloc,
    spec_verify_lmhead,
    spec_verify_probs,
    spec_verify_ragged,
    status_string,
)

__all__ = ["spec_verify", "spec_verify_noalloc", "spec_verify_lmhead", "lm_logits", "spec_verify_probs", "spec_verify_ragged", "DraftLengthController", "sample", "filtered_probs", "profile_start", "profile_stop", "read_floor", "release", "init", "stream_release", "scratch_bytes", "status_string", "lib",
           "SpecVerifyError"]
