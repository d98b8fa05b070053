"""Fused exact attention forward pass for AMD MI355X (gfx950).

The compute lives in the HIP library libfa_mi355x.so (C interface:
include/fa.h).  ``binding`` wraps it; ``inputs`` draws seeded synthetic inputs.
Importing the package does not load the library; the first call does, and
raises if it has not been built.
"""
from .binding import (  # noqa: F401
    FA_ERR_INVALID_ARG, FA_ERR_LAUNCH, FA_ERR_MISALIGNED, FA_ERR_NO_DEVICE, FA_ERR_UNSUPPORTED, FA_OK,
    FaError, attention_backward, attention_forward, attention_forward_fp8, decode_forward, fa_bwd, fa_bwd_workspace_size, fa_decode, fa_decode_workspace_size, fa_fwd, fa_fwd_f32, fa_fwd_fp8, fa_fwd_gqa,
    fa_fwd_gqa_f32, fa_status_str, load,
)
