"""Packed variable-length mixed-mask attention for MI355X (gfx950).

The compute path is the C-ABI library ``libpva.so`` (HIP kernels + host
planner) declared in ``include/pva.h``; this package is its thin binding.
Importing the package never needs the library; every call that does raises
if it is missing.
"""
from .binding import (PvaError, SegDesc, packed_attn_fwd, packed_attn_fwd_fp8, packed_attn_fwd_varlen,
                      packed_attn_fwd_varlen_fp8, packed_attn_fwd_partial, packed_attn_fwd_partial_fp8, merge_partials,
                      packed_attn_fwd_partial_accumulate, packed_attn_fwd_partial_accumulate_fp8,
                      packed_attn_fwd_paged, lib, version, LIB_PATH, EXPORTED, use_timeline_build, timeline_clear,
                      timeline_read, SEG_CAUSAL, SEG_FULL, PVA_OK,
                      PVA_ERR_INVALID_ARG, PVA_ERR_UNSUPPORTED, PVA_ERR_HIP, PVA_ERR_NO_MEMORY)

__all__ = [
    "PvaError", "SegDesc", "packed_attn_fwd", "packed_attn_fwd_fp8", "packed_attn_fwd_varlen",
    "packed_attn_fwd_varlen_fp8", "packed_attn_fwd_partial", "packed_attn_fwd_partial_fp8", "merge_partials",
    "packed_attn_fwd_partial_accumulate", "packed_attn_fwd_partial_accumulate_fp8", "packed_attn_fwd_paged", "lib", "version", "use_timeline_build", "timeline_clear",
    "timeline_read", "LIB_PATH", "EXPORTED", "SEG_CAUSAL", "SEG_FULL", "PVA_OK",
    "PVA_ERR_INVALID_ARG", "PVA_ERR_UNSUPPORTED", "PVA_ERR_HIP", "PVA_ERR_NO_MEMORY",
]
