"""Fused scaled-dot-product attention forward for MI355X (gfx950).

The computation lives in libsdpa.so (HIP kernels behind the C ABI of
include/sdpa.h); this package is its ctypes binding plus a seeded input
generator. The library loads on first use and raises if it is missing.
"""
from .binding import (EXPORTED, SDPA_BF16, SDPA_ERR_HIP, SDPA_ERR_INVALID, SDPA_ERR_UNSUPPORTED, SDPA_F16,
                      SDPA_F32, SDPA_MASK_ADDITIVE, SDPA_MASK_BOOL, SDPA_MASK_CAUSAL, SDPA_MASK_NONE, SDPA_OK,
                      SdpaError, attention, library_path, load, paged_attention, paged_write, sdpa_abi_version,
                      sdpa_forward, sdpa_forward_strided, sdpa_forward_windowed, sdpa_last_error,
                      sdpa_paged_forward, sdpa_paged_write, sdpa_plan, sdpa_plan_paged, sdpa_plan_windowed,
                      sdpa_release_workspace, sdpa_forward_noalloc, sdpa_noalloc_scratch_bytes)

__all__ = [
    "attention", "paged_attention", "paged_write", "sdpa_forward", "sdpa_plan", "sdpa_forward_windowed",
    "sdpa_plan_windowed", "sdpa_forward_strided", "sdpa_paged_forward", "sdpa_plan_paged", "sdpa_paged_write",
    "sdpa_last_error", "sdpa_release_workspace", "sdpa_abi_version", "sdpa_forward_noalloc",
    "sdpa_noalloc_scratch_bytes",
    "load", "library_path", "SdpaError", "EXPORTED",
    "SDPA_F32", "SDPA_F16", "SDPA_BF16", "SDPA_MASK_NONE", "SDPA_MASK_CAUSAL", "SDPA_MASK_BOOL", "SDPA_MASK_ADDITIVE",
    "SDPA_OK", "SDPA_ERR_INVALID", "SDPA_ERR_UNSUPPORTED", "SDPA_ERR_HIP",
]
