"""Batched Muon optimizer step for AMD MI355X (gfx950).

The computation lives in the HIP library libmuon_mi355x.so (C ABI declared in
include/muon_mi355x.h); this package is its Python binding.
"""
from ._binding import (  # noqa: F401
    CUBIC, EXPORTED, HEADER_PATH, KERNELS, LIB_PATH, MAX_DIM, MUON_BF16, MUON_ERR_HIP,
    MUON_ERR_INVALID_ARG, MUON_ERR_UNSUPPORTED, MUON_ERR_WORKSPACE, MUON_FP32, MUON_OK,
    NOALLOC_MAX_WORKSPACE, QUINTIC, AdamWParams, MuonError, NsParams, StepParams, adamw_batched,
    adamw_workspace_bytes, allocate_workspace, hbm_stream, last_error_detail, load_library,
    ns_batched, ns_batched_noalloc, status_string, step_batched, timing_enable, timing_read,
    timing_reset, workspace_bytes,
)
