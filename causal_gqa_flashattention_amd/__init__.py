"""Causal grouped-query FlashAttention (forward + fused backward) for AMD MI355X.

The computation lives in hand-written HIP kernels for gfx950 inside
``libcgqa_fa.so`` (C ABI in ``include/fa.h``); this package only loads that
library and marshals torch tensors into it.
"""
from .binding import (  # noqa: F401
    FAError,
    FA_BF16,
    FA_F16,
    MASK_BLOCK,
    FaTensor,
    fa_bwd,
    fa_bwd_delta_ex,
    fa_bwd_ex,
    fa_bwd_workspace_bytes,
    fa_bwd_short,
    fa_fwd_short,
    fa_fwd_short_noalloc,
    NOALLOC_SCRATCH_BYTES,
    fa_short_workspace_bytes,
    SHORT_MAX_LQ,
    fa_bwd_block_sparse,
    fa_bwd_delta,
    fa_bwd_dkv,
    fa_bwd_dkv_block_sparse,
    fa_bwd_dq,
    fa_bwd_dq_block_sparse,
    fa_fwd,
    fa_fwd_block_sparse,
    fa_fwd_ex,
    lib_path,
    load_library,
    status_str,
    version,
)

__all__ = [
    "FAError", "MASK_BLOCK", "fa_fwd", "fa_bwd_delta", "fa_bwd", "fa_bwd_dq", "fa_bwd_dkv",
    "fa_fwd_block_sparse", "fa_bwd_block_sparse", "fa_bwd_dq_block_sparse",
    "fa_bwd_dkv_block_sparse", "fa_fwd_ex", "fa_bwd_delta_ex", "fa_bwd_ex", "fa_bwd_workspace_bytes", "FaTensor", "FA_BF16",
    "FA_F16", "fa_fwd_short", "fa_fwd_short_noalloc", "NOALLOC_SCRATCH_BYTES", "fa_bwd_short", "fa_short_workspace_bytes", "SHORT_MAX_LQ", "lib_path", "load_library", "status_str", "version",
]
