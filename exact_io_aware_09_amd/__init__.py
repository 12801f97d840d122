"""Exact multi-head attention for AMD Instinct MI355X (gfx950).

The product is the C-ABI shared library ``libfa_mi355x.so`` (declared in
``include/fa.h``) built from the HIP kernels in ``csrc/``.  This package holds
its ctypes binding (``_lib``: the C entry points under the same names), thin
tensor wrappers (``attention.forward`` / ``attention.backward``) and the
seeded synthetic workloads (``workloads``).
"""
from ._lib import (FA_BF16, FA_F32, FA_FP8_KEYS, FA_FP8_ROWS, FAError,  # noqa: F401
                   fa_backward, fa_backward_workspace_bytes, fa_backward_dropout,
                   fa_backward_sparse, fa_forward, fa_forward_dropout, fa_forward_fp8,
                   fa_forward_sparse, fa_forward_split, fa_fp8_bytes, fa_fp8_scale_bytes,
                   fa_quantize_fp8, fa_sparse_schedule, fa_sparse_workspace_bytes,
                   fa_forward_sparse_balanced, fa_backward_sparse_balanced,
                   fa_forward_split_workspace_bytes, fa_merge_partials, fa_strerror, fa_version)
from .autograd import FlashAttentionFunction, flash_attention  # noqa: F401
from .attention import (SparseSchedule, backward, backward_dropout,  # noqa: F401
                        backward_sparse, backward_sparse_balanced, forward, forward_dropout,
                        forward_fp8, forward_sparse, forward_sparse_balanced, forward_split,
                        merge_partials, quantize_fp8, sparse_schedule, workspace_bytes)

__all__ = [
    "FA_BF16", "FA_F32", "FAError", "fa_forward", "fa_backward", "fa_backward_workspace_bytes",
    "fa_strerror", "fa_version", "forward", "backward", "workspace_bytes",
    "fa_forward_split", "fa_forward_split_workspace_bytes", "fa_merge_partials",
    "forward_split", "merge_partials", "fa_forward_sparse", "fa_backward_sparse",
    "forward_sparse", "backward_sparse", "fa_sparse_schedule", "fa_sparse_workspace_bytes",
    "fa_forward_sparse_balanced", "fa_backward_sparse_balanced", "SparseSchedule",
    "sparse_schedule", "forward_sparse_balanced", "backward_sparse_balanced",
    "fa_forward_dropout", "fa_backward_dropout",
    "forward_dropout", "backward_dropout", "FA_FP8_ROWS", "FA_FP8_KEYS", "fa_fp8_bytes",
    "fa_fp8_scale_bytes", "fa_quantize_fp8", "fa_forward_fp8", "quantize_fp8", "forward_fp8",
    "flash_attention", "FlashAttentionFunction",
]
