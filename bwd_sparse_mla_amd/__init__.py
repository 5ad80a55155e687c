"""DSA sparse-MLA attention (forward and backward) and its index-production
top-k step on AMD Instinct MI355X.

The computation runs in hand-written HIP kernels for gfx950 behind the C ABI
of libsmla.so (include/smla.h); this package only marshals arguments.
"""
from ._lib import SmlaError, load as load_library
from .ops import (NonfiniteGradientError, SparseMLA, SparseMLARunner, bwd_workspace_bytes,
                  count_nonfinite, fwd_workspace_bytes, replace_nonfinite_, sparse_mla_bwd,
                  sparse_mla_bwd_checked, sparse_mla_fwd, sparse_mla_fwd_fp8, timing_read, timing_start, timing_stop,
                  topk_indices, validate_indices)

__all__ = ["NonfiniteGradientError", "SmlaError", "SparseMLA", "SparseMLARunner",
           "bwd_workspace_bytes", "count_nonfinite", "fwd_workspace_bytes", "load_library",
           "replace_nonfinite_", "sparse_mla_bwd", "sparse_mla_bwd_checked", "sparse_mla_fwd",
           "sparse_mla_fwd_fp8",
           "timing_read", "timing_start", "timing_stop", "topk_indices", "validate_indices"]
