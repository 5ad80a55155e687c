"""fp64 CPU oracle for sparse-MLA attention and for the index-production
top-k step (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library.
"""
from .smla_oracle import (EMPTY_ROW_LSE, SUMEXP_FLOOR, OracleInputError,
                          sparse_mla_bwd, sparse_mla_fwd, token_backward,
                          token_forward, touched_rows, valid_slots)
from .topk_oracle import TopkInputError, causal_ranges, select_row, topk_indices

__all__ = ["EMPTY_ROW_LSE", "SUMEXP_FLOOR", "OracleInputError", "sparse_mla_bwd",
           "sparse_mla_fwd", "token_backward", "token_forward", "touched_rows",
           "valid_slots", "TopkInputError", "causal_ranges", "select_row", "topk_indices"]
