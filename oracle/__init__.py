"""fp64 CPU oracle for sparse-MLA attention (one or several KV groups), the
index-production top-k step and the nonfinite diagnostics (test
infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library.
"""
from .smla_oracle import (EMPTY_ROW_LSE, SUMEXP_FLOOR, OracleInputError,
                          sparse_mla_bwd, sparse_mla_fwd, token_backward,
                          token_forward, touched_rows, valid_slots)
from .topk_oracle import TopkInputError, causal_ranges, select_row, topk_indices
from .diag_oracle import count_nonfinite, nonfinite_mask, replace_nonfinite
from .grouped_oracle import sparse_mla_bwd_grouped, sparse_mla_fwd_grouped
from .fp8_oracle import decode_e4m3, decode_kv_records, kv_rows_bf16, round_bf16, sparse_mla_fwd_fp8

__all__ = ["EMPTY_ROW_LSE", "SUMEXP_FLOOR", "OracleInputError", "sparse_mla_bwd",
           "sparse_mla_fwd", "token_backward", "token_forward", "touched_rows",
           "valid_slots", "TopkInputError", "causal_ranges", "select_row", "topk_indices",
           "count_nonfinite", "nonfinite_mask", "replace_nonfinite", "sparse_mla_bwd_grouped",
           "sparse_mla_fwd_grouped", "decode_e4m3", "decode_kv_records", "kv_rows_bf16", "round_bf16",
           "sparse_mla_fwd_fp8"]
