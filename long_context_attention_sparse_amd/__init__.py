"""Block-sparse FlashAttention forward for AMD MI355X (gfx950).

Python face of libbsa.so; every entry point has the name of its C function in
include/bsa.h and only marshals arguments — the kernels do all the work:

  bsa_fwd             attention restricted to a key pattern (dense, block
                      lists or vertical-slash metadata), returning (O, LSE)
  bsa_fwd_partials    one (o, lse) partial per list entry
  bsa_combine         log-sum-exp combine of partials
  bsa_fwd_gated       BSFA gated causal attention (tile max vs threshold)
  bsfa_calibrate      BSFA thresholds: k-th largest off-diagonal tile maximum per row
  bsa_fwd_selected    selected attention: each query token over its top-k key blocks
  bsa_bwd             gradients (dQ, dK, dV) of bsa_fwd over dense or block patterns
  vs_convert_indexes  vertical-slash index conversion
  vs_convert_indexes_mergehead  the same with per-head counts of valid indices
  speculative_sparse  speculative pass + sparse repair pass + combine
                      (bsa_speculative_sparse; bsa_speculative_partials without
                      the combine; speculative_sparse_noalloc with the partials
                      in a library-resident scratch area, for callers that
                      cannot allocate)
  bsa_check_pattern   device check of a pattern's contents (the same check the
                      entry points run first when BSA_DEBUG_CHECKS is set)
"""
from ._binding import (EXPORTS, LIB_PATH, NOALLOC_SCRATCH_BYTES, BlockPattern, BSAError, VSPattern, bsa_check_pattern, bsa_combine, bsa_fwd,
                       bsa_fwd_gated, bsa_bwd, bsa_bwd_workspace_size, bsa_fwd_selected, bsa_selected_workspace_size, bsfa_calibrate,
                       bsa_fwd_partials, bsa_num_partials, bsa_speculative_partials, bsa_workspace_size, load,
                       speculative_sparse, speculative_sparse_noalloc, vs_convert_indexes,
                       vs_convert_indexes_mergehead)

__all__ = ["EXPORTS", "LIB_PATH", "NOALLOC_SCRATCH_BYTES", "BlockPattern", "BSAError", "VSPattern", "bsa_check_pattern", "bsa_combine", "bsa_fwd", "bsa_fwd_gated",
           "bsa_bwd", "bsa_bwd_workspace_size", "bsa_fwd_selected", "bsa_selected_workspace_size", "bsfa_calibrate",
           "bsa_fwd_partials", "bsa_num_partials", "bsa_speculative_partials", "bsa_workspace_size", "load",
           "speculative_sparse", "speculative_sparse_noalloc", "vs_convert_indexes",
           "vs_convert_indexes_mergehead"]
