"""CPU oracle for block-sparse attention — TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy implementations of what the GPU library computes,
written from the source pages, used to check the GPU path and nothing else.
Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package; the library never does, and nothing here is shared with
the HIP kernels or their C interface.

Modules:
  core            block-sparse softmax attention, per-entry partials, the
                  log-sum-exp combine and the speculative + sparse composition
  gate            BSFA tile-maximum gating and threshold calibration
  vertical_slash  vertical-slash index conversion and attention over it
  selected        selected attention: each query token attends to its top-k key blocks
  backward        gradients of block-sparse attention (dQ, dK, dV)

Pinning (see the tests marked "not gpu"): every function here is checked
against closed forms, invariants, brute force and an independent library
routine.  Two readings have no such pin and say "parity unpinned" in their
docstrings: the exact windows chosen by the vertical-slash conversion (own
greedy rule; only its coverage invariants are pinned), and which of the two
readings of a skipped tile's scores the gating page's own kernel takes (both
are implemented, "drop" and "count", each pinned by its own closed forms).
"""
from .backward import block_sparse_bwd
from .core import (as_f64, attend_rows, block_mask, block_sparse, block_sparse_partials, causal_mask,
                   combine, dense, default_scale, speculative_sparse)
from .gate import calibrate, gated, gated_rows, tile_max_row
from .gate import density as gated_density
from .selected import selected, selected_rows
from .vertical_slash import vs_attention, vs_attention_rows, vs_convert, vs_convert_item, vs_convert_mergehead

__all__ = [
    "block_sparse_bwd", "as_f64", "attend_rows", "block_mask", "block_sparse", "block_sparse_partials", "causal_mask",
    "combine", "dense", "default_scale", "speculative_sparse", "gated", "gated_rows", "tile_max_row", "calibrate", "gated_density",
    "selected", "selected_rows", "vs_attention", "vs_attention_rows", "vs_convert", "vs_convert_item", "vs_convert_mergehead",
]
