"""CPU oracle for FlexAttention-style block-sparse attention (test infrastructure).

This package is the slow, plainly written reference that the HIP path is
checked against.  It is test infrastructure only: the product library never
imports, links or executes it.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path; the
two meet only in the seeded input generators of ``workloads``.

Contents
  mods        score_mod / mask_mod menu, written from the pages' definitions
  attention   the dense definition: full score matrix in float64, g, then the
              -inf mask, then a row softmax (also how the pages describe the
              unfused fallback)
  blockmask   tile classification by counting visible cells, ordered lists,
              to_dense / sparsity helpers, the Q-side (transposed) lists, and the
              BlockMask utilities (slicing, cropping, the ASCII picture)
  blockwise   a second, independent float64 oracle that walks only the block
              lists with an online softmax; used to show the block mask loses
              nothing
  backward    the gradients dq, dk, dv of the same definition

Every function is pinned by tests under ``tests/`` that check it against
printed worked examples, closed forms and brute force (none of them re-types
the formula being checked).  Parity unpinned: NaN/Inf inputs, which the pages
only say must be checked separately.
"""
from .mods import ScoreMod, MaskMod, alibi_slope
from .attention import attention, attention_rows, default_scale
from .blockmask import (build_block_mask, to_dense, sparsity, visible_cells, transpose_block_mask,
                        slice_block_mask, adjust_block_mask, grid_classes, to_string)
from .blockwise import blockwise_attention
from .backward import attention_backward, score_derivative

__all__ = [
    "ScoreMod", "MaskMod", "alibi_slope", "attention", "attention_rows", "default_scale",
    "build_block_mask", "to_dense", "sparsity", "visible_cells", "blockwise_attention",
    "transpose_block_mask", "slice_block_mask", "adjust_block_mask", "grid_classes", "to_string",
    "attention_backward", "score_derivative",
]
