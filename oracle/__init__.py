"""CPU oracle for paged GQA attention and KV row moves.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test suite, the entry point's smoke check and the benchmark's CPU
baseline leg may call it.  It shares no code with the HIP library and is
written from the source pages directly:

* "Tiered KV cache — architecture", section "The paged-attention block
  model": tokens live in fixed-size physical blocks; a per-sequence
  logical->physical block table says which block holds which range; a table
  entry equal to the invalid-block sentinel scores -infinity, i.e. the token
  does not exist (also section "Kernel dispatch").
* "KV Cache Design — cells, format, sessions", section 1 "Positions and
  cells": a window is causal positions, one [lo, hi) range, or a map of
  (cell, len) runs; section 2: moves are applied in order_moves order
  (upward moves top-down, downward bottom-up, upward first) and rows move
  verbatim; section 3: the q8_0 cell format.
* "KV cache" (sipllm), section "Problem": a decode step dots the new query
  against the stored history; section "Design": the dense [pos][kv_dim]
  layout used here as the contiguous reference layout.
* "KV Cache Design", section 3: the store's q8_0 quantizer (scale amax/127
  kept as f16, codes rounded to nearest, ties to even); the store writes a
  token's rows through the block table.
* "Tiered KV cache — architecture", section "The paged-attention block
  model", and "KV Cache Design", sections 1-2: the copy-on-write block pool
  (forks share blocks by reference count; a write into a shared block
  copies it first, so readers of the shared prefix see no change).
* "Tiered KV cache — architecture", section "The three-tier model": the
  int4 cold-block codec (one f32 scale per block, packed nibbles).

Arithmetic is float64 numpy; byte work is exact.  Readings of points the
pages leave open are stated in the docstrings where they are used.
"""

from .formats import row_bytes, seg_bytes, decode_rows, f16_bits_to_f64  # noqa: F401
from .attention import (  # noqa: F401
    INVALID_BLOCK,
    KV_MAP_MAX_SPANS,
    window_candidates,
    visible_positions,
    physical_row,
    resolve_rows,
    attend,
    lse_merge,
    paged_attention,
    paged_decode,
    paged_prefill,
)
from .moves import order_moves, copy_cells, copy_cells_rowwise, provenance  # noqa: F401
from .store import quantize_q8_0, encode_rows, destination_rows, store_rows  # noqa: F401
from .cow import BlockPoolModel, copy_blocks  # noqa: F401
from .int4 import blob_bytes, encode_block, decode_block, encode_blocks, cosine  # noqa: F401
