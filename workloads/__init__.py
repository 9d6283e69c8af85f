"""Seeded synthetic workloads for paged GQA attention and row moves.

This package only draws inputs: block tables, sequence lengths, windows,
query positions, move lists and the random K/V/q values, encoded into the
storage formats the kernels read.  It holds none of the attention or move
arithmetic.  Both the kernels' tests and the CPU oracle's tests take their
inputs from here, so the two sides always see the same bytes.
"""

from .gen import (  # noqa: F401
    FMT_BYTES,
    Workload,
    MoveSet,
    make,
    make_moves,
    materialize,
    encode_q8_0,
    q8_0_row_bytes,
    q8_0_seg_bytes,
    make_custom,
    referenced_rows,
    host_subset,
)
