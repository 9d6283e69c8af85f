"""Row moves of the cell store, applied in order_moves order.

Source: "KV Cache Design — cells, format, sessions", section 2 "The cell
store: ownership, removal, compaction, sharing": a compaction changes only
cells, so rows move verbatim; whoever copies must order the moves upward
moves top-down, downward bottom-up, upward moves first, because a
destination may never land on a row that has not been copied yet; the
per-row copy runs in ascending row order when a run slides down and in
descending order when it slides up.

Readings where the pages are silent:
* a move is (src, dst, len) in pool rows; "up" means dst > src;
* "top-down" visits upward moves by descending src, "bottom-up" visits
  downward moves by ascending src; ties break on dst the same way, then on
  input index; moves with dst == src or len <= 0 are no-ops and dropped;
* for move sets where no order is safe (random, crossing moves) the result
  is defined as applying the moves one after another in that order, each as
  a memmove (the whole source run is read before it is written);
* the same moves apply to the K pool and to the V pool; tables are not
  touched;
* a row is one token cell: in a pool laid out [n_blocks, n_kv_heads,
  block_size, W], row r is slot r % block_size of block r // block_size
  across every kv head (a plain 2-d array is a list of rows).
"""

from __future__ import annotations

import numpy as np


def order_moves(moves) -> list:
    """Indices of the effective moves, in application order."""
    mv = [tuple(int(x) for x in m) for m in np.asarray(moves).reshape(-1, 3)]
    up = [i for i, (s, d, n) in enumerate(mv) if n > 0 and d > s]
    down = [i for i, (s, d, n) in enumerate(mv) if n > 0 and d < s]
    up.sort(key=lambda i: (-mv[i][0], -mv[i][1], i))
    down.sort(key=lambda i: (mv[i][0], mv[i][1], i))
    return up + down


def _get(pool, idx):
    if pool.ndim == 2:
        return pool[idx].copy()
    bs = pool.shape[2]
    return pool[idx // bs, :, idx % bs].copy()


def _set(pool, idx, val):
    if pool.ndim == 2:
        pool[idx] = val
    else:
        bs = pool.shape[2]
        pool[idx // bs, :, idx % bs] = val


def copy_cells(pools, moves):
    """Apply ``moves`` in order_moves order to every pool in ``pools`` (in
    place).  Each move copies its whole source run of rows, then writes it
    to the destination run (memmove)."""
    mv = np.asarray(moves).reshape(-1, 3)
    order = order_moves(mv)
    for pool in pools:
        for i in order:
            s, d, n = (int(x) for x in mv[i])
            src = np.arange(s, s + n)
            _set(pool, np.arange(d, d + n), _get(pool, src))
    return pools


def copy_cells_rowwise(pools, moves):
    """The same, one row at a time without staging: ascending rows when the
    run slides down, descending when it slides up."""
    mv = np.asarray(moves).reshape(-1, 3)
    order = order_moves(mv)
    for pool in pools:
        for i in order:
            s, d, n = (int(x) for x in mv[i])
            rng = range(n) if d < s else range(n - 1, -1, -1)
            for k in rng:
                _set(pool, np.array([d + k]), _get(pool, np.array([s + k])))
    return pools


def provenance(n_rows: int, moves) -> np.ndarray:
    """int64 [n_rows]: after the moves, row r holds the bytes that row
    provenance[r] held before them (the identity where nothing landed)."""
    src = np.arange(n_rows, dtype=np.int64)
    copy_cells([src.reshape(n_rows, 1)], moves)
    return src
