"""Storing new K/V rows into the paged pools, with the q8_0 quantizer.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* "KV Cache Design — cells, format, sessions", section 3 "The storage
  format is a gate, never a guess": the store quantizes with a single
  quantizer everywhere — the block scale is amax/127, kept as an f16, and
  codes round to nearest with ties to even; a Q8_0 block is 32 int8 codes
  with that scale, and a cell is whole Q8_0 blocks rounded up to whole f32
  words.  Section 2 names the store op of the fused decode family (positions
  rope, cells store) — the write that precedes every read.
* "Tiered KV cache — architecture", section "The paged-attention block
  model": position t of a sequence lives in physical block
  table[t // block_size] at slot t % block_size; a sentinel entry is a
  block that does not exist.

Readings where the pages are silent:
* the quantizer works in binary32: amax = max |x| over the 32 values (exact),
  d = amax / 127 rounded to binary32, each code = x / d rounded to binary32
  and then to the nearest integer, ties to even, clamped to [-127, 127];
  the stored scale is d rounded to binary16 (nearest, ties to even).  The
  codes are taken against d, not against the rounded f16 scale, so a block
  whose scale underflows f16 stores scale 0 with non-zero codes;
* amax = 0 stores scale 0 and zero codes; inputs are finite and amax / 127
  stays inside the f16 range (larger values are outside the format);
* bytes of a q8_0 segment past the last block (when head_dim / 32 is odd)
  are written as zero;
* f16 pool rows take the source rounded to binary16 (nearest, ties to
  even); f32 pool rows take it exactly;
* a store names its destination by (sequence, position); a position whose
  logical block lies outside the table or whose entry is not a pool block
  (the sentinel included) is not stored and is counted as skipped;
* destinations of one store are distinct (a row named twice is not a case
  this oracle defines: it applies the tokens in order).
"""

from __future__ import annotations

import numpy as np

from .formats import Q8_BLOCK, seg_bytes


def quantize_q8_0(x) -> np.ndarray:
    """Q8_0 bytes of float rows x [..., head_dim] (head_dim % 32 == 0):
    uint8 [..., seg_bytes('q8_0', head_dim)], per 32-value block the scale as
    little-endian binary16 then the 32 codes as int8."""
    x = np.asarray(x, dtype=np.float32)
    hd = x.shape[-1]
    if hd % Q8_BLOCK:
        raise ValueError("q8_0 needs head_dim divisible by 32")
    lead = x.shape[:-1]
    nb = hd // Q8_BLOCK
    blocks = x.reshape(*lead, nb, Q8_BLOCK)
    amax = np.max(np.abs(blocks), axis=-1)                 # float32, exact
    d = amax / np.float32(127.0)                           # float32 division
    live = d > 0
    safe = np.where(live, d, np.float32(1.0)).astype(np.float32)
    ratio = blocks / safe[..., None]                       # float32 division
    codes = np.clip(np.rint(ratio), -127, 127)             # rint: ties to even
    codes = np.where(live[..., None], codes, 0).astype(np.int8)
    scale = d.astype(np.float16)                           # nearest-even
    out = np.zeros((*lead, seg_bytes("q8_0", hd)), dtype=np.uint8)
    raw = np.concatenate([scale[..., None].view(np.uint8).reshape(*lead, nb, 2),
                          codes.view(np.uint8)], axis=-1)
    out[..., : nb * (2 + Q8_BLOCK)] = raw.reshape(*lead, nb * (2 + Q8_BLOCK))
    return out


def encode_rows(x, fmt: str) -> np.ndarray:
    """Rows x [..., head_dim] in pool format fmt: float32, float16 or q8_0
    bytes (the last axis is the segment)."""
    x = np.asarray(x, dtype=np.float32)
    if fmt == "f32":
        return x.copy()
    if fmt == "f16":
        return x.astype(np.float16)
    if fmt == "q8_0":
        return quantize_q8_0(x)
    raise ValueError(f"unknown KV format {fmt!r}")


def destination_rows(seq_ids, pos, block_table, n_pool_blocks: int, block_size: int) -> np.ndarray:
    """Pool row of each token (sequence seq_ids[t], position pos[t]):
    table[s][p // bs] * bs + p % bs, or -1 when the token has no row (the
    sequence or the logical block is outside the table, or the entry is not
    a block of the pool)."""
    table = np.asarray(block_table, dtype=np.int64)
    n_seqs, max_blocks = table.shape
    s = np.asarray(seq_ids, dtype=np.int64)
    p = np.asarray(pos, dtype=np.int64)
    rows = np.full(len(p), -1, dtype=np.int64)
    for t in range(len(p)):
        if not (0 <= s[t] < n_seqs) or not (0 <= p[t] < max_blocks * block_size):
            continue
        blk = table[s[t], p[t] // block_size]
        if 0 <= blk < n_pool_blocks:
            rows[t] = blk * block_size + p[t] % block_size
    return rows


def store_rows(k_pool, v_pool, k_fmt: str, v_fmt: str, k_new, v_new, seq_ids, pos, block_table):
    """Write token t's K row k_new[t] and V row v_new[t] ([n_tok, n_kv_heads,
    head_dim], any float dtype; f16 sources are exact in float32) into pool
    row destination_rows(...)[t] of copies of the pools ([n_blocks,
    n_kv_heads, block_size, W]), each in its pool's format.  v_pool may be
    None.  Returns (k_pool', v_pool', skipped)."""
    k_out = np.array(k_pool, copy=True)
    v_out = None if v_pool is None else np.array(v_pool, copy=True)
    nblk, _, bs, _ = k_out.shape
    rows = destination_rows(seq_ids, pos, block_table, nblk, bs)
    kx = encode_rows(np.asarray(k_new, dtype=np.float32), k_fmt)
    vx = None if v_out is None else encode_rows(np.asarray(v_new, dtype=np.float32), v_fmt)
    for t, r in enumerate(rows):
        if r < 0:
            continue
        k_out[r // bs, :, r % bs] = kx[t]
        if v_out is not None:
            v_out[r // bs, :, r % bs] = vx[t]
    return k_out, v_out, int(np.count_nonzero(rows < 0))
