"""Pool row formats, decoded to float64.

Source: "KV Cache Design — cells, format, sessions", section 3 "The storage
format is a gate, never a guess": the KV format is one of f32, f16, q8_0; a
Q8_0 block is 32 int8 codes with an f16 scale, and a q8_0 cell (one pool
row) is a whole number of Q8_0 blocks rounded up to whole f32 words.
"Tiered KV cache — architecture", section "The three-tier model": a block is
block_size tokens x n_kv_heads x head_dim, so one token's row holds every kv
head.

Readings:
* byte order inside a pool block: [kv head][slot][head_dim], i.e. a pool is
  [n_blocks, n_kv_heads, block_size, W]; pool row r (token cell) is slot
  r % block_size of block r // block_size, across all kv heads;
* q8_0: one token of one kv head is head_dim/32 blocks, each the scale (2
  bytes, little-endian IEEE half) followed by its 32 signed codes, rounded up
  to whole 4-byte words; the dequantized value is scale * code, which is
  exact in float64 (and in float32).  The query is not quantized.
"""

from __future__ import annotations

import numpy as np

Q8_BLOCK = 32
Q8_BLOCK_BYTES = 2 + Q8_BLOCK


def seg_bytes(fmt: str, head_dim: int) -> int:
    """Bytes of one token of one kv head."""
    if fmt == "f32":
        return 4 * head_dim
    if fmt == "f16":
        return 2 * head_dim
    if fmt == "q8_0":
        if head_dim % Q8_BLOCK:
            raise ValueError("q8_0 needs head_dim divisible by 32")
        raw = (head_dim // Q8_BLOCK) * Q8_BLOCK_BYTES
        return 4 * (-(-raw // 4))
    raise ValueError(f"unknown KV format {fmt!r}")


def row_bytes(fmt: str, n_kv_heads: int, head_dim: int) -> int:
    """Bytes of one token cell (all kv heads)."""
    return n_kv_heads * seg_bytes(fmt, head_dim)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) to float64, decoded field by field
    (sign, 5-bit exponent with bias 15, 10-bit fraction; exponent 0 is
    subnormal, 31 is inf/NaN)."""
    b = bits.astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = sign * (1.0 + f / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = sign * (f / 1024.0) * 2.0 ** -14
    special = np.where(f == 0, sign * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 31, special, normal))


def decode_rows(pool: np.ndarray, fmt: str, rows: np.ndarray, n_kv_heads: int, head_dim: int) -> np.ndarray:
    """Token cells ``rows`` (pool row r = block r // bs, slot r % bs) of
    ``pool`` [n_blocks, n_kv_heads, bs, W] as float64 [len(rows), n_kv_heads,
    head_dim]."""
    rows = np.asarray(rows, dtype=np.int64)
    bs = pool.shape[2]
    cells = pool[rows // bs, :, rows % bs]  # [n, n_kv_heads, W]
    if fmt in ("f32", "f16"):
        return cells.astype(np.float64)
    if fmt != "q8_0":
        raise ValueError(f"unknown KV format {fmt!r}")
    nb = head_dim // Q8_BLOCK
    blocks = np.ascontiguousarray(cells[..., : nb * Q8_BLOCK_BYTES]).reshape(len(rows), n_kv_heads, nb, Q8_BLOCK_BYTES)
    bits = blocks[..., 0].astype(np.uint16) | (blocks[..., 1].astype(np.uint16) << 8)
    scale = f16_bits_to_f64(bits)
    codes = blocks[..., 2:].astype(np.uint8).view(np.int8).astype(np.float64)
    return (scale[..., None] * codes).reshape(len(rows), n_kv_heads, head_dim)
