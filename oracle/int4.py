"""int4 cold-block codec.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "Tiered KV cache — architecture", section "The three-tier model":
cold blocks are kept as int4 with a scale, one scale per block — the block
is stored as an f32 scale followed by ceil(n_elts / 2) bytes of packed int4
nibbles — and the page measures a cosine similarity of about 0.99 against
the unquantized block.

Readings where the page is silent:
* a block is one pool block of one pool (K or V): block_size tokens x
  n_kv_heads x head_dim values, taken as a flat array in memory order;
* the quantizer is symmetric and works in binary32: scale = amax / 7
  (amax = max |x|), code = x / scale rounded to nearest with ties to even,
  clamped to [-7, 7]; amax = 0 gives scale 0 and zero codes;
* codes are 4-bit two's complement; value 2j sits in the low nibble of
  byte j and value 2j + 1 in its high nibble (a high nibble with no value
  is 0); the scale is stored little-endian;
* decoding gives scale * code rounded to binary32, then rounded to the
  pool's format (f16: nearest-even; f32: as is).
"""

from __future__ import annotations

import numpy as np


def blob_bytes(n_elts: int) -> int:
    """Bytes of one encoded block: the f32 scale and the nibbles."""
    return 4 + (int(n_elts) + 1) // 2


def encode_block(x) -> np.ndarray:
    """uint8 [blob_bytes(n)] of one block's values x (any float dtype)."""
    x = np.asarray(x, dtype=np.float32).reshape(-1)
    n = x.size
    amax = np.max(np.abs(x)) if n else np.float32(0)
    scale = np.float32(amax) / np.float32(7.0)  # binary32 division
    if scale > 0:
        codes = np.clip(np.rint(x / scale), -7, 7).astype(np.int8)  # x / scale in binary32
    else:
        codes = np.zeros(n, dtype=np.int8)
    nib = (codes.astype(np.int16) & 0xF).astype(np.uint8)
    if n % 2:
        nib = np.concatenate([nib, np.zeros(1, dtype=np.uint8)])
    packed = nib[0::2] | (nib[1::2] << 4)
    return np.concatenate([np.array([scale], dtype="<f4").view(np.uint8), packed.astype(np.uint8)])


def decode_block(blob, n_elts: int, fmt: str = "f32") -> np.ndarray:
    """The block's n_elts values from its blob, in the pool format."""
    blob = np.asarray(blob, dtype=np.uint8).reshape(-1)
    scale = blob[:4].view("<f4")[0]
    packed = blob[4 : 4 + (n_elts + 1) // 2]
    nib = np.empty(2 * packed.size, dtype=np.uint8)
    nib[0::2] = packed & 0xF
    nib[1::2] = packed >> 4
    codes = nib[:n_elts].astype(np.int16)
    codes = np.where(codes >= 8, codes - 16, codes).astype(np.float32)
    vals = (scale * codes).astype(np.float32)  # binary32 product
    if fmt == "f16":
        return vals.astype(np.float16)
    if fmt == "f32":
        return vals
    raise ValueError(f"no int4 decode into {fmt!r}")


def encode_blocks(pool, blocks) -> np.ndarray:
    """Blobs [len(blocks), blob_bytes] of the pool blocks (pool [n_blocks, ...])."""
    pool = np.asarray(pool)
    n = int(np.prod(pool.shape[1:]))
    out = np.zeros((len(blocks), blob_bytes(n)), dtype=np.uint8)
    for i, b in enumerate(blocks):
        out[i] = encode_block(pool[int(b)])
    return out


def cosine(a, b) -> float:
    a = np.asarray(a, dtype=np.float64).reshape(-1)
    b = np.asarray(b, dtype=np.float64).reshape(-1)
    return float(a @ b / np.sqrt((a @ a) * (b @ b)))
