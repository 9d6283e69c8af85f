"""The exactness argument behind the q8_0 path of the matrix-core prefill,
replayed in binary16/binary32 arithmetic on the CPU.

The prefill kernel turns each int8 code of a q8_0 block ("KV Cache Design —
cells, format, sessions", section 3: 32 int8 codes and an f16 scale) into an
f16 value with a bit trick: the code's byte with its sign bit flipped is
u = code + 128, the f16 with bits 0x6400 | u is 1024 + u, and subtracting
1152 gives the code.  The matrix cores then multiply f16 codes by f16 query
values with f32 products, and the block scale (an f16, widened to f32) is
applied to each 32-wide partial in f32.  These tests check, exhaustively,
that every step before the f32 accumulation is exact: no scale-times-code
product is ever rounded to f16, so no f16 scale can overflow it."""

import numpy as np


def test_every_code_byte_becomes_the_exact_f16_code():
    codes = np.arange(-128, 128, dtype=np.int32)
    u = (codes.astype(np.int8).view(np.uint8) ^ 0x80).astype(np.uint16)
    biased = (np.uint16(0x6400) | u).view(np.float16)
    assert np.array_equal(biased.astype(np.float64), 1024.0 + u)
    got = (biased - np.float16(1152.0)).astype(np.float16)  # one binary16 subtraction
    assert np.array_equal(got.astype(np.float64), codes.astype(np.float64))


def test_code_times_any_f16_is_exact_in_f32():
    # every finite binary16 value (subnormals included) times every code
    q = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    q = q[np.isfinite(q)].astype(np.float32)
    for c in range(-127, 128):
        p32 = q * np.float32(c)
        p64 = q.astype(np.float64) * c
        assert np.array_equal(p32.astype(np.float64), p64), f"code {c}"


def test_every_f16_scale_widens_exactly_to_f32():
    s = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    s = s[np.isfinite(s)]
    assert np.array_equal(s.astype(np.float32).astype(np.float64), s.astype(np.float64))
    # the old widening formed scale * code as an f16 product: it overflows
    # for scales above 65504 / 127 ~ 516, which the f32 path never does
    big = np.float16(600.0)
    with np.errstate(over="ignore"):
        assert np.isinf(big * np.float16(127.0))
    assert np.isfinite(np.float32(big) * np.float32(127.0))
