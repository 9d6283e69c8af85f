"""Pins of the oracle's int4 cold-block codec.

* hand-worked blocks (tests/golden/int4_block_worked.json): exact scales
  with ties to even, an odd length, a scale that is not a power of two,
  all zeros;
* brute force in exact rational arithmetic with the IEEE roundings written
  out as scalar code, on random and near-tie blocks;
* closed forms: the largest value codes to +-7, every code is within 1/2
  of x/scale, decoded values are scale * code;
* the page's figure: cosine similarity about 0.99 between N(0, 1) blocks of
  the real block size and their decoded blocks.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.int4 import blob_bytes, cosine, decode_block, encode_block

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    with open(os.path.join(GOLDEN, "int4_block_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_worked_blocks(case):
    x = np.array([float.fromhex(v) for v in case["x"]], dtype=np.float32)
    blob = encode_block(x)
    assert blob.tolist() == case["blob"]
    assert blob.size == blob_bytes(x.size) == 4 + (x.size + 1) // 2


def _rn(a: Fraction, mant_bits: int, emin: int) -> Fraction:
    if a == 0:
        return Fraction(0)
    sign = -1 if a < 0 else 1
    a = abs(a)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - mant_bits)
    return sign * round(a / q) * q


def rn32(a):
    return _rn(Fraction(a), 23, -126)


def _brute(x):
    fx = [Fraction(float(v)) for v in x]
    amax = max(abs(v) for v in fx)
    s = rn32(amax / 7)
    if s == 0:
        return s, [0] * len(fx)
    return s, [max(-7, min(7, round(rn32(v / s)))) for v in fx]


def test_brute_force_exact_rationals():
    rng = np.random.default_rng(4)
    blocks = []
    for i in range(200):
        n = int(rng.integers(1, 40))
        x = (rng.standard_normal(n) * 2.0 ** rng.integers(-30, 10)).astype(np.float32)
        blocks.append(x)
    for i in range(100):  # values on and beside code boundaries (k + 1/2) * scale
        amax = np.float32(rng.uniform(0.1, 10))
        s = np.float32(amax / np.float32(7))
        x = ((rng.integers(-7, 7, size=24) + 0.5) * np.float64(s)).astype(np.float32)
        step = rng.integers(-1, 2, size=24)
        x = np.where(step > 0, np.nextafter(x, np.float32(np.inf)),
                     np.where(step < 0, np.nextafter(x, np.float32(-np.inf)), x)).astype(np.float32)
        x[0] = amax
        blocks.append(x)
    for x in blocks:
        s, codes = _brute(x)
        blob = encode_block(x)
        assert Fraction(float(blob[:4].view("<f4")[0])) == s
        nib = np.empty(2 * (blob.size - 4), dtype=np.int16)
        nib[0::2] = blob[4:] & 0xF
        nib[1::2] = blob[4:] >> 4
        got = np.where(nib >= 8, nib - 16, nib)[: x.size].tolist()
        assert got == codes
        if x.size % 2:
            assert blob[-1] >> 4 == 0


def test_closed_forms_and_decode():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(16384) * 3).astype(np.float32)
    blob = encode_block(x)
    s = np.float64(blob[:4].view("<f4")[0])
    dec32 = decode_block(blob, x.size, "f32")
    codes = np.rint(dec32.astype(np.float64) / s)
    assert np.all(np.abs(codes) <= 7)
    i = np.argmax(np.abs(x))
    assert codes[i] == np.sign(x[i]) * 7
    assert np.max(np.abs(x / s - codes)) <= 0.5 + 1e-5
    # decoded = scale * code in binary32, and f16 decoding rounds that once more
    assert np.array_equal(dec32, (np.float32(s) * codes.astype(np.float32)).astype(np.float32))
    assert np.array_equal(decode_block(blob, x.size, "f16"), dec32.astype(np.float16))
    with pytest.raises(ValueError):
        decode_block(blob, x.size, "q8_0")


def test_cosine_about_099_on_gaussian_blocks():
    """The page's quality figure, on blocks of the real size (16 tokens x 8
    kv heads x 128 dims = 16,384 values, one scale each)."""
    rng = np.random.default_rng(12)
    cs = []
    for _ in range(20):
        x = rng.standard_normal(16384).astype(np.float32)
        cs.append(cosine(x, decode_block(encode_block(x), x.size, "f32")))
    assert 0.97 <= min(cs) and max(cs) <= 0.995
    assert abs(np.mean(cs) - 0.99) < 0.006
