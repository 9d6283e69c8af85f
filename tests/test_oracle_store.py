"""Pins of the oracle's store and q8_0 quantizer against facts fixed outside it.

* hand-worked blocks (tests/golden/q8_0_store_worked.json): exact scales,
  ties to even, subnormal and flushed scales, all-zero blocks;
* brute force in exact rational arithmetic: every rounding step (binary32,
  binary16, ties-to-even to an integer) done by a scalar routine written
  here from the IEEE definitions, not by numpy;
* closed forms: the code of the largest value is +-127, every code is within
  1/2 of x/d, the dequantized error bound;
* an independent encoder (the input generator's, written with torch);
* placement: a store through a block table puts each token's row where
  position t -> (table[t // bs], t % bs) says, leaves every other byte
  alone, skips tokens without a block, and attention over the stored pools
  equals attention over the same rows laid out densely.
"""

import json
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.store import destination_rows, encode_rows, quantize_q8_0, store_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_cases():
    with open(os.path.join(GOLDEN, "q8_0_store_worked.json")) as f:
        return json.load(f)["cases"]


def _block_of(case):
    x = np.zeros(32, dtype=np.float32)
    for i, v in case["x"].items():
        x[int(i)] = np.float32(float.fromhex(v))
    codes = np.zeros(32, dtype=np.int8)
    for i, v in case["codes"].items():
        codes[int(i)] = v
    return x, codes


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_quantizer_worked_blocks(case):
    x, codes = _block_of(case)
    b = quantize_q8_0(x[None])[0]
    assert b.shape == (36,)  # 34 bytes rounded up to whole words
    assert int(b[0]) | (int(b[1]) << 8) == case["scale_bits"]
    assert np.array_equal(b[2:34].view(np.int8), codes)
    assert b[34] == 0 and b[35] == 0


def test_quantizer_block_order_in_a_segment():
    """Seven worked blocks side by side: head_dim 224, segment 7 * 34 = 238
    bytes rounded to 240; block j sits at bytes 34j .. 34j + 33."""
    cases = _golden_cases()
    xs, cs = zip(*(_block_of(c) for c in cases))
    seg = quantize_q8_0(np.concatenate(xs)[None])[0]
    assert seg.shape == (240,)
    for j, c in enumerate(cases):
        blk = seg[34 * j : 34 * j + 34]
        assert int(blk[0]) | (int(blk[1]) << 8) == c["scale_bits"]
        assert np.array_equal(blk[2:].view(np.int8), cs[j])
    assert np.all(seg[238:] == 0)


# ---------------------------------------------------------------------------
# brute force: exact rationals, IEEE rounding written out


def _round_binary(a: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Nearest value with mant_bits fraction bits and minimum normal exponent
    emin (subnormals below), ties to even."""
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
    quantum = Fraction(2) ** (e - mant_bits)
    return sign * round(a / quantum) * quantum  # Fraction.__round__: ties to even


def rn32(a):
    return _round_binary(Fraction(a), 23, -126)


def rn16(a):
    return _round_binary(Fraction(a), 10, -14)


def brute_block(x):
    """(scale_bits, codes) of 32 binary32 values by the stated reading."""
    fx = [Fraction(float(v)) for v in x]
    amax = max(abs(v) for v in fx)
    d = rn32(amax / 127)
    if d == 0:
        return 0, [0] * 32
    codes = [max(-127, min(127, round(rn32(v / d)))) for v in fx]
    (bits,) = struct.unpack("<H", struct.pack("<e", float(rn16(d))))  # exact: already a half
    return bits, codes


def _near_tie_blocks(rng, n):
    """Blocks whose values sit on, or one binary32 step beside, the code
    boundaries (k + 1/2) * d."""
    out = []
    for _ in range(n):
        amax = np.float32(rng.uniform(0.05, 4.0))
        d = np.float32(amax / np.float32(127))
        k = rng.integers(-126, 126, size=32)
        x = ((k + 0.5) * np.float64(d)).astype(np.float32)
        step = rng.integers(-1, 2, size=32)
        up = np.nextafter(x, np.float32(np.inf))
        down = np.nextafter(x, np.float32(-np.inf))
        x = np.where(step > 0, up, np.where(step < 0, down, x)).astype(np.float32)
        x[0] = amax
        out.append(x)
    return out


def _random_blocks(rng, n):
    """N(0,1) blocks at several magnitudes, down to f16-subnormal and
    flushed scales, plus blocks with exact zeros."""
    out = []
    for i in range(n):
        x = rng.standard_normal(32).astype(np.float32)
        x *= np.float32(2.0 ** rng.integers(-28, 8))
        if i % 7 == 0:
            x[rng.integers(0, 32, size=8)] = 0
        out.append(x.astype(np.float32))
    out.append(np.zeros(32, dtype=np.float32))
    return out


def test_quantizer_brute_force_exact_rationals():
    rng = np.random.default_rng(1234)
    blocks = _random_blocks(rng, 300) + _near_tie_blocks(rng, 150)
    got = quantize_q8_0(np.stack(blocks))
    ties = 0
    for x, b in zip(blocks, got):
        bits, codes = brute_block(x)
        assert int(b[0]) | (int(b[1]) << 8) == bits
        assert b[2:34].view(np.int8).tolist() == codes
    # the near-tie blocks do land on exact binary32 ties
    for x in _near_tie_blocks(np.random.default_rng(5), 20):
        d = rn32(Fraction(float(max(abs(x)))) / 127)
        ties += sum(1 for v in x if (rn32(Fraction(float(v)) / d) * 2).denominator == 1
                    and (rn32(Fraction(float(v)) / d) * 2).numerator % 2 == 1)
    assert ties > 50


# ---------------------------------------------------------------------------
# closed forms


def test_quantizer_closed_forms():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 4, 128)) * 3).astype(np.float32)
    q = quantize_q8_0(x).reshape(64, 4, 4, 34)
    codes = q[..., 2:].view(np.int8).astype(np.int64)
    blocks = x.reshape(64, 4, 4, 32)
    amax = np.abs(blocks).max(-1)
    d = (amax / np.float32(127)).astype(np.float64)
    # the largest magnitude maps to +-127 and every code is within 1/2 (plus
    # the binary32 rounding of x/d) of x/d
    arg = np.abs(blocks).argmax(-1)
    top = np.take_along_axis(codes, arg[..., None], -1)[..., 0]
    top_x = np.take_along_axis(blocks, arg[..., None], -1)[..., 0]
    assert np.all(top == np.sign(top_x) * 127)
    assert np.all(np.abs(blocks / d[..., None] - codes) <= 0.5 + 1e-5)
    # decoded through the pinned reader: |x - s*c| <= d/2 + 127 |s - d| (+ a
    # relative 2^-20 for the binary32 steps)
    s = oracle.f16_bits_to_f64(q[..., 0].astype(np.uint16) | (q[..., 1].astype(np.uint16) << 8))
    pool = quantize_q8_0(x)[:, :, None, :]  # [64 blocks, 4 heads, 1 slot, 136 bytes]
    dec = oracle.decode_rows(pool, "q8_0", np.arange(64), 4, 128).reshape(64, 4, 4, 32)
    bound = d / 2 + 127 * np.abs(s - d) + amax * 2.0 ** -20
    assert np.all(np.abs(dec - blocks) <= bound[..., None])


def test_quantizer_matches_independent_encoder():
    """The input generator's torch encoder implements the same reading
    separately; both must give the same bytes."""
    import torch

    from workloads import gen as wgen

    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, 8, 128)).astype(np.float32)
    x[3] *= np.float32(1e-6)
    x[4] = 0
    ref = wgen.encode_q8_0(torch.from_numpy(x), 8, 128).numpy()
    assert np.array_equal(quantize_q8_0(x), ref)


def test_encode_rows_formats():
    x = np.array([[1.0, 2.0 ** -25, 65519.0, 1 + 2.0 ** -11]], dtype=np.float32)
    assert encode_rows(x, "f32").dtype == np.float32 and np.array_equal(encode_rows(x, "f32"), x)
    h = encode_rows(x, "f16")
    # 2^-25 is half the smallest subnormal: tie to even -> 0; 65519 rounds to
    # 65504 (below the overflow threshold 65520); 1 + 2^-11 is a tie -> 1
    assert h.dtype == np.float16
    assert h.view(np.uint16).tolist() == [[0x3C00, 0x0000, 0x7BFF, 0x3C00]]
    with pytest.raises(ValueError):
        encode_rows(x, "q4")


# ---------------------------------------------------------------------------
# placement through the block table


def _pools(rng, nblk, hkv, bs, hd, kfmt, vfmt):
    """Pools [nblk, hkv, bs, W] filled with random bytes (NaN patterns
    included), so that an untouched byte is recognisable."""
    def one(fmt):
        dt = np.dtype({"f32": np.float32, "f16": np.float16, "q8_0": np.uint8}[fmt])
        nbytes = oracle.seg_bytes(fmt, hd)
        return rng.integers(0, 256, size=(nblk, hkv, bs, nbytes), dtype=np.uint8).view(dt)
    return one(kfmt), one(vfmt)


@pytest.mark.parametrize("kfmt,vfmt", [("f32", "f32"), ("f16", "f16"), ("q8_0", "f16"), ("q8_0", "f32")])
def test_store_places_rows_by_scalar_index(kfmt, vfmt):
    rng = np.random.default_rng(3)
    nblk, hkv, bs, hd, S, mb = 12, 2, 4, 64, 3, 5
    kp, vp = _pools(rng, nblk, hkv, bs, hd, kfmt, vfmt)
    table = np.array([[7, 2, -1, 11, 0], [3, 3, 5, -1, -1], [1, 9, 4, 6, 8]], dtype=np.int32)
    seq = np.array([0, 0, 0, 1, 1, 2, 2, 2, 0], dtype=np.int32)
    pos = np.array([0, 5, 13, 2, 9, 19, 4, 17, 9], dtype=np.int32)
    # token 2: position 13 -> block 3 -> pool block 11 slot 1; token 4: seq 1
    # position 9 -> logical block 2 -> pool block 5 slot 1; token 8: seq 0
    # position 9 -> logical block 2 = hole (skipped)
    k_new = rng.standard_normal((len(pos), hkv, hd)).astype(np.float32)
    v_new = rng.standard_normal((len(pos), hkv, hd)).astype(np.float32)
    k2, v2, skipped = store_rows(kp, vp, kfmt, vfmt, k_new, v_new, seq, pos, table)
    assert skipped == 1
    touched = set()
    for t in range(len(pos)):
        s, p = int(seq[t]), int(pos[t])
        blk = int(table[s][p // bs])
        if blk < 0:
            continue
        slot = p - (p // bs) * bs
        touched.add((blk, slot))
        for h in range(hkv):
            for pool, new, fmt in ((k2, k_new, kfmt), (v2, v_new, vfmt)):
                cell = pool[blk, h, slot]
                if fmt == "f32":
                    assert cell.tolist() == new[t, h].tolist()
                elif fmt == "f16":
                    assert np.array_equal(cell.astype(np.float64), new[t, h].astype(np.float16).astype(np.float64))
                else:
                    raw = cell.tobytes()
                    for e in range(hd):
                        off = (e // 32) * 34
                        (sc,) = struct.unpack("<e", raw[off : off + 2])
                        (c,) = struct.unpack("<b", raw[off + 2 + e % 32 : off + 3 + e % 32])
                        assert abs(sc * c - float(new[t, h, e])) <= 0.5 * sc + 2e-3 * abs(float(new[t, h, e])) + 1e-3
    # every other byte unchanged, bit for bit
    for b in range(nblk):
        for slot in range(bs):
            if (b, slot) in touched:
                continue
            assert kp[b, :, slot].tobytes() == k2[b, :, slot].tobytes()
            assert vp[b, :, slot].tobytes() == v2[b, :, slot].tobytes()


def test_store_skips_tokens_without_a_block():
    table = np.array([[0, -1, 5, 9]], dtype=np.int32)  # 9 is past a 6-block pool
    seq = np.array([0, 0, 0, 0, 1, -1, 0, 0], dtype=np.int32)
    pos = np.array([0, 4, 8, 12, 0, 0, -1, 16], dtype=np.int32)
    rows = destination_rows(seq, pos, table, n_pool_blocks=6, block_size=4)
    assert rows.tolist() == [0, -1, 20, -1, -1, -1, -1, -1]


def test_store_then_attention_equals_dense_rows():
    """A sequence stored through a permuted table reads back, through the
    attention oracle, exactly like the same rows stored contiguously."""
    rng = np.random.default_rng(9)
    hq, hkv, hd, bs, L = 4, 2, 64, 16, 150
    nblk = 24
    for kfmt, vfmt in (("f16", "f16"), ("q8_0", "f16"), ("f32", "f32")):
        k_new = rng.standard_normal((L, hkv, hd)).astype(np.float32)
        v_new = rng.standard_normal((L, hkv, hd)).astype(np.float32)
        q = rng.standard_normal((1, hq, hd)).astype(np.float32)
        results = []
        for table_row in (np.arange(10), rng.permutation(nblk)[:10]):
            table = table_row.astype(np.int32)[None]
            kp, vp = _pools(rng, nblk, hkv, bs, hd, kfmt, vfmt)
            kp, vp, sk = store_rows(kp, vp, kfmt, vfmt, k_new, v_new, np.zeros(L, np.int32),
                                    np.arange(L, dtype=np.int32), table)
            assert sk == 0
            out, lse = oracle.paged_decode(q, kp, vp, kfmt, vfmt, table, np.array([L]), bs, hkv, hd,
                                           0.125)
            results.append((out, lse))
        assert np.array_equal(results[0][0], results[1][0]) and np.array_equal(results[0][1], results[1][1])
        # and both equal plain attention over the dense decoded rows
        dense_k = oracle.decode_rows(encode_rows(k_new, kfmt)[:, :, None, :], kfmt, np.arange(L), hkv, hd)
        dense_v = oracle.decode_rows(encode_rows(v_new, vfmt)[:, :, None, :], vfmt, np.arange(L), hkv, hd)
        for h in range(hq):
            o, l = oracle.attend(q[0, h][None].astype(np.float64), dense_k[:, h // 2], dense_v[:, h // 2], 0.125)
            assert np.allclose(results[0][0][0, h], o[0], atol=1e-12, rtol=0)
