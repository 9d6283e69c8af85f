"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test names the property it pins and where the property comes from:
worked examples from the pages (fixtures under tests/golden/), closed forms
of softmax attention, brute force with scalar Python loops on tiny inputs,
and invariants the pages state (a permuted table, a hole, a window slice, a
map of runs, GQA head sharing, NaN in rows nobody may read).
"""

import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
from oracle.attention import window_candidates
from workloads import gen as wgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# brute force: scalar loops, math.exp, struct-decoded halves (independent of
# the oracle's vectorized gather and of its field-by-field f16 decoder)


def _bf_value(pool, fmt, row, kvh, d, hkv, hd):
    """Element d of kv head kvh of pool row `row`; pool is [blocks, hkv, bs, W]."""
    bs = pool.shape[2]
    cell = pool[row // bs, kvh, row % bs]
    if fmt in ("f32", "f16"):
        return float(cell[d])
    raw = cell.tobytes()
    off = (d // 32) * 34
    (scale,) = struct.unpack("<e", raw[off : off + 2])
    (code,) = struct.unpack("<b", raw[off + 2 + d % 32 : off + 3 + d % 32])
    return scale * code


def brute_attention(q, q_seq, q_pos, kpool, vpool, kfmt, vfmt, table, seq_lens, bs, hkv, hd,
                    scale, mode, window=None, kv_map=None):
    nq, hq, _ = q.shape
    g = hq // hkv
    out = [[[0.0] * hd for _ in range(hq)] for _ in range(nq)]
    lse = [[0.0] * hq for _ in range(nq)]
    for j in range(nq):
        s = int(q_seq[j])
        L = int(seq_lens[s])
        limit = min(L, int(q_pos[j]) + 1)
        if mode == "causal":
            cand = list(range(L))
        elif mode == "span":
            cand = list(range(int(window[s][0]), int(window[s][1])))
        else:
            cand = []
            for c, n in kv_map[s]:
                for t in range(int(c), int(c) + int(n)):
                    cand.append(t)
        rows = []
        for t in cand:
            if t < 0 or t >= limit:
                continue
            blk = int(table[s][t // bs])
            if blk == -1:
                continue
            rows.append(blk * bs + t % bs)
        for h in range(hq):
            kvh = h // g
            if not rows:
                lse[j][h] = -math.inf
                continue
            xs = []
            for r in rows:
                acc = 0.0
                for d in range(hd):
                    acc += float(q[j, h, d]) * _bf_value(kpool, kfmt, r, kvh, d, hkv, hd)
                xs.append(scale * acc)
            m = max(xs)
            ws = [math.exp(x - m) for x in xs]
            z = sum(ws)
            for d in range(hd):
                acc = 0.0
                for w, r in zip(ws, rows):
                    acc += w * _bf_value(vpool, vfmt, r, kvh, d, hkv, hd)
                out[j][h][d] = acc / z
            lse[j][h] = m + math.log(z)
    return np.array(out), np.array(lse)


def _tiny_case(seed, mode, kfmt="f32", vfmt="f32", hkv=2, g=2, hd=32, bs=4, nseq=2, nq_per=3):
    """A tiny random paged case with holes, a partial last block, NaN garbage
    in unused rows, and windows of the requested mode."""
    import torch

    rng = np.random.default_rng(seed)
    pool_blocks = 12
    mb = 5
    seq_lens = rng.integers(bs + 1, mb * bs + 1, size=nseq).astype(np.int32)
    perm = rng.permutation(pool_blocks)
    table = np.full((nseq, mb), -1, dtype=np.int32)
    off = 0
    for s in range(nseq):
        nb = -(-int(seq_lens[s]) // bs)
        table[s, :nb] = perm[off : off + nb]
        off += nb
    table[0, 1] = -1  # a hole
    w = wgen.Workload(name="tiny", cfg=0, seed=seed, n_seqs=nseq, n_q_heads=hkv * g, n_kv_heads=hkv,
                      head_dim=hd, block_size=bs, n_pool_blocks=pool_blocks, q_fmt="f32",
                      k_fmt=kfmt, v_fmt=vfmt, scale=1.0 / math.sqrt(hd), block_table=table,
                      seq_lens=seq_lens, mode=mode, kind="prefill")
    w.cu_q = (np.arange(nseq + 1) * nq_per).astype(np.int32)
    w.q_pos = np.concatenate([np.sort(rng.choice(int(L), size=nq_per, replace=False))
                              for L in seq_lens]).astype(np.int32)
    w.window = np.stack([np.sort(rng.integers(-2, int(L) + 3, size=2)) for L in seq_lens]).astype(np.int32)
    km = np.zeros((nseq, 3, 2), dtype=np.int32)
    for s in range(nseq):
        L = int(seq_lens[s])
        km[s, 0] = (0, min(3, L))
        km[s, 1] = (max(0, L - 5), 5)
        km[s, 2] = (2, 0)
    km[1, 2] = (1, 2)  # overlaps run 0 of seq 1: counted twice
    w.kv_map = km
    q, k, v = wgen.materialize(w, "cpu")
    return w, q.numpy(), k.numpy(), v.numpy()


def _oracle(w, q, k, v, mode=None):
    return oracle.paged_attention(q, w.q_seq(), w.query_pos(), k, v, w.k_fmt, w.v_fmt,
                                  w.block_table, w.seq_lens, w.block_size, w.n_kv_heads,
                                  w.head_dim, w.scale, mode or w.mode, w.window, w.kv_map)


@pytest.mark.parametrize("mode", ["causal", "span", "kv_map"])
@pytest.mark.parametrize("kfmt,vfmt", [("f32", "f32"), ("f16", "f16"), ("q8_0", "f16")])
def test_p1_brute_force(mode, kfmt, vfmt):
    w, q, k, v = _tiny_case(11, mode, kfmt, vfmt)
    out, lse = _oracle(w, q, k, v)
    bo, bl = brute_attention(q, w.q_seq(), w.query_pos(), k, v, kfmt, vfmt, w.block_table, w.seq_lens,
                             w.block_size, w.n_kv_heads, w.head_dim, w.scale, mode, w.window, w.kv_map)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(out - bo)) <= 1e-12
    assert np.max(np.abs(lse[fin] - bl[fin])) <= 1e-12
    assert np.all(out[~fin] == 0.0)


def test_golden_block_table_figure():
    gdat = golden("block_table_figure.json")
    table = np.array(gdat["table"], dtype=np.int32)
    rows = oracle.physical_row(table, np.array(gdat["positions"]), gdat["block_size"])
    assert rows.tolist() == gdat["expected_rows"]


def test_golden_q8_0_row_bytes():
    for c in golden("q8_0_row_bytes.json")["cases"]:
        assert oracle.seg_bytes("q8_0", c["head_dim"]) == c["segment_bytes"]
        assert oracle.row_bytes("q8_0", c["n_kv_heads"], c["head_dim"]) == c["row_bytes"]
        assert wgen.q8_0_row_bytes(c["n_kv_heads"], c["head_dim"]) == c["row_bytes"]
    assert oracle.row_bytes("f16", 8, 128) == 2048
    assert oracle.row_bytes("f32", 2, 64) == 512


def _dense_to_paged(Kd, Vd, bs, perm):
    """Dense [L, hkv, hd] K/V into a paged pool whose logical block b sits in
    physical block perm[b] (p3's contiguous layout is perm = identity)."""
    L, hkv, hd = Kd.shape
    nb = -(-L // bs)
    pool_k = np.full((len(perm), hkv, bs, hd), np.nan)
    pool_v = np.full((len(perm), hkv, bs, hd), np.nan)
    for b in range(nb):
        n = min(bs, L - b * bs)
        pool_k[perm[b], :, :n] = Kd[b * bs : b * bs + n].transpose(1, 0, 2)
        pool_v[perm[b], :, :n] = Vd[b * bs : b * bs + n].transpose(1, 0, 2)
    table = np.array([perm[:nb]], dtype=np.int32)
    return pool_k, pool_v, table


def test_p2_permuted_table_equals_contiguous():
    rng = np.random.default_rng(2)
    L, hkv, hd, bs, g = 83, 2, 16, 8, 3
    Kd, Vd = rng.standard_normal((L, hkv, hd)), rng.standard_normal((L, hkv, hd))
    q = rng.standard_normal((1, hkv * g, hd))
    nb = -(-L // bs)
    ident = np.arange(nb + 3)
    perm = rng.permutation(nb + 3)
    res = []
    for p in (ident, perm):
        pk, pv, table = _dense_to_paged(Kd, Vd, bs, p)
        res.append(oracle.paged_decode(q, pk, pv, "f32", "f32", table, np.array([L]), bs, hkv, hd, 0.3))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    # and both equal attention over the dense rows directly
    for kvh in range(hkv):
        o, l = oracle.attend(q[0, kvh * g : (kvh + 1) * g], Kd[:, kvh], Vd[:, kvh], 0.3)
        assert np.max(np.abs(res[1][0][0, kvh * g : (kvh + 1) * g] - o)) <= 1e-13
        assert np.max(np.abs(res[1][1][0, kvh * g : (kvh + 1) * g] - l)) <= 1e-13


def test_p3_hole_equals_deleting_positions():
    rng = np.random.default_rng(3)
    L, hkv, hd, bs, g = 70, 1, 8, 8, 2
    Kd, Vd = rng.standard_normal((L, hkv, hd)), rng.standard_normal((L, hkv, hd))
    q = rng.standard_normal((1, hkv * g, hd))
    perm = rng.permutation(12)
    pk, pv, table = _dense_to_paged(Kd, Vd, bs, perm)
    holes = [2, 5]
    for b in holes:
        pk[table[0, b]] = np.nan
        table[0, b] = -1
    out, lse = oracle.paged_decode(q, pk, pv, "f32", "f32", table, np.array([L]), bs, hkv, hd, 0.5)
    keep = np.array([t for t in range(L) if t // bs not in holes])
    o, l = oracle.attend(q[0], Kd[keep, 0], Vd[keep, 0], 0.5)
    assert np.max(np.abs(out[0] - o)) <= 1e-12 and np.max(np.abs(lse[0] - l)) <= 1e-12


def test_p4_span_is_slice_and_map_is_concatenation():
    rng = np.random.default_rng(4)
    L, hkv, hd, bs, g = 97, 2, 16, 16, 2
    Kd, Vd = rng.standard_normal((L, hkv, hd)), rng.standard_normal((L, hkv, hd))
    q = rng.standard_normal((1, hkv * g, hd))
    pk, pv, table = _dense_to_paged(Kd, Vd, bs, rng.permutation(10))
    lo, hi = 13, 61
    out, _ = oracle.paged_decode(q, pk, pv, "f32", "f32", table, np.array([L]), bs, hkv, hd, 0.25,
                                 mode="span", window=np.array([[lo, hi]]))
    for kvh in range(hkv):
        o, _ = oracle.attend(q[0, kvh * g : (kvh + 1) * g], Kd[lo:hi, kvh], Vd[lo:hi, kvh], 0.25)
        assert np.max(np.abs(out[0, kvh * g : (kvh + 1) * g] - o)) <= 1e-12
    runs = np.array([[[0, 9], [40, 3], [70, 27], [5, 0]]])
    out, _ = oracle.paged_decode(q, pk, pv, "f32", "f32", table, np.array([L]), bs, hkv, hd, 0.25,
                                 mode="kv_map", kv_map=runs)
    idx = np.concatenate([np.arange(0, 9), np.arange(40, 43), np.arange(70, 97)])
    for kvh in range(hkv):
        o, _ = oracle.attend(q[0, kvh * g : (kvh + 1) * g], Kd[idx, kvh], Vd[idx, kvh], 0.25)
        assert np.max(np.abs(out[0, kvh * g : (kvh + 1) * g] - o)) <= 1e-12
    # a span clamps to [0, seq_len): [-5, 200) reads the whole sequence
    a, _ = oracle.paged_decode(q, pk, pv, "f32", "f32", table, np.array([L]), bs, hkv, hd, 0.25,
                               mode="span", window=np.array([[-5, 200]]))
    b, _ = oracle.paged_decode(q, pk, pv, "f32", "f32", table, np.array([L]), bs, hkv, hd, 0.25)
    assert np.array_equal(a, b)


def test_kv_map_duplicate_run_counts_twice():
    # listing a position twice gives it twice the weight (multiset reading)
    rng = np.random.default_rng(41)
    L, hd, bs = 20, 8, 4
    Kd, Vd = rng.standard_normal((L, 1, hd)), rng.standard_normal((L, 1, hd))
    q = rng.standard_normal((1, 1, hd))
    pk, pv, table = _dense_to_paged(Kd, Vd, bs, np.arange(5))
    out, _ = oracle.paged_decode(q, pk, pv, "f32", "f32", table, np.array([L]), bs, 1, hd, 1.0,
                                 mode="kv_map", kv_map=np.array([[[3, 2], [3, 1]]]))
    x = Kd[[3, 4], 0] @ q[0, 0]
    w = np.exp(x - x.max()) * np.array([2.0, 1.0])
    expect = (w[:, None] * Vd[[3, 4], 0]).sum(0) / w.sum()
    assert np.max(np.abs(out[0, 0] - expect)) <= 1e-13


def test_p5_closed_forms():
    rng = np.random.default_rng(5)
    L, hd, bs = 45, 8, 8
    Kd, Vd = rng.standard_normal((L, 1, hd)), rng.standard_normal((L, 1, hd))
    pk, pv, table = _dense_to_paged(Kd, Vd, bs, rng.permutation(8))
    # q = 0: plain mean of the visible values
    out, lse = oracle.paged_decode(np.zeros((1, 1, hd)), pk, pv, "f32", "f32", table, np.array([L]), bs, 1, hd, 1.0)
    assert np.max(np.abs(out[0, 0] - Vd[:, 0].mean(0))) <= 1e-13
    assert abs(lse[0, 0] - math.log(L)) <= 1e-13
    # one visible slot: that value row, exactly
    q = rng.standard_normal((1, 1, hd))
    out, lse = oracle.paged_decode(q, pk, pv, "f32", "f32", table, np.array([L]), bs, 1, hd, 1.0,
                                   mode="span", window=np.array([[17, 18]]))
    assert np.array_equal(out[0, 0], Vd[17, 0])
    assert abs(lse[0, 0] - float(Kd[17, 0] @ q[0, 0])) <= 1e-13
    # all value rows equal c: the output is c
    c = rng.standard_normal(hd)
    pv2 = pv.copy()
    pv2[np.isfinite(pv2).all(axis=3)] = c
    out, _ = oracle.paged_decode(q, pk, pv2, "f32", "f32", table, np.array([L]), bs, 1, hd, 1.0)
    assert np.max(np.abs(out[0, 0] - c)) <= 1e-13
    # identical keys: uniform weights
    pk2 = pk.copy()
    pk2[np.isfinite(pk2).all(axis=3)] = rng.standard_normal(hd)
    out, _ = oracle.paged_decode(q, pk2, pv, "f32", "f32", table, np.array([L]), bs, 1, hd, 1.0)
    assert np.max(np.abs(out[0, 0] - Vd[:, 0].mean(0))) <= 1e-13
    # empty window: out 0, lse -inf
    out, lse = oracle.paged_decode(q, pk, pv, "f32", "f32", table, np.array([L]), bs, 1, hd, 1.0,
                                   mode="span", window=np.array([[30, 30]]))
    assert np.all(out == 0) and lse[0, 0] == -np.inf


def test_p6_split_invariance_of_lse_merge():
    rng = np.random.default_rng(6)
    n, hd, g = 300, 16, 4
    K, V = rng.standard_normal((n, hd)), rng.standard_normal((n, hd))
    q = rng.standard_normal((g, hd)) * 2
    full = oracle.attend(q, K, V, 0.7)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, n), size=trial + 2, replace=False))
        idx = rng.permutation(n)
        parts = [oracle.attend(q, K[p], V[p], 0.7) for p in np.split(idx, cuts)]
        parts.append(oracle.attend(q, K[:0], V[:0], 0.7))  # an empty part weighs nothing
        out, lse = oracle.lse_merge(parts)
        assert np.max(np.abs(out - full[0])) <= 1e-13
        assert np.max(np.abs(lse - full[1])) <= 1e-13
    e = oracle.lse_merge([oracle.attend(q, K[:0], V[:0], 0.7)] * 2)
    assert np.all(e[0] == 0) and np.all(e[1] == -np.inf)


def test_p7_gqa_equals_mha_with_repeated_heads():
    w, q, k, v = _tiny_case(7, "causal", hkv=2, g=3)
    out, lse = _oracle(w, q, k, v)
    g = w.group
    # repeat kv head h // g for every q head h: an MHA pool with hq kv heads
    k2 = np.repeat(k, g, axis=1)
    v2 = np.repeat(v, g, axis=1)
    out2, lse2 = oracle.paged_attention(q, w.q_seq(), w.query_pos(), k2, v2, "f32", "f32",
                                        w.block_table, w.seq_lens, w.block_size, w.n_q_heads,
                                        w.head_dim, w.scale, "causal")
    # equal up to float64 rounding of differently blocked products; a wrong
    # head mapping would differ by O(1)
    assert np.max(np.abs(out - out2)) <= 1e-13 and np.max(np.abs(lse - lse2)) <= 1e-13


@pytest.mark.parametrize("kfmt", ["f32", "q8_0"])
def test_p8_nan_garbage_is_never_read(kfmt):
    w, q, k, v = _tiny_case(8, "causal", kfmt, "f32")
    live = wgen.referenced_rows(w)
    assert not live.all()
    out, lse = _oracle(w, q, k, v)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    # the generator really poisoned the dead rows (cells of every kv head)
    bs = w.block_size
    rows = np.arange(len(live))
    cells = v[rows // bs, :, rows % bs]
    assert np.all(np.isnan(cells[~live])) and np.all(np.isfinite(cells[live]))
    # replacing the garbage by anything else changes nothing
    v2 = v.copy()
    dead = rows[~live]
    v2[dead // bs, :, dead % bs] = 1e30
    out2, _ = _oracle(w, q, k, v2)
    assert np.array_equal(out, out2)


def test_p9_q8_0_decode_and_encoder_bound():
    import torch

    rng = np.random.default_rng(9)
    hkv, hd, n = 3, 64, 200
    x = rng.standard_normal((n, hkv, hd)).astype(np.float32)
    x[0, 0, :32] = 0.0  # an all-zero block: scale 0, codes 0
    x[1, 1, 5] = 1e-3
    enc = wgen.encode_q8_0(torch.from_numpy(x), hkv, hd).numpy()
    assert enc.shape == (n, hkv, oracle.seg_bytes("q8_0", hd))
    enc = enc[:, :, None, :]  # a pool of n one-token blocks
    dec = oracle.decode_rows(enc, "q8_0", np.arange(n), hkv, hd)
    # decoding equals scale * code read with struct (Python's own binary16)
    for r in (0, 1, 77, 199):
        for h in range(hkv):
            for d in (0, 31, 32, 63):
                assert dec[r, h, d] == _bf_value(enc, "q8_0", r, h, d, hkv, hd)
    xb = x.reshape(n, hkv, hd // 32, 32).astype(np.float64)
    d = np.abs(xb).max(-1, keepdims=True) / 127.0
    err = np.abs(xb - dec.reshape(xb.shape))
    bound = d / 2 + 2.0 ** -11 * (np.abs(xb) + d / 2) + 1e-12
    assert np.all(err <= bound)
    assert np.all(dec[0, 0, :32] == 0.0)
    # codes stay in [-127, 127] and the block max hits +-127
    codes = enc[:, :, 0, : 2 * 34].reshape(n, hkv * 2, 34)[:, :, 2:].view(np.int8)
    assert codes.min() >= -127 and codes.max() <= 127
    assert np.all(np.abs(codes.astype(np.int32)).max(-1)[1:] == 127)


def test_f16_decoder_matches_struct():
    bits = np.array([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0xBC00, 0x7BFF, 0x3555, 0xC800], dtype=np.uint16)
    got = oracle.f16_bits_to_f64(bits)
    for b, v in zip(bits, got):
        assert v == struct.unpack("<e", int(b).to_bytes(2, "little"))[0]
    assert np.isinf(oracle.f16_bits_to_f64(np.array([0x7C00], dtype=np.uint16)))[0]
    assert np.isnan(oracle.f16_bits_to_f64(np.array([0x7E00], dtype=np.uint16)))[0]


def test_resolver_brute_force():
    w, q, k, v = _tiny_case(10, "kv_map")
    for mode in ("causal", "span", "kv_map"):
        n_cand = w.max_blocks_per_seq * w.block_size + 4
        got = oracle.resolve_rows(mode, w.block_table, w.seq_lens, w.block_size, w.q_seq(),
                                  w.query_pos(), n_cand, w.window, w.kv_map)
        for j, s in enumerate(w.q_seq()):
            cand = window_candidates(mode, int(w.seq_lens[s]), w.window[s], w.kv_map[s])
            limit = min(int(w.seq_lens[s]), int(w.query_pos()[j]) + 1)
            for i in range(n_cand):
                if i >= len(cand) or not (0 <= cand[i] < limit):
                    assert got[j, i] == -1
                    continue
                t = int(cand[i])
                blk = int(w.block_table[s][t // w.block_size])
                assert got[j, i] == (-1 if blk == -1 else blk * w.block_size + t % w.block_size)
