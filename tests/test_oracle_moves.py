"""Pins of the oracle's order_moves / copy_cells.

Facts: the worked example in tests/golden/order_moves_worked.json (hand
computed from the rule in "KV Cache Design — cells, format, sessions",
section 2), a row-by-row brute force that honours the ascending/descending
direction rule, and the stated safety property on compactions: a
destination never lands on a row not yet copied, so the sequential result
equals gathering every destination from the original pool at once.
"""

import itertools
import json
import os

import numpy as np

import oracle
from workloads import gen as wgen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _pool_ids(n, width=1):
    return np.repeat(np.arange(n, dtype=np.int64)[:, None], width, axis=1)


def test_golden_worked_example():
    with open(os.path.join(GOLDEN, "order_moves_worked.json")) as f:
        g = json.load(f)
    assert oracle.order_moves(g["moves"]) == g["order"]
    p = _pool_ids(g["n_rows"])
    oracle.copy_cells([p], g["moves"])
    assert p[:, 0].tolist() == g["final_rows"]
    assert oracle.provenance(g["n_rows"], g["moves"]).tolist() == g["final_rows"]
    for key in ("slide_down_overlap", "slide_up_overlap"):
        c = g[key]
        p = _pool_ids(c["n_rows"])
        oracle.copy_cells([p], c["moves"])
        assert p[:, 0].tolist() == c["final_rows"]


def test_p11_rowwise_equals_memmove_exhaustive():
    # every set of up to two moves on a 6-row pool
    n = 6
    single = [(s, d, ln) for s in range(n) for d in range(n) for ln in range(0, 4)
              if s + ln <= n and d + ln <= n]
    for k in (1, 2):
        for mv in itertools.product(single, repeat=k):
            a, b = _pool_ids(n), _pool_ids(n)
            oracle.copy_cells([a], mv)
            oracle.copy_cells_rowwise([b], mv)
            assert np.array_equal(a, b), mv


def test_p11_random_sets_rowwise_equals_memmove():
    rng = np.random.default_rng(111)
    for _ in range(200):
        n = int(rng.integers(4, 40))
        mv = []
        for _ in range(int(rng.integers(1, 8))):
            ln = int(rng.integers(0, 6))
            ln = min(ln, n)
            mv.append((int(rng.integers(0, n - ln + 1)), int(rng.integers(0, n - ln + 1)), ln))
        a, b = _pool_ids(n, 3), _pool_ids(n, 3)
        oracle.copy_cells([a], mv)
        oracle.copy_cells_rowwise([b], mv)
        assert np.array_equal(a, b)


def _compaction(rng, n_runs, gap_max, direction):
    """Runs packed with gaps; every run slides down to close the gaps (or up
    to open them): moves that neither cross nor reorder."""
    lens = rng.integers(1, 6, size=n_runs)
    gaps = rng.integers(0, gap_max + 1, size=n_runs)
    starts = np.cumsum(np.concatenate([[gaps[0]], lens[:-1] + gaps[1:]]))
    packed = np.concatenate([[0], np.cumsum(lens)[:-1]])
    moves = []
    for s, p, ln in zip(starts, packed, lens):
        if direction == "down":
            moves.append((int(s), int(p), int(ln)))
        else:
            moves.append((int(p), int(s), int(ln)))
    n = int(starts[-1] + lens[-1]) + 2
    return n, moves


def test_p12_order_moves_is_safe_on_compactions():
    rng = np.random.default_rng(12)
    for trial in range(100):
        direction = "down" if trial % 2 else "up"
        n, mv = _compaction(rng, int(rng.integers(1, 10)), 4, direction)
        mv = [mv[i] for i in rng.permutation(len(mv))]  # order of the input does not matter
        order = oracle.order_moves(mv)
        # no destination row may be written while a later move still has to read it
        pending = {}
        for i in order:
            s, d, ln = mv[i]
            for r in range(s, s + ln):
                pending[r] = pending.get(r, 0) + 1
        for i in order:
            s, d, ln = mv[i]
            for r in range(s, s + ln):
                pending[r] -= 1
            written = set(range(d, d + ln)) - set(range(s, s + ln))
            for r in written:
                assert pending.get(r, 0) == 0, (mv, i, r)
        # so the sequential result is the simultaneous gather
        a = _pool_ids(n)
        oracle.copy_cells([a], mv)
        gather = np.arange(n)
        for s, d, ln in mv:
            gather[d : d + ln] = np.arange(s, s + ln)
        assert a[:, 0].tolist() == gather.tolist()


def test_mixed_up_and_down_compaction_is_safe():
    # runs on the left slide up, runs on the right slide down, nothing crosses
    mv = [(0, 2, 3), (6, 8, 2), (20, 14, 2), (25, 17, 4)]
    a = _pool_ids(32)
    oracle.copy_cells([a], mv)
    gather = np.arange(32)
    for s, d, ln in mv:
        gather[d : d + ln] = np.arange(s, s + ln)
    assert a[:, 0].tolist() == gather.tolist()


def test_p13_provenance_reads_out_row_ids():
    ms = wgen.make_moves(seed=5, n_moves=300, n_rows=1 << 12, region=1 << 10, max_len=16)
    prov = oracle.provenance(ms.n_rows, ms.moves)
    rng = np.random.default_rng(0)
    pool = rng.integers(0, 255, size=(ms.n_rows, 12), dtype=np.uint8)
    before = pool.copy()
    oracle.copy_cells([pool], ms.moves)
    assert np.array_equal(pool, before[prov])
    # K and V pools in the block layout [blocks, kv heads, block_size, W],
    # of different widths, move together: a row is one slot of every kv head
    k = rng.standard_normal((ms.n_rows // 4, 2, 4, 3))
    v = rng.integers(0, 1 << 30, size=(ms.n_rows // 4, 3, 4, 5))
    k0, v0 = k.copy(), v.copy()
    oracle.copy_cells([k, v], ms.moves)
    r = np.arange(ms.n_rows)
    for t, t0 in ((k, k0), (v, v0)):
        assert np.array_equal(t[r // 4, :, r % 4], t0[prov // 4, :, prov % 4])


def test_move_generator_shape():
    ms = wgen.make_moves(seed=55, n_moves=2000)
    m = ms.moves
    assert m.shape == (2000, 3)
    assert (m[:, 2] >= 1).all() and (m[:, 2] <= 32).all()
    assert (m[:, 0] >= 0).all() and (m[:, 0] + m[:, 2] <= 1 << 16).all()
    assert (m[:, 1] >= 0).all() and (m[:, 1] + m[:, 2] <= ms.n_rows).all()
    assert (m[:, 0] != m[:, 1]).mean() > 0.95
