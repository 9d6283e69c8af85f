"""The host half of copy_cells (pkv_copy_cells_plan) without a GPU: each plan
is applied here in numpy, exactly as the device kernels read it (run plans
as simultaneous gathers; staged-row plans as a gather into the stage and
then a scatter whose reads all precede its writes), and the rows it leaves
must equal the oracle's sequential application of the moves in order_moves
order ("KV Cache Design — cells, format, sessions", section 2) — bit for
bit, read out as row provenance."""

import ctypes

import numpy as np
import pytest

import oracle
import paged_kv_cache_table_amd as pkv


def plan_of(moves, n_rows):
    mv = np.ascontiguousarray(np.asarray(moves, dtype=np.int32).reshape(-1, 3))
    L = pkv.lib()
    words = L.pkv_copy_cells_plan_words(mv.ctypes.data, mv.shape[0])
    buf = np.zeros(max(words, 1) + 1, dtype=np.int64).view(np.int32)[: max(words, 1)]  # 8-byte aligned
    info = pkv.CopyPlan()
    st = L.pkv_copy_cells_plan(mv.ctypes.data, mv.shape[0], n_rows, buf.ctypes.data, words, ctypes.byref(info))
    assert st == 0, pkv.last_error()
    return info, buf[: info.n_words].copy()


def apply_plan(info, plan, n_rows):
    """Provenance after applying the plan to rows holding their own index."""
    rows = np.arange(n_rows, dtype=np.int64)
    if info.kind == 1:
        m = info.n_moves
        mv = plan[: 3 * m].reshape(m, 3)
        cum = plan[3 * m : 4 * m + 1]
        assert cum[0] == 0 and np.array_equal(np.diff(cum), mv[:, 2]) and cum[-1] == info.total_rows
        before = rows.copy()
        written = np.zeros(n_rows, dtype=bool)
        for s, d, n in mv.tolist():
            assert not written[d : d + n].any(), "a run plan writes a row twice"
            written[d : d + n] = True
            rows[d : d + n] = before[s : s + n]
        src = np.concatenate([np.arange(s, s + n) for s, _, n in mv.tolist()])
        assert not written[src].any(), "a run plan reads a row it writes"
    elif info.kind == 2:
        g = plan[: 2 * info.n_gather].reshape(-1, 2)
        sc = plan[2 * info.n_gather : 2 * (info.n_gather + info.n_scatter)].reshape(-1, 2)
        assert np.array_equal(g[:, 1], np.arange(info.n_gather)), "stage slots are 0..n_gather-1 in order"
        stage = np.concatenate([rows[g[:, 0]], [-1]])  # one spare entry so both branches index safely
        dst = sc[:, 0]
        assert len(np.unique(dst)) == len(dst), "a row is written twice"
        src = sc[:, 1]
        from_pool = src >= 0
        assert not np.isin(src[from_pool], dst).any(), "a scatter reads a row it writes"
        vals = np.where(from_pool, rows[np.maximum(src, 0)], stage[np.maximum(-src - 1, 0)])
        rows[dst] = vals
    else:
        assert info.kind == 0 and info.n_words == 0
    return rows


def check(moves, n_rows):
    info, plan = plan_of(moves, n_rows)
    got = apply_plan(info, plan, n_rows)
    want = oracle.provenance(n_rows, moves)
    assert np.array_equal(got, want)
    return info


@pytest.mark.parametrize("seed", range(40))
def test_random_overlapping_moves(seed):
    rng = np.random.default_rng(seed)
    n_rows = int(rng.choice([64, 300, 2048]))
    n = int(rng.integers(1, 60))
    ln = rng.integers(-1, 20, n)
    src = rng.integers(0, n_rows, n)
    mode = seed % 3
    if mode == 0:  # slides: each move overlaps itself
        dst = src + rng.integers(-2 * 20, 2 * 20 + 1, n)
    else:
        dst = rng.integers(0, n_rows, n)
    ln = np.minimum(ln, n_rows - np.maximum(src, dst))
    src, dst = np.clip(src, 0, n_rows - 1), np.clip(dst, 0, n_rows - 1)
    ln = np.minimum(ln, n_rows - np.maximum(src, dst))
    moves = np.stack([src, dst, ln], 1).astype(np.int32)
    check(moves, n_rows)


def test_disjoint_moves_give_a_run_plan():
    rng = np.random.default_rng(3)
    for _ in range(20):
        blocks = rng.permutation(200)[:40]
        moves = np.array([[b * 8, (200 + i) * 8, 8] for i, b in enumerate(blocks)], dtype=np.int32)
        info = check(moves, 300 * 8)
        assert info.kind == 1 and info.n_moves == 40 and info.total_rows == 320


def test_sparse_moves_over_a_wide_range():
    """Moves scattered over 2^30 rows: the planner lays the touched rows out
    compactly instead of covering the whole span."""
    rng = np.random.default_rng(5)
    n_rows = 1 << 30
    base = rng.integers(0, n_rows - 4096, 30)
    moves = []
    for b in base.tolist():
        moves.append([b, b + int(rng.integers(-8, 9)) or b + 3, int(rng.integers(1, 16))])
    moves.append([int(base[0]), int(base[1]), 10])  # across two far-apart places
    moves = np.array(moves, dtype=np.int64)
    moves[:, 1] = np.clip(moves[:, 1], 0, n_rows - 16)
    moves = moves.astype(np.int32)
    info, plan = plan_of(moves, n_rows)
    assert info.kind == 2
    # provenance only of the touched rows (the oracle's index array would be 2^30 long)
    touched = np.unique(np.concatenate([np.arange(s, s + n) for s, d, n in moves.tolist()] +
                                       [np.arange(d, d + n) for s, d, n in moves.tolist()]))
    local = {int(r): i for i, r in enumerate(touched)}
    lmoves = np.array([[local[s], local[d], n] for s, d, n in moves.tolist()], dtype=np.int32)
    # every move's source and destination runs stay contiguous in the local numbering
    for (s, d, n), (ls, ld, _) in zip(moves.tolist(), lmoves.tolist()):
        assert local[s + n - 1] - ls == n - 1 and local[d + n - 1] - ld == n - 1
    want_local = oracle.provenance(len(touched), lmoves)
    rows = {int(r): int(r) for r in touched}
    g = plan[: 2 * info.n_gather].reshape(-1, 2)
    sc = plan[2 * info.n_gather :].reshape(-1, 2)
    stage = [rows[int(x)] for x in g[:, 0]]
    vals = [rows[int(y)] if y >= 0 else stage[-int(y) - 1] for y in sc[:, 1]]
    for r, v in zip(sc[:, 0].tolist(), vals):
        rows[r] = v
    got = np.array([rows[int(r)] for r in touched])
    assert np.array_equal(got, touched[want_local])


def test_plan_refusals_and_empty_plans():
    L = pkv.lib()
    mv = np.array([[0, 5, 3], [10, 98, 4]], dtype=np.int32)
    info = pkv.CopyPlan()
    words = L.pkv_copy_cells_plan_words(mv.ctypes.data, 2)
    buf = np.zeros(words, dtype=np.int64).view(np.int32)
    st = L.pkv_copy_cells_plan(mv.ctypes.data, 2, 100, buf.ctypes.data, words, ctypes.byref(info))
    assert st == 1 and "move 1" in pkv.last_error()
    st = L.pkv_copy_cells_plan(mv.ctypes.data, 2, 200, buf.ctypes.data, words - 1, ctypes.byref(info))
    assert st == 3 and "plan buffer" in pkv.last_error()
    mv0 = np.array([[3, 3, 5], [1, 9, 0]], dtype=np.int32)
    assert L.pkv_copy_cells_plan_words(mv0.ctypes.data, 2) == 0
    st = L.pkv_copy_cells_plan(mv0.ctypes.data, 2, 100, None, 0, ctypes.byref(info))
    assert st == 0 and info.kind == 0 and info.n_words == 0


def test_golden_order_example_plans_to_the_oracle():
    import json
    import os

    with open(os.path.join(os.path.dirname(__file__), "golden", "order_moves_worked.json")) as f:
        g = json.load(f)
    n_rows = int(max(max(s, d) + n for s, d, n in g["moves"])) + 4
    check(np.array(g["moves"], dtype=np.int32), n_rows)
