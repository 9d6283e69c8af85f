"""Pins of the oracle's copy-on-write block pool.

* a naive model in which every sequence owns a plain list of its tokens
  (no sharing, no blocks): after any sequence of forks, writes and
  removals, every position a sequence can read through its table holds the
  token the naive model says — so a reader of a shared prefix never sees
  another sequence's write;
* reference-count invariants after every operation;
* worked scenarios: the number of block copies a fork storm costs, the
  parent keeping its block, refusal leaving the state unchanged, the
  watermark;
* compaction: after defrag and its row moves (applied by the oracle's
  sequential copy_cells), every sequence reads the same tokens, the top
  `need` blocks are free, every move goes down onto rows no move reads
  (so the sequential result equals a simultaneous gather), and only the
  live blocks of the top range move.
"""

import numpy as np
import pytest

from oracle.cow import INVALID, BlockPoolModel, copy_blocks

UNSPEC = object()  # a position whose contents the pages leave unspecified


class Paged:
    """The model plus a pool of token ids [n_blocks, bs]."""

    def __init__(self, n_blocks, n_seqs, max_blocks, bs):
        self.m = BlockPoolModel(n_blocks, n_seqs, max_blocks, bs)
        self.data = np.full((n_blocks, bs), -7, dtype=np.int64)

    def write(self, writes, tokens):
        copies = self.m.prepare_writes([(s, p0, len(t)) for s, p0, t in zip(*writes, tokens)])
        copy_blocks([self.data], copies)
        for s, p0, toks in zip(writes[0], writes[1], tokens):
            for i, tok in enumerate(toks):
                p = p0 + i
                self.data[self.m.table[s, p // self.m.bs], p % self.m.bs] = tok
        return copies

    def read(self, s):
        m = self.m
        out = []
        for p in range(int(m.length[s])):
            b = m.table[s, p // m.bs]
            out.append(None if b == INVALID else int(self.data[b, p % m.bs]))
        return out


class Naive:
    """Every sequence is a list; None = removed, UNSPEC = unspecified."""

    def __init__(self, n_seqs, bs):
        self.seq = [[] for _ in range(n_seqs)]
        self.bs = bs

    def fork(self, src, dst, n):
        self.seq[dst] = list(self.seq[src][:n])
        # rows of a shared partial block past n are not the fork's
        return

    def remove(self, s, p0, p1):
        L = len(self.seq[s])
        p0, p1 = max(0, p0), min(L, p1)
        if p0 >= p1:
            return
        if p1 == L:
            del self.seq[s][p0:]
            return
        first = -(-p0 // self.bs)
        for lb in range(first, p1 // self.bs):
            for p in range(lb * self.bs, (lb + 1) * self.bs):
                self.seq[s][p] = None

    def write(self, s, p0, toks):
        q = self.seq[s]
        # blocks the write touches that are wiped (removal wipes whole blocks,
        # so one removed position below the length marks the whole block)
        touched = range(p0 // self.bs, (p0 + len(toks) - 1) // self.bs + 1)
        was_hole = {lb for lb in touched
                    if any(q[p] is None for p in range(lb * self.bs, min(len(q), (lb + 1) * self.bs)))}
        while len(q) < p0 + len(toks):
            q.append(None)
        for i, t in enumerate(toks):
            q[p0 + i] = t
        # a revived hole block: its other positions hold whatever the pool held
        for lb in was_hole:
            for p in range(lb * self.bs, min(len(q), (lb + 1) * self.bs)):
                if not p0 <= p < p0 + len(toks):
                    q[p] = UNSPEC

    def read(self, s):
        return self.seq[s]


def _agree(pg, nv, n_seqs):
    pg.m.check()
    for s in range(n_seqs):
        got, want = pg.read(s), nv.read(s)
        assert len(got) == len(want), (s, len(got), len(want))
        for p, (g, w) in enumerate(zip(got, want)):
            if w is UNSPEC:
                continue
            assert g == w, (s, p, g, w)


@pytest.mark.parametrize("seed", range(12))
def test_random_operations_match_the_naive_model(seed):
    rng = np.random.default_rng(seed)
    bs = [1, 2, 4, 16][seed % 4]
    n_seqs, max_blocks = 8, 40 // bs + 4
    pg = Paged(n_seqs * max_blocks, n_seqs, max_blocks, bs)
    nv = Naive(n_seqs, bs)
    tok = iter(range(10 ** 9))
    for step in range(300):
        op = rng.integers(0, 10)
        s = int(rng.integers(0, n_seqs))
        L = int(pg.m.length[s])
        if op < 5:  # a batch of appends (or rewrites) over several sequences
            seqs = rng.choice(n_seqs, size=int(rng.integers(1, 4)), replace=False)
            ws, p0s, toks = [], [], []
            for q in seqs:
                Lq = int(pg.m.length[q])
                n = int(rng.integers(1, 6))
                p0 = Lq if rng.random() < 0.8 else int(rng.integers(0, Lq + 1))
                if p0 + n > max_blocks * bs:
                    continue
                ws.append(int(q)); p0s.append(p0); toks.append([next(tok) for _ in range(n)])
            if not ws:
                continue
            pg.write((ws, p0s), toks)
            for q, p0, t in zip(ws, p0s, toks):
                nv.write(q, p0, t)
        elif op < 7:  # fork into an empty sequence
            empty = [d for d in range(n_seqs)
                     if d != s and pg.m.length[d] == 0 and np.all(pg.m.table[d] == INVALID)]
            if not empty:
                continue
            dst = int(rng.choice(empty))
            n = int(rng.integers(0, L + 1))
            pg.m.fork(s, dst, n)
            nv.fork(s, dst, n)
        else:  # remove a range (tail or middle)
            if L == 0:
                continue
            p0 = int(rng.integers(0, L))
            p1 = L if rng.random() < 0.4 else int(rng.integers(p0, L + 1))
            pg.m.remove(s, p0, p1)
            nv.remove(s, p0, p1)
        _agree(pg, nv, n_seqs)


def test_fork_storm_copies_once_per_writing_fork():
    """A parent of 40 tokens (block 16: the third block holds 8) forked 3
    times: each fork's first append copies the shared third block, the
    parent's own append (the block then unshared) writes in place, and
    the first two blocks are never copied."""
    pg = Paged(32, 4, 8, 16)
    pg.write(([0], [0]), [list(range(100, 140))])
    for d in (1, 2, 3):
        pg.m.fork(0, d)
    shared = int(pg.m.table[0, 2])
    assert pg.m.ref[shared] == 4 and pg.m.ref[pg.m.table[0, 0]] == 4
    copies = pg.write(([1, 2, 3, 0], [40, 40, 40, 40]), [[1], [2], [3], [0]])
    assert [c[0] for c in copies] == [shared] * 3
    assert len({c[1] for c in copies}) == 3
    assert pg.m.table[0, 2] == shared and pg.m.ref[shared] == 1
    for d in (1, 2, 3):
        assert pg.read(d) == list(range(100, 140)) + [d]
    assert pg.read(0) == list(range(100, 140)) + [0]
    assert pg.m.ref[pg.m.table[0, 0]] == 4  # untouched prefix blocks stay shared


def test_smallest_free_block_first_and_release():
    m = BlockPoolModel(8, 2, 4, 4)
    m.prepare_writes([(0, 0, 9)])  # three blocks
    assert m.table[0, :3].tolist() == [0, 1, 2]
    m.remove(0, 4, 8)  # the middle block becomes a hole
    assert m.table[0].tolist() == [0, INVALID, 2, INVALID] and m.ref[1] == 0
    m.prepare_writes([(1, 0, 1)])
    assert m.table[1, 0] == 1  # the freed id is the smallest
    m.remove(0, 0, 100)
    assert m.length[0] == 0 and np.all(m.table[0] == INVALID)
    assert m.n_free() == 7
    m.check()


def test_refused_prepare_changes_nothing():
    m = BlockPoolModel(3, 3, 4, 4)
    m.prepare_writes([(0, 0, 8)])
    m.fork(0, 1)
    before = (m.ref.copy(), m.table.copy(), m.length.copy(), m.n_free())
    with pytest.raises(ValueError):
        m.prepare_writes([(1, 8, 1), (0, 8, 1), (1, 0, 1)])  # needs 3 fresh blocks, 1 free
    with pytest.raises(ValueError):
        m.prepare_writes([(2, 1, 1)])  # gap
    with pytest.raises(ValueError):
        m.prepare_writes([(2, 0, 17)])  # past the table
    after = (m.ref, m.table, m.length, m.n_free())
    for a, b in zip(before[:3], after[:3]):
        assert np.array_equal(a, b)
    assert before[3] == after[3]


def test_watermark_governs_admission_only():
    m = BlockPoolModel(10, 2, 8, 4, watermark=3)
    assert m.can_allocate(7) and not m.can_allocate(8)
    m.prepare_writes([(0, 0, 32)])  # eight blocks: below the watermark is still allowed for writes
    assert m.n_free() == 2 and not m.can_allocate(0)


def test_fork_refusals():
    m = BlockPoolModel(8, 3, 4, 4)
    m.prepare_writes([(0, 0, 5)])
    with pytest.raises(ValueError):
        m.fork(0, 0)
    with pytest.raises(ValueError):
        m.fork(0, 1, 6)
    m.fork(0, 1, 5)
    with pytest.raises(ValueError):
        m.fork(0, 1)  # destination not empty


def _apply_moves_to_blocks(pg, moves):
    """Row moves on the token-id pool [n_blocks, bs], through the oracle's
    sequential copy_cells (a pool of rows is [n_rows, 1])."""
    rows = pg.data.reshape(-1, 1)
    before = rows.copy()
    oracle_copy_cells([rows], moves)
    # simultaneous gather: every destination row takes its source's old value
    gathered = before.copy()
    for s_, d_, n_ in moves:
        gathered[d_ : d_ + n_] = before[s_ : s_ + n_]
    assert np.array_equal(rows, gathered)


from oracle.moves import copy_cells as oracle_copy_cells  # noqa: E402


@pytest.mark.parametrize("seed", range(8))
def test_defrag_keeps_every_sequence_and_frees_the_top(seed):
    rng = np.random.default_rng(50 + seed)
    bs = [1, 4, 16, 2][seed % 4]
    n_seqs, max_blocks = 12, 60 // bs + 2
    n_blocks = n_seqs * max_blocks
    pg = Paged(n_blocks, n_seqs, max_blocks, bs)
    nv = Naive(n_seqs, bs)
    tok = iter(range(10 ** 9))
    for _ in range(120):  # fragment the pool: writes, forks, removals
        s = int(rng.integers(0, n_seqs))
        op = rng.integers(0, 6)
        L = int(pg.m.length[s])
        if op < 3:
            n = int(rng.integers(1, 12))
            if L + n <= max_blocks * bs:
                toks = [next(tok) for _ in range(n)]
                pg.write(([s], [L]), [toks])
                nv.write(s, L, toks)
        elif op < 4:
            empty = [d for d in range(n_seqs) if d != s and pg.m.length[d] == 0]
            if empty:
                d = int(rng.choice(empty))
                n = int(rng.integers(0, L + 1))
                pg.m.fork(s, d, n)
                nv.fork(s, d, n)
        else:
            p0 = int(rng.integers(0, L + 1))
            p1 = L if op == 5 else int(rng.integers(p0, L + 1))
            pg.m.remove(s, p0, p1)
            nv.remove(s, p0, p1)
    n_free = pg.m.n_free()
    need = [-1, n_free, n_free // 2, 0][seed % 4]
    live_top = int(np.count_nonzero(pg.m.ref[n_blocks - (n_free if need < 0 else need):] > 0))
    moves = pg.m.defrag(need)
    # only the live blocks of the top range moved, each down onto a free row
    assert sum(m[2] for m in moves) == live_top * bs
    srcs = set()
    for s_, d_, n_ in moves:
        assert d_ < s_ and n_ > 0 and n_ % bs == 0
        srcs.update(range(s_, s_ + n_))
    for s_, d_, n_ in moves:
        assert not srcs.intersection(range(d_, d_ + n_))
    _apply_moves_to_blocks(pg, moves)
    top = n_blocks - (n_free if need < 0 else need)
    assert np.all(pg.m.ref[top:] == 0)
    _agree(pg, nv, n_seqs)


def test_defrag_worked_example():
    """Blocks 0..7, block size 2: live blocks 1, 4, 6 and 7 (7 shared by two
    sequences); defrag(4) frees 4..7: 4 -> 0, 6 -> 2, 7 -> 3 (6 and 7 land on
    consecutive blocks: one move of 4 rows)."""
    m = BlockPoolModel(8, 3, 4, 2)
    m.table[0, :2] = [1, 7]
    m.table[1, :3] = [4, 6, 7]
    m.length[:2] = [4, 6]
    m.ref[[1, 4, 6, 7]] = [1, 1, 1, 2]
    m._free = [0, 2, 3, 5]
    moves = m.defrag(4)
    assert moves == [(8, 0, 2), (12, 4, 4)]
    assert m.table[0, :2].tolist() == [1, 3] and m.table[1, :3].tolist() == [0, 2, 3]
    assert m.ref.tolist() == [1, 1, 1, 2, 0, 0, 0, 0]
    m.check()
    with pytest.raises(ValueError):
        m.defrag(5)
    assert m.defrag(4) == []
