"""The library's copy-on-write block pool (host C++) against the oracle model.

Both are driven through the same random forks, batched writes and
removals; after every operation the tables, lengths, reference counts,
free counts and returned block copies must be identical, and a refused
operation must be refused by both and change neither.  Host only: no GPU."""

import numpy as np
import pytest

import paged_kv_cache_table_amd as pkv
from oracle.cow import INVALID, BlockPoolModel


def _same(lib_pool, model):
    t, l = lib_pool.export()
    assert np.array_equal(t, model.table)
    assert np.array_equal(l, model.length)
    assert lib_pool.free_blocks() == model.n_free()
    refs = np.array([lib_pool.refcount(b) for b in range(model.n_blocks)])
    assert np.array_equal(refs, model.ref)


@pytest.mark.parametrize("seed", range(10))
def test_random_operations_match_the_model(seed):
    rng = np.random.default_rng(100 + seed)
    bs = [1, 3, 4, 16, 32][seed % 5]
    n_seqs = 10
    max_blocks = 64 // bs + 3
    n_blocks = int(n_seqs * max_blocks * (0.6 if seed % 2 else 1.2)) + 1  # odd seeds run out of blocks
    lp = pkv.BlockPool(n_blocks, n_seqs, max_blocks, bs, watermark=seed % 3)
    mp = BlockPoolModel(n_blocks, n_seqs, max_blocks, bs, watermark=seed % 3)
    refusals = copies = moved = 0
    for step in range(400):
        op = rng.integers(0, 13)
        s = int(rng.integers(0, n_seqs))
        L = int(mp.length[s])
        if op < 5:
            k = int(rng.integers(1, 6))
            seqs = rng.integers(0, n_seqs, size=k)  # a sequence may appear twice in a batch
            p0s, cnts = [], []
            for q in seqs:
                Lq = int(mp.length[q])
                p0s.append(Lq if rng.random() < 0.7 else int(rng.integers(0, Lq + 2)))  # +2: sometimes a gap
                cnts.append(int(rng.integers(-1, 3 * bs + 2)))
            writes = [(int(a), int(b), int(c)) for a, b, c in zip(seqs, p0s, cnts)]
            try:
                want = mp.prepare_writes(writes)
                err = None
            except ValueError as e:
                err = e
            if err is None:
                ops = lp.prepare_writes(seqs, p0s, cnts)
                assert [(a, b) for a, b, _ in ops.tolist() if a >= 0] == want
                # every op names the entry it changed, which now holds its block
                t, _ = lp.export()
                assert all(t.reshape(-1)[e] == b for _, b, e in ops.tolist())
                copies += len(want)
            else:
                refusals += 1
                with pytest.raises(pkv.PkvError):
                    lp.prepare_writes(seqs, p0s, cnts)
        elif op < 7:
            dst = int(rng.integers(0, n_seqs))
            n = int(rng.integers(-1, L + 2))
            try:
                mp.fork(s, dst, None if n < 0 else n)
                ok = True
            except ValueError:
                ok = False
            if ok:
                lp.fork(s, dst, n)
            else:
                with pytest.raises(pkv.PkvError):
                    lp.fork(s, dst, n)
        elif op < 9:
            p0 = int(rng.integers(-2, L + 2))
            p1 = int(rng.integers(p0, L + 3)) if rng.random() < 0.6 else L
            mp.remove(s, p0, p1)
            lp.remove(s, p0, p1)
        elif op < 11:  # drop a whole sequence, which makes room for forks
            mp.remove(s, 0, L)
            lp.remove(s, 0, L)
        else:  # compaction
            need = int(rng.integers(-1, mp.n_free() + 2))
            try:
                want = mp.defrag(need)
                err = None
            except ValueError as e:
                err = e
            if err is None:
                got = lp.defrag(need)
                assert [tuple(m) for m in got.tolist()] == want
                moved += sum(m[2] for m in want)
            else:
                with pytest.raises(pkv.PkvError):
                    lp.defrag(need)
        n = int(rng.integers(0, n_blocks + 1))
        assert lp.can_allocate(n) == mp.can_allocate(n)
        _same(lp, mp)
        mp.check()
    assert copies + moved > 0
    if seed % 2:
        assert refusals > 0


def test_capacity_and_copy_buffer_refusals():
    lp = pkv.BlockPool(3, 3, 4, 4)
    lp.prepare_writes([0], [0], [8])
    lp.fork(0, 1)
    before = lp.export()
    with pytest.raises(pkv.PkvError) as ei:
        lp.prepare_writes([1, 0, 1], [8, 8, 0], [1, 1, 1])  # needs 3 fresh blocks, 1 free
    assert ei.value.status == 5
    after = lp.export()
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
    # copies_out too small: call the C entry directly with room for none
    import ctypes

    seqs = np.array([1], dtype=np.int32)
    p0s = np.array([0], dtype=np.int32)
    cnts = np.array([1], dtype=np.int32)
    nc = ctypes.c_int32(-1)
    st = pkv.lib().pkv_pool_prepare_writes(lp._h, 1, seqs.ctypes.data, p0s.ctypes.data, cnts.ctypes.data,
                                           None, 0, ctypes.byref(nc))  # one op needed, room for none
    assert st == 3 and nc.value == 0
    assert np.array_equal(lp.export()[0], before[0])


def test_pool_argument_refusals():
    with pytest.raises(pkv.PkvError):
        pkv.BlockPool(0, 1, 1, 16)
    lp = pkv.BlockPool(8, 2, 4, 4)
    for call in (lambda: lp.fork(0, 0), lambda: lp.fork(0, 5), lambda: lp.remove(7, 0, 1),
                 lambda: lp.prepare_writes([3], [0], [1]), lambda: lp.prepare_writes([0], [1], [1]),
                 lambda: lp.prepare_writes([0], [0], [17])):
        with pytest.raises(pkv.PkvError):
            call()
    assert lp.refcount(-1) == -1 and lp.refcount(8) == -1 and lp.seq_len(2) == -1
    assert lp.free_blocks() == 8 and np.all(lp.export()[0] == INVALID)


def test_large_batch_is_fast():
    """A fork storm on a big pool: 1024 sequences writing one token each
    into a shared partial block costs 1024 host steps, not a quadratic scan."""
    import time

    lp = pkv.BlockPool(1 << 17, 1024, 512, 16)
    for g in range(256):
        lp.prepare_writes([4 * g], [0], [1000 + 17 * g])
        for k in range(1, 4):
            lp.fork(4 * g, 4 * g + k)
    seqs = np.arange(1024, dtype=np.int32)
    _, lens = lp.export()
    t0 = time.perf_counter()
    ops = lp.prepare_writes(seqs, lens[seqs], np.ones(1024, dtype=np.int32))
    dt = time.perf_counter() - t0
    copies = ops[ops[:, 0] >= 0]
    partial = sum(1 for g in range(256) if (1000 + 17 * g) % 16)
    # in each group whose shared last block is partial, the first three
    # writers copy it and the fourth finds it unshared and writes in place
    assert len(copies) == 3 * partial
    assert dt < 0.05


@pytest.mark.parametrize("bs", [1, 16])
def test_defrag_of_a_fragmented_pool_matches_the_model(bs):
    """Twelve sequences (some forked), every other one dropped: defrag to a
    partial target, then fully; moves, tables and counts as the model says."""
    rng = np.random.default_rng(bs)
    n_seqs, max_blocks = 12, 200 // bs + 2
    n_blocks = n_seqs * max_blocks
    lp = pkv.BlockPool(n_blocks, n_seqs, max_blocks, bs)
    mp = BlockPoolModel(n_blocks, n_seqs, max_blocks, bs)
    for s in range(0, n_seqs, 3):
        n = int(rng.integers(20, 200))
        lp.prepare_writes([s], [0], [n])
        mp.prepare_writes([(s, 0, n)])
        for d in (s + 1, s + 2):
            lp.fork(s, d, n // 2)
            mp.fork(s, d, n // 2)
            lp.prepare_writes([d], [n // 2], [30])
            mp.prepare_writes([(d, n // 2, 30)])
    for s in range(0, n_seqs, 2):
        lp.remove(s, 0, 1 << 30)
        mp.remove(s, 0, 1 << 30)
    _same(lp, mp)
    total = 0
    for need in (mp.n_free() // 3, -1, -1):
        want = mp.defrag(need)
        got = lp.defrag(need)
        assert [tuple(m) for m in got.tolist()] == want
        _same(lp, mp)
        mp.check()
        total += len(want)
    assert total > 0
    live = n_blocks - mp.n_free()
    assert np.all(mp.ref[live:] == 0) and np.all(mp.ref[:live] > 0)
