"""Copy-on-write on the GPU: block copies + table patches (cow_apply) and the
whole fork-and-write flow (pool plan on the host, cow_apply, store) against
the oracle's block-pool model, copies and store, bit for bit.  Readers of a
shared prefix must see bitwise the same attention before and after other
sequences write."""

import numpy as np
import pytest

import oracle
import paged_kv_cache_table_amd as pkv

from gpu_util import log

pytestmark = pytest.mark.gpu


def _bytes_equal(a, b):
    return np.array_equal(np.ascontiguousarray(a).view(np.uint8), np.ascontiguousarray(b).view(np.uint8))


@pytest.mark.parametrize("hkv,bs,kw,vw", [(4, 16, 136, 256), (8, 16, 136, 256), (1, 5, 68, 128), (3, 7, 36, 64)])
def test_cow_apply_copies_and_patches_bit_exact(hkv, bs, kw, vw):
    """Blocks of 8.5 KiB / 16 KiB (two 8 KiB chunks, one partial), 17 / 32 KiB,
    and blocks whose size is not a multiple of 16 bytes (word copies)."""
    import torch

    rng = np.random.default_rng(hkv * 100 + bs)
    nb = 96
    kh = rng.integers(0, 256, size=(nb, hkv, bs, kw), dtype=np.uint8)
    vh = rng.integers(0, 256, size=(nb, hkv, bs, vw), dtype=np.uint8).view(np.float16)
    table_h = rng.integers(-1, nb, size=(7, 20), dtype=np.int32)
    perm = rng.permutation(nb)
    srcs, dsts = perm[:30], perm[30:60]
    entries = rng.permutation(140)  # distinct entries, as prepare_writes emits them
    ops = [(int(s), int(d), int(e)) for s, d, e in zip(srcs, dsts, entries[:30])]
    ops += [(-1, int(perm[60]), int(entries[30])), (int(perm[61]), int(perm[61]), int(entries[31])),  # fresh; src == dst
            (nb + 5, int(perm[62]), int(entries[32])), (int(perm[63]), nb, int(entries[33])),  # outside the pool
            (int(perm[64]), int(perm[65]), 140), (int(perm[66]), int(perm[67]), -4)]  # entry outside the table
    k, v, table = torch.from_numpy(kh).cuda(), torch.from_numpy(vh).cuda(), torch.from_numpy(table_h).cuda()
    pkv.cow_apply(k, v, np.array(ops, dtype=np.int32), table)
    torch.cuda.synchronize()
    copies = [(s, d) for s, d, _ in ops if 0 <= s < nb and 0 <= d < nb and s != d]
    rk, rv = kh.copy(), vh.copy()
    oracle.copy_blocks([rk, rv], copies)
    want_t = table_h.reshape(-1).copy()
    for _, d, e in ops:
        if 0 <= e < want_t.size:
            want_t[e] = d
    assert _bytes_equal(k.cpu().numpy(), rk) and _bytes_equal(v.cpu().numpy(), rv)
    assert np.array_equal(table.cpu().numpy().reshape(-1), want_t)


class Both:
    """The library path (BlockPool + device pools/table) and the oracle path
    (BlockPoolModel + host pools) driven by the same operations."""

    def __init__(self, rng, n_blocks, n_seqs, max_blocks, bs, hkv, hd, kfmt="q8_0", vfmt="f16"):
        import torch

        self.bs, self.hkv, self.hd, self.kfmt, self.vfmt = bs, hkv, hd, kfmt, vfmt
        self.lp = pkv.BlockPool(n_blocks, n_seqs, max_blocks, bs)
        self.mp = oracle.BlockPoolModel(n_blocks, n_seqs, max_blocks, bs)
        wk, wv = oracle.seg_bytes(kfmt, hd), oracle.seg_bytes(vfmt, hd)
        dt = {"f32": np.float32, "f16": np.float16, "q8_0": np.uint8}
        self.kh = rng.integers(0, 256, size=(n_blocks, hkv, bs, wk), dtype=np.uint8).view(dt[kfmt])
        self.vh = rng.integers(0, 256, size=(n_blocks, hkv, bs, wv), dtype=np.uint8).view(dt[vfmt])
        self.k, self.v = torch.from_numpy(self.kh.copy()).cuda(), torch.from_numpy(self.vh.copy()).cuda()
        self.table = torch.full((n_seqs, max_blocks), -1, dtype=torch.int32, device="cuda")
        self.rng = rng
        self.n_ops = self.n_copies = 0

    def sync_table(self):
        import torch

        t, _ = self.lp.export()
        self.table.copy_(torch.from_numpy(t))

    def fork(self, src, dst, n=None):
        self.lp.fork(src, dst, -1 if n is None else n)
        self.mp.fork(src, dst, n)
        self.sync_table()

    def write(self, seqs, counts):
        """Append counts[i] new tokens to seqs[i] (one batch)."""
        import torch

        p0s = [int(self.mp.length[s]) for s in seqs]
        ops = self.lp.prepare_writes(seqs, p0s, counts)
        copies = self.mp.prepare_writes(list(zip(seqs, p0s, counts)))
        assert [(a, b) for a, b, _ in ops.tolist() if a >= 0] == copies
        self.n_ops += len(ops)
        self.n_copies += len(copies)
        sid = np.concatenate([np.full(c, s, dtype=np.int32) for s, c in zip(seqs, counts)])
        pos = np.concatenate([np.arange(p, p + c, dtype=np.int32) for p, c in zip(p0s, counts)])
        kx = self.rng.standard_normal((len(pos), self.hkv, self.hd)).astype(np.float32)
        vx = self.rng.standard_normal((len(pos), self.hkv, self.hd)).astype(np.float32)
        # device: copies + table patches, then the store through the patched table
        pkv.cow_apply(self.k, self.v, ops, self.table)
        pkv.kv_store(torch.from_numpy(kx).cuda(), torch.from_numpy(vx).cuda(), torch.from_numpy(pos).cuda(),
                     self.k, self.v, self.table, seq_ids=torch.from_numpy(sid).cuda())
        # oracle: copies, then the store through the model's table
        oracle.copy_blocks([self.kh, self.vh], copies)
        self.kh, self.vh, skipped = oracle.store_rows(self.kh, self.vh, self.kfmt, self.vfmt, kx, vx, sid, pos,
                                                      self.mp.table)
        assert skipped == 0

    def check(self):
        import torch

        torch.cuda.synchronize()
        t, l = self.lp.export()
        assert np.array_equal(t, self.mp.table) and np.array_equal(l, self.mp.length)
        assert np.array_equal(self.table.cpu().numpy(), self.mp.table)
        assert _bytes_equal(self.k.cpu().numpy(), self.kh), "K pool differs"
        assert _bytes_equal(self.v.cpu().numpy(), self.vh), "V pool differs"

    def decode(self, q, seqs):
        import torch

        lens = torch.from_numpy(self.mp.length.astype(np.int32)).cuda()
        out, lse = pkv.paged_attn_decode(q, self.k, self.v, self.table, lens, 1.0 / np.sqrt(self.hd))
        return out[seqs].cpu().numpy(), lse[seqs].cpu().numpy()


@pytest.mark.parametrize("bs", [16, 32])
def test_fork_storm_bit_exact_and_readers_unchanged(bs):
    import torch

    rng = np.random.default_rng(bs)
    hkv, hd, hq = 8, 128, 32
    n_par, max_blocks = 4, 400 // bs + 2
    n_seqs = n_par * 4
    b = Both(rng, 420, n_seqs, max_blocks, bs, hkv, hd)
    lens = [37, 64, 100, 5]
    for p, L in enumerate(lens):  # parents, written in chunks of up to 50 tokens
        done = 0
        while done < L:
            c = min(50, L - done)
            b.write([p], [c])
            done += c
    # per parent: two writers forked at full length and mid-block, one reader
    writers, readers = list(range(n_par)), []
    for p, L in enumerate(lens):
        w1, w2, r = n_par + 3 * p, n_par + 3 * p + 1, n_par + 3 * p + 2
        b.fork(p, w1)
        b.fork(p, w2, max(1, L - 3))
        b.fork(p, r)
        writers += [w1, w2]
        readers.append(r)
    b.check()
    q = torch.randn((n_seqs, hq, hd), generator=torch.Generator().manual_seed(1)).half().cuda()
    before = b.decode(q, readers)
    for rnd in range(3):
        order = rng.permutation(writers).tolist()
        counts = [int(rng.integers(1, 21)) for _ in order]
        b.write(order, counts)
        b.check()
    after = b.decode(q, readers)
    log(f"  bs {bs}: {b.n_ops} table changes, {b.n_copies} block copies")
    assert b.n_copies >= 8
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
    # every sequence's attention matches the oracle over the oracle's pools
    out, lse = b.decode(q, list(range(n_seqs)))
    ro, rl = oracle.paged_decode(q.cpu().numpy(), b.kh, b.vh, "q8_0", "f16", b.mp.table,
                                 b.mp.length, bs, hkv, hd, 1.0 / np.sqrt(hd))
    assert np.abs(out - ro).max() <= 2e-3 and np.abs(lse - rl).max() <= 2e-3


def test_remove_then_rewrite_through_the_pool():
    """Removal (tail and middle), then appends: table, pools and attention
    stay in step with the oracle."""
    rng = np.random.default_rng(5)
    b = Both(rng, 64, 4, 12, 16, 2, 64, kfmt="f16", vfmt="f16")
    b.write([0, 1], [150, 90])
    b.fork(0, 2, 120)
    b.lp.remove(0, 32, 64)  # a middle block becomes a hole
    b.mp.remove(0, 32, 64)
    b.lp.remove(1, 40, 90)  # tail
    b.mp.remove(1, 40, 90)
    b.sync_table()
    b.write([1, 2, 0], [30, 9, 4])
    b.check()


@pytest.mark.parametrize("bs,need_kind", [(16, "full"), (16, "part"), (32, "full")])
def test_defrag_moves_rows_and_attention_is_bitwise_unchanged(bs, need_kind):
    """Fragment the pool (writes, forks, dropped sequences), then compact:
    the library's moves equal the oracle's, the pools after kv_copy_cells
    equal the oracle's sequential copy_cells bit for bit, and decode over
    every sequence gives bitwise the same result as before the compaction."""
    import torch

    rng = np.random.default_rng(70 + bs)
    hkv, hd, hq = 8, 128, 32
    n_seqs, max_blocks = 12, 600 // bs + 2
    b = Both(rng, n_seqs * max_blocks, n_seqs, max_blocks, bs, hkv, hd)
    for s in range(0, n_seqs, 3):
        b.write([s], [int(rng.integers(50, 400))])
        for d in (s + 1, s + 2):
            b.fork(s, d, int(b.mp.length[s]) // 2)
            b.write([d], [int(rng.integers(1, 120))])
    for s in (0, 4, 5, 9):
        b.lp.remove(s, 0, 1 << 30)
        b.mp.remove(s, 0, 1 << 30)
    b.lp.remove(7, 40, 90)  # a middle removal: holes in a live sequence
    b.mp.remove(7, 40, 90)
    b.sync_table()
    b.check()
    q = torch.randn((n_seqs, hq, hd), generator=torch.Generator().manual_seed(2)).half().cuda()
    before = b.decode(q, list(range(n_seqs)))
    # "part": all but a few free blocks, so the top range still holds live blocks
    need = -1 if need_kind == "full" else b.mp.n_free() - 5
    moves = b.lp.defrag(need)
    want = b.mp.defrag(need)
    assert [tuple(m) for m in moves.tolist()] == want and len(want) > 0
    pkv.kv_copy_cells(b.k, b.v, moves)
    oracle.copy_cells([b.kh, b.vh], want)
    b.sync_table()
    b.check()
    after = b.decode(q, list(range(n_seqs)))
    log(f"  defrag bs {bs} {need_kind}: {len(want)} moves, {sum(m[2] for m in want)} rows")
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
