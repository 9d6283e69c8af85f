"""Copy-on-write block pool: refcounted physical blocks shared by forks.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources:
* "Tiered KV cache — architecture", section "The paged-attention block
  model": tokens live in fixed-size physical blocks named by a per-sequence
  table; forking a sequence only raises per-block reference counts and
  copies the table, so forks cost no K/V copies until one of them writes;
  a partial removal wipes whole logical blocks in the middle of a sequence
  by setting their entries to the invalid-block sentinel.  Section "Files"
  lists the physical allocator with reference counting and a watermark.
* "KV Cache Design — cells, format, sessions", sections 1 and 2: a store
  may never land in a prefix that another sequence reads in place; before
  the first row of a write is resolved, the shared part is copied so that
  the writer gets private rows (the share shrinks to the first written
  position), and readers of the shared prefix see no change.

Readings where the pages are silent:
* allocation takes the free block with the smallest id (deterministic);
  a block is free exactly when its reference count is 0;
* fork(src, dst, n): dst must be empty; it gets src's first ceil(n / bs)
  table entries (holes stay holes) and length n, and every block it now
  names gains one reference;
* remove(s, p0, p1) on [p0, p1) clipped to [0, len): when it reaches the
  end of the sequence, the length becomes p0 and every logical block that
  starts at or after p0 is released; otherwise every logical block lying
  wholly inside [p0, p1) is released and becomes a hole, and blocks only
  partly inside keep their rows (removal is block-granular);
* prepare_write(s, p0, n) before writing positions [p0, p0 + n) (p0 <= len,
  no gap): each logical block those positions touch is, in order, (a) kept
  if the sequence alone references it, (b) copied into a fresh block if it
  is shared (the copy keeps every row of the block; the shared block loses
  one reference), or (c) a fresh block if the entry is empty (a hole or
  never allocated; its rows other than the written ones hold whatever the
  pool held).  The length becomes max(len, p0 + n).  A batch of writes is
  prepared in order; all block copies of a batch are applied before any row
  is stored, so a copy reads the block as it was before the batch;
* a prepare that needs more fresh blocks than are free is refused and
  changes nothing; the watermark only affects can_allocate (admission):
  free - n >= watermark.

Compaction ("KV Cache Design", section 2: a compaction changes only cells,
so rows move verbatim through copy_cells in order_moves order; the
defragmenter returns the moves and whoever caches block ids applies them):
* defrag(need) makes the top `need` blocks of the pool free (need < 0: all
  free blocks, i.e. every live block ends below the number of live
  blocks).  The live blocks found in that top range, in ascending id order,
  move into the lowest free blocks below it, in ascending order; every
  table entry follows its block and reference counts move along.  In a
  block-table pool a sequence's blocks need not be contiguous, so holes are
  filled rather than everything slid down: the fewest blocks move, and no
  destination is ever a source (every move goes down, onto a free row).
  Moves are pool rows (src_row, dst_row, len), consecutive blocks that land
  on consecutive blocks merged into one move; need larger than the free
  blocks is refused and changes nothing.
"""

from __future__ import annotations

import heapq

import numpy as np

INVALID = -1
PRIVATE = -2  # scratch marker: a block this batch already made private


class BlockPoolModel:
    def __init__(self, n_blocks: int, n_seqs: int, max_blocks: int, block_size: int, watermark: int = 0):
        self.n_blocks, self.n_seqs, self.max_blocks, self.bs = n_blocks, n_seqs, max_blocks, block_size
        self.watermark = watermark
        self.ref = np.zeros(n_blocks, dtype=np.int64)
        self.table = np.full((n_seqs, max_blocks), INVALID, dtype=np.int32)
        self.length = np.zeros(n_seqs, dtype=np.int64)
        self._free = list(range(n_blocks))
        heapq.heapify(self._free)

    # -- blocks ---------------------------------------------------------------
    def n_free(self) -> int:
        return len(self._free)

    def can_allocate(self, n: int) -> bool:
        return self.n_free() - n >= self.watermark

    def _alloc(self) -> int:
        b = heapq.heappop(self._free)
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _release(self, b: int):
        self.ref[b] -= 1
        assert self.ref[b] >= 0
        if self.ref[b] == 0:
            heapq.heappush(self._free, b)

    def _nblk(self, n_tokens: int) -> int:
        return -(-int(n_tokens) // self.bs)

    # -- sequences ------------------------------------------------------------
    def fork(self, src: int, dst: int, n_tokens=None):
        n = int(self.length[src]) if n_tokens is None else int(n_tokens)
        if src == dst or self.length[dst] != 0 or np.any(self.table[dst] != INVALID):
            raise ValueError("fork needs a distinct, empty destination")
        if not 0 <= n <= self.length[src]:
            raise ValueError("fork length outside the source")
        nb = self._nblk(n)
        self.table[dst, :nb] = self.table[src, :nb]
        for b in self.table[dst, :nb]:
            if b != INVALID:
                self.ref[b] += 1
        self.length[dst] = n

    def remove(self, s: int, p0: int, p1: int):
        L = int(self.length[s])
        p0, p1 = max(0, int(p0)), min(L, int(p1))
        if p0 >= p1:
            return
        first = self._nblk(p0)  # first logical block starting at or after p0
        if p1 == L:  # the tail goes: every block from `first` on
            last = self.max_blocks
            self.length[s] = p0
        else:  # a middle range: blocks lying wholly inside become holes
            last = p1 // self.bs
        for lb in range(first, last):
            b = int(self.table[s, lb])
            if b != INVALID:
                self._release(b)
                self.table[s, lb] = INVALID

    def prepare_writes(self, writes):
        """writes: [(seq, p0, n)].  Returns the block copies [(src, dst)] to
        apply before the rows are stored.  Refused (ValueError, no change)
        if a write leaves a gap, overruns the table or the pool runs out."""
        # validate on a scratch copy first (verify before apply)
        need = 0
        ref = self.ref.copy()
        table = self.table.copy()
        length = self.length.copy()
        for s, p0, n in writes:
            if n <= 0:
                continue
            if p0 > length[s] or p0 < 0:
                raise ValueError("write leaves a gap")
            if p0 + n > self.max_blocks * self.bs:
                raise ValueError("write overruns the table")
            for lb in range(p0 // self.bs, (p0 + n - 1) // self.bs + 1):
                b = int(table[s, lb])
                if b == PRIVATE:
                    continue
                if b == INVALID or ref[b] > 1:
                    need += 1
                    if b != INVALID:
                        ref[b] -= 1
                    table[s, lb] = PRIVATE
            length[s] = max(length[s], p0 + n)
        if need > self.n_free():
            raise ValueError("pool out of free blocks")
        copies = []
        for s, p0, n in writes:
            if n <= 0:
                continue
            for lb in range(p0 // self.bs, (p0 + n - 1) // self.bs + 1):
                b = int(self.table[s, lb])
                if b == INVALID:
                    self.table[s, lb] = self._alloc()
                elif self.ref[b] > 1:
                    nb = self._alloc()
                    copies.append((b, nb))
                    self.ref[b] -= 1
                    self.table[s, lb] = nb
            self.length[s] = max(self.length[s], p0 + n)
        return copies

    def defrag(self, need: int):
        """Returns the row moves [(src_row, dst_row, len)] and applies the
        block relocation to the tables, counts and free set."""
        nf = self.n_free()
        if need < 0:
            need = nf
        if need > nf:
            raise ValueError("fewer free blocks than needed")
        top = self.n_blocks - need
        srcs = [b for b in range(top, self.n_blocks) if self.ref[b] > 0]
        holes = [b for b in range(top) if self.ref[b] == 0][: len(srcs)]
        assert len(holes) == len(srcs)
        where = {}
        for s, d in zip(srcs, holes):
            where[s] = d
        for q in range(self.n_seqs):
            for lb in range(self.max_blocks):
                b = int(self.table[q, lb])
                if b in where:
                    self.table[q, lb] = where[b]
        for s, d in zip(srcs, holes):
            self.ref[d], self.ref[s] = self.ref[s], 0
        self._free = [b for b in range(self.n_blocks) if self.ref[b] == 0]
        heapq.heapify(self._free)
        moves = []
        for s, d in zip(srcs, holes):
            if moves and moves[-1][0] + moves[-1][2] == s * self.bs and moves[-1][1] + moves[-1][2] == d * self.bs:
                moves[-1][2] += self.bs
            else:
                moves.append([s * self.bs, d * self.bs, self.bs])
        return [tuple(m) for m in moves]

    # -- checks ---------------------------------------------------------------
    def check(self):
        """Reference counts equal the number of table entries naming each
        block; a block is free exactly when unreferenced."""
        cnt = np.zeros(self.n_blocks, dtype=np.int64)
        live = self.table[self.table != INVALID]
        np.add.at(cnt, live, 1)
        assert np.array_equal(cnt, self.ref)
        assert sorted(self._free) == sorted(np.nonzero(self.ref == 0)[0].tolist())


def copy_blocks(pools, copies):
    """Apply block copies (src, dst) to every pool [n_blocks, ...] (numpy,
    in place); each destination takes the source block as it was before any
    copy of the list (sources and destinations are disjoint)."""
    for p in pools:
        if p is None:
            continue
        before = p.copy()
        for src, dst in copies:
            p[dst] = before[src]
