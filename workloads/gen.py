"""Synthetic inputs with the shapes of the five paged-attention workloads.

Structure (tables, lengths, windows, positions, moves) is drawn with numpy's
PCG64 ``default_rng(seed)``, so it is identical on every machine.  Values
(q, K, V) are N(0, 1) float32 draws from a seeded ``torch.Generator`` on the
device that will hold them, then cast to f16 or encoded to q8_0; pool rows
that no table entry references, rows behind a hole, and tail rows past a
sequence's length are filled with NaN so any stray read shows up.

The five workloads (ids 1..5) and their reduced "small" variants, which keep
the same structure at sizes the CPU oracle finishes in seconds:

1. tiny decode: 1 seq, 4 q / 2 kv heads, head_dim 64, block 16, 256 tokens
   in 16 blocks scattered by a random permutation of a 32-block pool, f32.
2. SmolLM2-135M-like layer: 9 q / 3 kv heads, head_dim 64, block 16, f16,
   32 seqs with 512..8192 tokens, 5% of logical blocks are holes.
3. 7B-class: 32 q / 8 kv heads, head_dim 128, block 16, f16, 64 seqs in 16
   groups of 4 copy-on-write forks sharing a 2048-token prefix (identical
   physical block ids) plus private tails, 4096..32768 tokens each.
4. windowed prefill: 32 q / 8 kv heads, head_dim 128, block 32, K q8_0,
   V f16, 16 seqs x 64-query chunks; seqs 0-7 read one [lo, hi) span,
   seqs 8-15 a map of 4 (cell, len) runs; causal inside the window.
5. long context: 32 q / 8 kv heads, head_dim 256, block 16, f16, 8 seqs of
   131072 tokens from a pool of 2**17 blocks; plus 10k overlapping row moves.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

FMT_BYTES = {"f32": 4, "f16": 2}

# Window modes.  The causal mode reads positions [0, seq_len); a span reads
# one [lo, hi) pair per sequence; a kv_map reads up to 8 (cell, len) runs.
MODES = ("causal", "span", "kv_map")
KV_MAP_MAX_SPANS = 8
INVALID_BLOCK = -1


def q8_0_seg_bytes(head_dim: int) -> int:
    """Bytes of one token of one kv head in q8_0: head_dim/32 blocks of
    (f16 scale + 32 int8), rounded up to whole 4-byte words."""
    return ((head_dim // 32) * 34 + 3) // 4 * 4


def q8_0_row_bytes(n_kv_heads: int, head_dim: int) -> int:
    """Bytes of one token (all kv heads) in q8_0."""
    return n_kv_heads * q8_0_seg_bytes(head_dim)


@dataclasses.dataclass
class Workload:
    name: str
    cfg: int
    seed: int
    n_seqs: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    n_pool_blocks: int
    q_fmt: str
    k_fmt: str
    v_fmt: str
    scale: float
    block_table: np.ndarray  # int32 [S, MB]; -1 marks a hole
    seq_lens: np.ndarray  # int32 [S]
    mode: str  # "causal" | "span" | "kv_map"
    window: Optional[np.ndarray] = None  # span: int32 [S, 2] (lo, hi)
    kv_map: Optional[np.ndarray] = None  # kv_map: int32 [S, K, 2] (cell, len)
    # prefill only: queries of seq s are rows cu_q[s]..cu_q[s+1]-1
    cu_q: Optional[np.ndarray] = None  # int32 [S+1]
    q_pos: Optional[np.ndarray] = None  # int32 [Nq]
    kind: str = "decode"  # "decode" | "prefill"

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def n_queries(self) -> int:
        if self.kind == "decode":
            return self.n_seqs
        return int(self.cu_q[-1])

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    def row_bytes(self, which: str) -> int:
        fmt = self.k_fmt if which == "k" else self.v_fmt
        if fmt == "q8_0":
            return q8_0_row_bytes(self.n_kv_heads, self.head_dim)
        return self.n_kv_heads * self.head_dim * FMT_BYTES[fmt]

    def q_seq(self) -> np.ndarray:
        """Sequence index of each query row."""
        if self.kind == "decode":
            return np.arange(self.n_seqs, dtype=np.int32)
        return np.repeat(np.arange(self.n_seqs, dtype=np.int32), np.diff(self.cu_q))

    def query_pos(self) -> np.ndarray:
        """Position of each query; a decode query sits at seq_len - 1."""
        if self.kind == "decode":
            return (self.seq_lens - 1).astype(np.int32)
        return self.q_pos


@dataclasses.dataclass
class MoveSet:
    seed: int
    n_rows: int
    moves: np.ndarray  # int32 [n, 3] (src, dst, len) in pool rows


# ----------------------------------------------------------------------------
# structure


def _tables_from_perm(perm, nblocks, mb):
    s = len(nblocks)
    table = np.full((s, mb), INVALID_BLOCK, dtype=np.int32)
    off = 0
    for i, nb in enumerate(nblocks):
        table[i, :nb] = perm[off : off + nb]
        off += nb
    return table, off


def _cfg1(seed, small):
    rng = np.random.default_rng(seed)
    bs, ctx, pool = 16, 256, 32
    table = rng.permutation(pool)[: ctx // bs].astype(np.int32)[None, :]
    return Workload(
        name="tiny-decode", cfg=1, seed=seed, n_seqs=1, n_q_heads=4, n_kv_heads=2,
        head_dim=64, block_size=bs, n_pool_blocks=pool, q_fmt="f32", k_fmt="f32",
        v_fmt="f32", scale=1.0 / math.sqrt(64), block_table=table,
        seq_lens=np.array([ctx], dtype=np.int32), mode="causal")


def _holes(rng, table, nblocks, frac):
    """Set round(frac * total logical blocks) entries to -1, chosen uniformly
    among all logical blocks except each sequence's last one."""
    cand = [(s, b) for s, nb in enumerate(nblocks) for b in range(nb - 1)]
    n_holes = int(round(frac * sum(nblocks)))
    pick = rng.choice(len(cand), size=min(n_holes, len(cand)), replace=False)
    for i in np.sort(pick):
        s, b = cand[i]
        table[s, b] = INVALID_BLOCK


def _cfg2(seed, small):
    rng = np.random.default_rng(seed)
    bs = 16
    if small:
        s, lo, hi, pool = 6, 40, 300, 1 << 7
    else:
        s, lo, hi, pool = 32, 512, 8192, 1 << 15
    ctx = rng.integers(lo, hi + 1, size=s).astype(np.int32)
    nblocks = [(int(c) + bs - 1) // bs for c in ctx]
    mb = (hi + bs - 1) // bs
    table, _ = _tables_from_perm(rng.permutation(pool), nblocks, mb)
    _holes(rng, table, nblocks, 0.05)
    return Workload(
        name="smollm2-135m-like" + ("-small" if small else ""), cfg=2, seed=seed,
        n_seqs=s, n_q_heads=9, n_kv_heads=3, head_dim=64, block_size=bs,
        n_pool_blocks=pool, q_fmt="f16", k_fmt="f16", v_fmt="f16",
        scale=1.0 / math.sqrt(64), block_table=table, seq_lens=ctx, mode="causal")


def _cfg3(seed, small):
    rng = np.random.default_rng(seed)
    bs = 16
    if small:
        groups, forks, prefix_blocks, lo, hi, pool = 2, 4, 4, 80, 400, 1 << 8
    else:
        groups, forks, prefix_blocks, lo, hi, pool = 16, 4, 128, 4096, 32768, 1 << 17
    s = groups * forks
    mb = (hi + bs - 1) // bs
    ctx = rng.integers(lo, hi + 1, size=s).astype(np.int32)
    perm = rng.permutation(pool)
    table = np.full((s, mb), INVALID_BLOCK, dtype=np.int32)
    off = 0
    for g in range(groups):
        prefix = perm[off : off + prefix_blocks]
        off += prefix_blocks
        for f in range(forks):
            i = g * forks + f
            nb = (int(ctx[i]) + bs - 1) // bs
            table[i, :prefix_blocks] = prefix
            tail = nb - prefix_blocks
            table[i, prefix_blocks:nb] = perm[off : off + tail]
            off += tail
    assert off <= pool
    return Workload(
        name="7b-class-cow-forks" + ("-small" if small else ""), cfg=3, seed=seed,
        n_seqs=s, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=bs,
        n_pool_blocks=pool, q_fmt="f16", k_fmt="f16", v_fmt="f16",
        scale=1.0 / math.sqrt(128), block_table=table, seq_lens=ctx, mode="causal")


def _cfg4(seed, small, mode=None):
    rng = np.random.default_rng(seed)
    bs = 32
    if small:
        s, nq, lo, hi, pool, rlo, rhi = 4, 16, 96, 400, 1 << 6, 16, 64
    else:
        s, nq, lo, hi, pool, rlo, rhi = 16, 64, 2048, 8192, 1 << 13, 64, 512
    L = rng.integers(lo, hi + 1, size=s).astype(np.int32)
    nblocks = [(int(c) + bs - 1) // bs for c in L]
    mb = (hi + bs - 1) // bs
    table, _ = _tables_from_perm(rng.permutation(pool), nblocks, mb)
    half = s // 2
    # every sequence gets a kv_map; the first half read one [lo, L) span,
    # stored both as a span window and as a one-run map with 3 empty runs.
    kv_map = np.zeros((s, 4, 2), dtype=np.int32)
    window = np.zeros((s, 2), dtype=np.int32)
    for i in range(s):
        Li = int(L[i])
        if i < half:
            lo_i = int(rng.integers(0, Li // 2 + 1))
            window[i] = (lo_i, Li)
            kv_map[i, 0] = (lo_i, Li - lo_i)
        else:
            r = int(rng.integers(rlo, rhi + 1))
            cuts = np.sort(rng.choice(Li - r, size=6, replace=False))
            runs = [(int(cuts[2 * k]), int(cuts[2 * k + 1] - cuts[2 * k])) for k in range(3)]
            runs.append((Li - r, r))
            kv_map[i] = np.array(runs, dtype=np.int32)
            window[i] = (Li - r, Li)  # unused by the kv_map half
    cu_q = np.arange(s + 1, dtype=np.int32) * nq
    q_pos = np.concatenate([np.arange(int(Li) - nq, int(Li), dtype=np.int32) for Li in L])
    w = Workload(
        name="windowed-prefill" + ("-small" if small else ""), cfg=4, seed=seed,
        n_seqs=s, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=bs,
        n_pool_blocks=pool, q_fmt="f16", k_fmt="q8_0", v_fmt="f16",
        scale=1.0 / math.sqrt(128), block_table=table, seq_lens=L, mode="kv_map",
        window=window, kv_map=kv_map, cu_q=cu_q, q_pos=q_pos, kind="prefill")
    if mode == "span":
        w = _select_seqs(w, np.arange(half))
        w.mode, w.kv_map = "span", None
    elif mode == "kv_map_only":
        w = _select_seqs(w, np.arange(half, s))
    return w


def _select_seqs(w: Workload, idx) -> Workload:
    """The same workload restricted to a subset of its sequences (same pool)."""
    idx = np.asarray(idx)
    d = dataclasses.replace(w)
    d.n_seqs = len(idx)
    d.block_table = w.block_table[idx].copy()
    d.seq_lens = w.seq_lens[idx].copy()
    if w.window is not None:
        d.window = w.window[idx].copy()
    if w.kv_map is not None:
        d.kv_map = w.kv_map[idx].copy()
    if w.kind == "prefill":
        qs = [np.arange(w.cu_q[i], w.cu_q[i + 1]) for i in idx]
        lens = np.array([len(x) for x in qs], dtype=np.int32)
        d.cu_q = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        d.q_pos = np.concatenate([w.q_pos[x] for x in qs]).astype(np.int32)
    return d


def _cfg5(seed, small):
    rng = np.random.default_rng(seed)
    bs = 16
    if small:
        s, ctx, pool = 2, 1024, 1 << 8
    else:
        s, ctx, pool = 8, 131072, 1 << 17
    nb = ctx // bs
    table, _ = _tables_from_perm(rng.permutation(pool), [nb] * s, nb)
    return Workload(
        name="long-context" + ("-small" if small else ""), cfg=5, seed=seed,
        n_seqs=s, n_q_heads=32, n_kv_heads=8, head_dim=256, block_size=bs,
        n_pool_blocks=pool, q_fmt="f16", k_fmt="f16", v_fmt="f16",
        scale=1.0 / math.sqrt(256), block_table=table,
        seq_lens=np.full(s, ctx, dtype=np.int32), mode="causal")


def make(cfg: int, small: bool = False, seed: Optional[int] = None, mode: Optional[str] = None) -> Workload:
    """Structure of workload ``cfg`` (1..5); ``small`` keeps the structure at
    reduced size.  Workload 4 accepts mode="span" (its span half) or
    "kv_map_only" (its map half); by default it is the whole batch as maps."""
    seed = cfg if seed is None else seed
    if cfg == 1:
        return _cfg1(seed, small)
    if cfg == 2:
        return _cfg2(seed, small)
    if cfg == 3:
        return _cfg3(seed, small)
    if cfg == 4:
        return _cfg4(seed, small, mode)
    if cfg == 5:
        return _cfg5(seed, small)
    raise ValueError(f"no workload {cfg}")


def make_moves(seed: int = 55, n_moves: int = 10000, n_rows: int = 1 << 21,
               region: int = 1 << 16, max_len: int = 32) -> MoveSet:
    """Random overlapping row moves: len ~ U{1..max_len}, src ~ U{0..region-len};
    half slide by delta ~ U{-2len..2len}\\{0} (redrawn until in range), the
    other half jump to dst ~ U{0..region-len}."""
    rng = np.random.default_rng(seed)
    kinds = rng.permutation(np.arange(n_moves) % 2)
    out = np.zeros((n_moves, 3), dtype=np.int32)
    for i in range(n_moves):
        ln = int(rng.integers(1, max_len + 1))
        src = int(rng.integers(0, region - ln + 1))
        if kinds[i] == 0:
            while True:
                d = int(rng.integers(-2 * ln, 2 * ln + 1))
                if d != 0 and 0 <= src + d <= n_rows - ln:
                    break
            dst = src + d
        else:
            dst = int(rng.integers(0, region - ln + 1))
        out[i] = (src, dst, ln)
    return MoveSet(seed=seed, n_rows=n_rows, moves=out)


@dataclasses.dataclass
class StoreSet:
    """New K/V rows to store: token t belongs to sequence seq_ids[t] and sits
    at position pos[t]; its rows go to the pool through block_table."""
    name: str
    seed: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    n_pool_blocks: int
    src_fmt: str  # "f32" | "f16": type of the new rows
    k_fmt: str
    v_fmt: str
    block_table: np.ndarray  # int32 [S, MB]; -1 marks a hole
    seq_ids: np.ndarray  # int32 [n_tok]
    pos: np.ndarray  # int32 [n_tok]

    @property
    def n_tok(self) -> int:
        return int(len(self.pos))

    @property
    def n_seqs(self) -> int:
        return int(self.block_table.shape[0])


def make_store(seed: int, n_seqs: int, n_kv_heads: int, head_dim: int, block_size: int, n_pool_blocks: int,
               max_blocks: int, tok=(1, 40), src_fmt: str = "f16", k_fmt: str = "q8_0", v_fmt: str = "f16",
               hole_frac: float = 0.0, shuffle: bool = True) -> StoreSet:
    """Each sequence owns distinct pool blocks from one permutation (its whole
    table is filled, then hole_frac of the entries become holes) and receives
    a run of n_s ~ U{tok} new tokens at positions [p0, p0 + n_s), p0 drawn so
    the run fits the table: a prefill chunk, or a decode append when n_s = 1.
    Tokens are listed in random order when shuffle."""
    rng = np.random.default_rng(seed)
    if n_seqs * max_blocks > n_pool_blocks:
        raise ValueError("pool too small for the tables")
    perm = rng.permutation(n_pool_blocks)[: n_seqs * max_blocks]
    table = perm.reshape(n_seqs, max_blocks).astype(np.int32)
    if hole_frac > 0:
        table[rng.random(table.shape) < hole_frac] = INVALID_BLOCK
    cap = max_blocks * block_size
    seq_ids, pos = [], []
    for s_ in range(n_seqs):
        n = int(rng.integers(tok[0], min(tok[1], cap) + 1))
        p0 = int(rng.integers(0, cap - n + 1))
        seq_ids.append(np.full(n, s_, dtype=np.int32))
        pos.append(np.arange(p0, p0 + n, dtype=np.int32))
    seq_ids = np.concatenate(seq_ids)
    pos = np.concatenate(pos)
    if shuffle:
        order = rng.permutation(len(pos))
        seq_ids, pos = seq_ids[order], pos[order]
    return StoreSet(name="store", seed=seed, n_kv_heads=n_kv_heads, head_dim=head_dim, block_size=block_size,
                    n_pool_blocks=n_pool_blocks, src_fmt=src_fmt, k_fmt=k_fmt, v_fmt=v_fmt, block_table=table,
                    seq_ids=seq_ids, pos=pos)


def store_of_workload(w: Workload, src_fmt: str = "f16") -> StoreSet:
    """The store that fills workload w's pools: every position [0, seq_len)
    of every sequence, in sequence order (the prefill of the whole context)."""
    seq_ids = np.concatenate([np.full(int(L), s_, dtype=np.int32) for s_, L in enumerate(w.seq_lens)])
    pos = np.concatenate([np.arange(int(L), dtype=np.int32) for L in w.seq_lens])
    return StoreSet(name=f"store-{w.name}", seed=w.seed, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                    block_size=w.block_size, n_pool_blocks=w.n_pool_blocks, src_fmt=src_fmt, k_fmt=w.k_fmt,
                    v_fmt=w.v_fmt, block_table=w.block_table.copy(), seq_ids=seq_ids, pos=pos)


def store_values(st: StoreSet, device="cpu", seed_offset: int = 0):
    """New rows (k_new, v_new) [n_tok, n_kv_heads, head_dim] in st.src_fmt:
    N(0, 1) float32 draws from a torch.Generator seeded with st.seed on the
    target device, cast to float16 when the source is f16."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(1000003 * st.seed + 17 + seed_offset)
    shape = (st.n_tok, st.n_kv_heads, st.head_dim)
    k = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if st.src_fmt == "f16":
        k, v = k.half(), v.half()
    return k.contiguous(), v.contiguous()


def pool_width(fmt: str, head_dim: int) -> int:
    """Last-axis length of a pool tensor: head_dim values, or q8_0 bytes."""
    return q8_0_seg_bytes(head_dim) if fmt == "q8_0" else head_dim


# ----------------------------------------------------------------------------
# values


def referenced_rows(w: Workload) -> np.ndarray:
    """Boolean [n_pool_blocks * block_size]: rows that hold a live token, i.e.
    row table[s][b]*bs + slot for every non-hole logical block b and slot
    position b*bs + slot < seq_len[s]."""
    bs = w.block_size
    live = np.zeros(w.n_pool_blocks * bs, dtype=bool)
    for s in range(w.n_seqs):
        L = int(w.seq_lens[s])
        nb = (L + bs - 1) // bs
        ids = w.block_table[s, :nb].astype(np.int64)
        pos = np.arange(nb * bs)
        keep = (pos < L) & (np.repeat(ids, bs) >= 0)
        rows = np.repeat(ids, bs) * bs + np.tile(np.arange(bs), nb)
        live[rows[keep]] = True
    return live


def encode_q8_0(x, n_kv_heads: int, head_dim: int):
    """Encode float32 rows [N, n_kv_heads, head_dim] as q8_0 bytes
    [N, n_kv_heads, seg_bytes]:
    per 32-element block d = amax/127 (f32), stored as f16 (round to nearest
    even), codes = clamp(round_half_even(x / d), -127, 127); amax = 0 gives
    d = 0 and zero codes.  Block = 2 bytes of little-endian f16 then 32 int8."""
    import torch

    n = x.shape[0]
    nb = head_dim // 32
    xb = x.reshape(n, n_kv_heads, nb, 32).to(torch.float32)
    amax = xb.abs().amax(dim=-1)
    d = amax / 127.0
    safe = torch.where(d > 0, d, torch.ones_like(d))
    codes = torch.round(xb / safe[..., None]).clamp_(-127, 127)
    codes = torch.where((d > 0)[..., None], codes, torch.zeros_like(codes)).to(torch.int8)
    d16 = d.to(torch.float16)
    blk = torch.cat([d16.contiguous().view(torch.uint8).reshape(n, n_kv_heads, nb, 2),
                     codes.view(torch.uint8)], dim=-1)
    raw = blk.reshape(n, n_kv_heads, nb * 34)
    sb = q8_0_seg_bytes(head_dim)
    if sb != raw.shape[2]:
        pad = torch.zeros((n, n_kv_heads, sb - raw.shape[2]), dtype=torch.uint8, device=raw.device)
        raw = torch.cat([raw, pad], dim=2)
    return raw.contiguous()


def _gen_pool(w: Workload, fmt: str, gen, device, live_rows, chunk_rows: int):
    """One pool in the block layout [n_blocks, n_kv_heads, block_size, W]
    (W = head_dim values, or q8_0 segment bytes): inside a block, each kv
    head's block_size token entries are contiguous.  Values are drawn one
    token row [n_kv_heads, head_dim] at a time in pool row order."""
    import torch

    bs, hkv, hd = w.block_size, w.n_kv_heads, w.head_dim
    nblk = w.n_pool_blocks
    if fmt == "q8_0":
        out = torch.empty((nblk, hkv, bs, q8_0_seg_bytes(hd)), dtype=torch.uint8, device=device)
    else:
        dt = torch.float32 if fmt == "f32" else torch.float16
        out = torch.empty((nblk, hkv, bs, hd), dtype=dt, device=device)
    live = torch.from_numpy(live_rows).to(device)
    cb = max(1, chunk_rows // bs)  # whole blocks per chunk
    for b0 in range(0, nblk, cb):
        b1 = min(nblk, b0 + cb)
        r0, r1 = b0 * bs, b1 * bs
        x = torch.randn((r1 - r0, hkv, hd), generator=gen, device=device, dtype=torch.float32)
        dead = ~live[r0:r1]
        if fmt == "q8_0":
            enc = encode_q8_0(x, hkv, hd)  # [rows, hkv, seg]
            # poisoned rows: every q8_0 block's scale is a quiet NaN (f16 0x7E00)
            nb = hd // 32
            blk = enc[:, :, : nb * 34].reshape(r1 - r0, hkv, nb, 34)
            blk[dead, :, :, 0] = 0x00
            blk[dead, :, :, 1] = 0x7E
            enc[:, :, : nb * 34] = blk.reshape(r1 - r0, hkv, nb * 34)
            rows = enc
        else:
            x[dead] = float("nan")
            rows = x.to(out.dtype)
        out[b0:b1] = rows.reshape(b1 - b0, bs, hkv, -1).permute(0, 2, 1, 3)
    return out


def materialize(w: Workload, device="cpu", chunk_rows: int = 1 << 16):
    """Draw (q, k_pool, v_pool) as torch tensors on ``device``.

    q is [Nq, Hq, hd] in q_fmt; pools are [n_blocks, Hkv, bs, hd] (f32/f16)
    or uint8 [n_blocks, Hkv, bs, seg_bytes] (q8_0).  Seeds: q from seed*1000+1, K from
    seed*1000+2, V from seed*1000+3, each on its own generator."""
    import torch

    live = referenced_rows(w)
    gq = torch.Generator(device=device).manual_seed(w.seed * 1000 + 1)
    gk = torch.Generator(device=device).manual_seed(w.seed * 1000 + 2)
    gv = torch.Generator(device=device).manual_seed(w.seed * 1000 + 3)
    qdt = torch.float32 if w.q_fmt == "f32" else torch.float16
    q = torch.randn((w.n_queries, w.n_q_heads, w.head_dim), generator=gq, device=device,
                    dtype=torch.float32).to(qdt)
    k = _gen_pool(w, w.k_fmt, gk, device, live, chunk_rows)
    v = _gen_pool(w, w.v_fmt, gv, device, live, chunk_rows)
    return q, k, v


def host_subset(w: Workload, seqs, k_pool, v_pool):
    """Copy just the pool blocks that sequences ``seqs`` reference to host
    numpy arrays, with block ids renumbered densely.  Returns
    (sub_workload, k_host, v_host); the attention result is unchanged because
    the table is rewritten to match the moved blocks."""
    import torch

    seqs = np.asarray(seqs)
    sub = _select_seqs(w, seqs)
    ids = np.unique(sub.block_table[sub.block_table >= 0])
    remap = np.full(w.n_pool_blocks, INVALID_BLOCK, dtype=np.int64)
    remap[ids] = np.arange(len(ids))
    t = sub.block_table.astype(np.int64)
    sub.block_table = np.where(t >= 0, remap[np.maximum(t, 0)], INVALID_BLOCK).astype(np.int32)
    sub.n_pool_blocks = len(ids)
    idx = torch.from_numpy(ids.astype(np.int64)).to(k_pool.device)
    kh = k_pool.index_select(0, idx).cpu().numpy()
    vh = v_pool.index_select(0, idx).cpu().numpy()
    return sub, kh, vh


def make_custom(seed: int, n_seqs: int, n_q_heads: int, n_kv_heads: int, head_dim: int, block_size: int,
                fmts=("f16", "f16", "f16"), ctx=(1, 300), hole_frac: float = 0.05, mode: str = "causal",
                n_runs: int = 4, kind: str = "decode", q_per_seq=(1, 40), pool_slack: int = 8,
                max_blocks: Optional[int] = None) -> Workload:
    """A random workload of any supported geometry: seq lengths ~ U{ctx},
    blocks from one pool permutation, a fraction of non-final logical blocks
    turned into holes, and random windows.  Spans are drawn to also reach
    outside [0, seq_len); kv_map runs may overlap, be empty or stick out.
    Prefill draws q_per_seq queries per sequence at sorted distinct
    positions in [0, seq_len)."""
    rng = np.random.default_rng(seed)
    bs = block_size
    L = rng.integers(ctx[0], ctx[1] + 1, size=n_seqs).astype(np.int32)
    nblocks = [(int(c) + bs - 1) // bs for c in L]
    mb = max_blocks or max(1, (ctx[1] + bs - 1) // bs)
    pool = sum(nblocks) + pool_slack
    table, _ = _tables_from_perm(rng.permutation(pool), nblocks, mb)
    if hole_frac > 0:
        _holes(rng, table, nblocks, hole_frac)
    q_fmt, k_fmt, v_fmt = fmts
    w = Workload(name="custom", cfg=0, seed=seed, n_seqs=n_seqs, n_q_heads=n_q_heads,
                 n_kv_heads=n_kv_heads, head_dim=head_dim, block_size=bs, n_pool_blocks=pool,
                 q_fmt=q_fmt, k_fmt=k_fmt, v_fmt=v_fmt, scale=1.0 / math.sqrt(head_dim),
                 block_table=table, seq_lens=L, mode=mode, kind=kind)
    win = np.zeros((n_seqs, 2), dtype=np.int32)
    km = np.zeros((n_seqs, n_runs, 2), dtype=np.int32)
    for s in range(n_seqs):
        Ls = int(L[s])
        a, b = sorted(rng.integers(-3, Ls + 4, size=2).tolist())
        win[s] = (a, b)
        for r in range(n_runs):
            c = int(rng.integers(-2, Ls + 2))
            n = int(rng.integers(-1, max(2, Ls // 3)))
            km[s, r] = (c, n)
    w.window = win
    w.kv_map = km
    if kind == "prefill":
        nq = [int(rng.integers(q_per_seq[0], q_per_seq[1] + 1)) for _ in range(n_seqs)]
        nq = [min(n, int(Ls)) for n, Ls in zip(nq, L)]
        w.cu_q = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
        w.q_pos = np.concatenate([np.sort(rng.choice(int(Ls), size=n, replace=False))
                                  for n, Ls in zip(nq, L)]).astype(np.int32)
    return w
