"""Paged GQA attention, as its plain definition, in float64.

Sources:
* "Tiered KV cache — architecture", section "The paged-attention block
  model" (and its figure): token position t of a sequence lives in physical
  block table[t // block_size] at slot t % block_size; a table entry equal to
  the invalid-block sentinel wipes those positions, which score -infinity and
  so get zero softmax weight.  Section "Kernel dispatch" restates the -inf
  rule for the kernel.
* "KV Cache Design — cells, format, sessions", section 1 "Positions and
  cells": a window is causal positions, one [lo, hi) range, or a map of up to
  KV_MAP_MAX_SPANS (cell, len) runs (a shared prefix plus a private run read
  in place).
* "KV cache" (sipllm), section "Problem": a decode step dots the new query
  against the stored history (softmax attention over the cached positions).

Readings where the pages are silent:
* the sentinel is -1; other negative ids are not produced by the inputs;
* a window cell is a logical position of the sequence, resolved through its
  own block table (so a hole scores -inf in every mode);
* the window belongs to the sequence and causality to the query: query j of
  sequence s sees W_s intersected with [0, min(seq_len_s, q_pos_j + 1));
  windows reaching outside [0, seq_len) are clamped, never an error;
* kv_map runs concatenate as a multiset (a position listed twice counts
  twice); a run of length 0 is unused; at most 8 runs;
* GQA: q head h reads kv head h // (n_q_heads / n_kv_heads);
* scores are scale * q.k; an empty visible set gives out = 0, lse = -inf;
* a decode query sits at position seq_len - 1 (so it sees all of W_s that
  lies in [0, seq_len)).
"""

from __future__ import annotations

import math

import numpy as np

from .formats import decode_rows

INVALID_BLOCK = -1
KV_MAP_MAX_SPANS = 8


def window_candidates(mode: str, seq_len: int, window_row=None, kv_map_row=None) -> np.ndarray:
    """Logical positions a sequence's window names, in window order (int64).

    causal: 0..seq_len-1; span (lo, hi): lo..hi-1; kv_map: the concatenation
    of cell..cell+len-1 over its runs (runs with len <= 0 are unused)."""
    if mode == "causal":
        return np.arange(seq_len, dtype=np.int64)
    if mode == "span":
        lo, hi = int(window_row[0]), int(window_row[1])
        return np.arange(lo, max(lo, hi), dtype=np.int64)
    if mode == "kv_map":
        runs = np.asarray(kv_map_row).reshape(-1, 2)
        if len(runs) > KV_MAP_MAX_SPANS:
            raise ValueError("more runs than KV_MAP_MAX_SPANS")
        parts = [np.arange(int(c), int(c) + int(n), dtype=np.int64) for c, n in runs if int(n) > 0]
        return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
    raise ValueError(f"unknown window mode {mode!r}")


def physical_row(block_table_row: np.ndarray, t: np.ndarray, block_size: int) -> np.ndarray:
    """Pool row of logical positions t: table[t // bs] * bs + t % bs, or -1
    where the table entry is the invalid-block sentinel."""
    t = np.asarray(t, dtype=np.int64)
    blk = block_table_row.astype(np.int64)[t // block_size]
    return np.where(blk == INVALID_BLOCK, -1, blk * block_size + t % block_size)


def visible_positions(cand: np.ndarray, block_table_row, block_size: int, seq_len: int, q_pos: int) -> np.ndarray:
    """Boolean mask over ``cand``: in [0, min(seq_len, q_pos+1)) and not in a hole."""
    limit = min(int(seq_len), int(q_pos) + 1)
    inside = (cand >= 0) & (cand < limit)
    ok = np.zeros(len(cand), dtype=bool)
    if inside.any():
        rows = physical_row(block_table_row, cand[inside], block_size)
        ok[inside] = rows >= 0
    return ok


def resolve_rows(w_mode, block_table, seq_lens, block_size, q_seq, q_pos, n_cand,
                 window=None, kv_map=None) -> np.ndarray:
    """int32 [Nq, n_cand]: for query j and candidate index i of its sequence's
    window enumeration, the pool row that slot reads, or -1 if the slot is
    past the enumeration, outside [0, min(seq_len, q_pos+1)) or in a hole."""
    nq = len(q_seq)
    out = np.full((nq, n_cand), -1, dtype=np.int64)
    for j in range(nq):
        s = int(q_seq[j])
        cand = window_candidates(w_mode, int(seq_lens[s]),
                                 None if window is None else window[s],
                                 None if kv_map is None else kv_map[s])[:n_cand]
        ok = visible_positions(cand, block_table[s], block_size, int(seq_lens[s]), int(q_pos[j]))
        rows = np.full(len(cand), -1, dtype=np.int64)
        if ok.any():
            rows[ok] = physical_row(block_table[s], cand[ok], block_size)
        out[j, : len(cand)] = rows
    return out.astype(np.int32)


def attend(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Softmax attention of query rows [g, hd] over keys/values [n, hd].

    out = sum_t w_t V_t / sum_t w_t with w_t = exp(x_t - max x), x_t = scale q.K_t;
    lse = max x + ln sum_t w_t.  Empty n gives out = 0 and lse = -inf."""
    g, hd = q_rows.shape
    if K.shape[0] == 0:
        return np.zeros((g, V.shape[1] if V.ndim == 2 else hd)), np.full(g, -np.inf)
    x = scale * (q_rows @ K.T)
    m = x.max(axis=1, keepdims=True)
    w = np.exp(x - m)
    z = w.sum(axis=1, keepdims=True)
    out = (w @ V) / z
    lse = m[:, 0] + np.log(z[:, 0])
    return out, lse


def lse_merge(parts):
    """Merge partial results (out_i, lse_i) of disjoint parts of one visible
    set: out = sum_i exp(lse_i - L) out_i with L = ln sum_i exp(lse_i).  Parts
    with lse = -inf (empty) carry no weight."""
    lses = np.stack([p[1] for p in parts])  # [P, g]
    outs = np.stack([p[0] for p in parts])  # [P, g, hd]
    m = lses.max(axis=0)
    empty = ~np.isfinite(m)
    mm = np.where(empty, 0.0, m)
    w = np.where(np.isfinite(lses), np.exp(lses - mm), 0.0)
    z = w.sum(axis=0)
    zs = np.where(empty, 1.0, z)
    out = (w[..., None] * outs).sum(axis=0) / zs[:, None]
    out = np.where(empty[:, None], 0.0, out)
    lse = np.where(empty, -np.inf, mm + np.log(zs))
    return out, lse


def paged_attention(q, q_seq, q_pos, k_pool, v_pool, k_fmt, v_fmt, block_table, seq_lens,
                    block_size, n_kv_heads, head_dim, scale, mode="causal", window=None,
                    kv_map=None, seqs=None):
    """Attention of every query row through its sequence's block table.

    q: [Nq, Hq, hd] (any float dtype); pools as in ``formats.decode_rows``.
    Returns out float64 [Nq, Hq, hd] and lse float64 [Nq, Hq] (natural log).
    ``seqs`` restricts the work to those sequences (other rows stay NaN)."""
    q = np.asarray(q)
    nq, hq, hd = q.shape
    g = hq // n_kv_heads
    out = np.full((nq, hq, hd), np.nan)
    lse = np.full((nq, hq), np.nan)
    q_seq = np.asarray(q_seq)
    todo = range(block_table.shape[0]) if seqs is None else seqs
    for s in todo:
        js = np.nonzero(q_seq == s)[0]
        if len(js) == 0:
            continue
        L = int(seq_lens[s])
        cand = window_candidates(mode, L, None if window is None else window[s],
                                 None if kv_map is None else kv_map[s])
        limit = min(L, int(np.max(np.asarray(q_pos)[js])) + 1)
        keep = visible_positions(cand, block_table[s], block_size, L, limit - 1)
        pos = cand[keep]
        rows = physical_row(block_table[s], pos, block_size)
        K = decode_rows(k_pool, k_fmt, rows, n_kv_heads, head_dim)
        V = decode_rows(v_pool, v_fmt, rows, n_kv_heads, head_dim)
        for j in js:
            vis = pos < min(L, int(q_pos[j]) + 1)
            for kvh in range(n_kv_heads):
                hs = slice(kvh * g, (kvh + 1) * g)
                o, l = attend(q[j, hs].astype(np.float64), K[vis, kvh], V[vis, kvh], scale)
                out[j, hs] = o
                lse[j, hs] = l
    return out, lse


def paged_decode(q, k_pool, v_pool, k_fmt, v_fmt, block_table, seq_lens, block_size,
                 n_kv_heads, head_dim, scale, mode="causal", window=None, kv_map=None, seqs=None):
    """One decode query per sequence, at position seq_len - 1."""
    S = block_table.shape[0]
    q_seq = np.arange(S)
    q_pos = np.asarray(seq_lens, dtype=np.int64) - 1
    return paged_attention(q, q_seq, q_pos, k_pool, v_pool, k_fmt, v_fmt, block_table,
                           seq_lens, block_size, n_kv_heads, head_dim, scale, mode,
                           window, kv_map, seqs)


def paged_prefill(q, cu_q, q_pos, k_pool, v_pool, k_fmt, v_fmt, block_table, seq_lens,
                  block_size, n_kv_heads, head_dim, scale, mode="kv_map", window=None,
                  kv_map=None, seqs=None):
    """A chunk of queries per sequence (rows cu_q[s]..cu_q[s+1]-1) at
    positions q_pos, causal inside the sequence's window."""
    cu_q = np.asarray(cu_q)
    q_seq = np.repeat(np.arange(len(cu_q) - 1), np.diff(cu_q))
    return paged_attention(q, q_seq, q_pos, k_pool, v_pool, k_fmt, v_fmt, block_table,
                           seq_lens, block_size, n_kv_heads, head_dim, scale, mode,
                           window, kv_map, seqs)


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
