"""Paged GQA attention for MI355X (gfx950): Python binding of libpkv.so.

Every function here only marshals torch tensors into the C ABI declared in
include/pkv.h (pointers, sizes, the current HIP stream) and calls it; all
computation runs in the library's HIP kernels.  If the library is missing,
or a call is refused, the call raises: there is no fallback path.

Pools are [n_blocks, n_kv_heads, block_size, W] (inside a block, each kv
head's token entries are contiguous).  Formats follow the tensors' dtypes:
float32 -> f32, float16 -> f16, and a uint8 pool with W = q8_0 segment bytes
-> q8_0.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpkv.so")

F32, F16, Q8_0 = 0, 1, 2
WIN_CAUSAL, WIN_SPAN, WIN_KV_MAP = 0, 1, 2
MODES = {"causal": WIN_CAUSAL, "span": WIN_SPAN, "kv_map": WIN_KV_MAP}
FLAG_CHECKED = 1
INVALID_BLOCK_ID = -1
KV_MAP_MAX_SPANS = 8

STATUS = {0: "PKV_OK", 1: "PKV_E_ARG", 2: "PKV_E_UNSUPPORTED", 3: "PKV_E_WORKSPACE", 4: "PKV_E_DEVICE",
          5: "PKV_E_CAPACITY"}

# Every symbol include/pkv.h declares.
EXPORTS = (
    "pkv_row_bytes",
    "pkv_decode_workspace_bytes",
    "pkv_decode_split_tokens",
    "pkv_paged_attn_decode_noalloc",
    "pkv_paged_attn_decode",
    "pkv_paged_attn_decode_partials",
    "pkv_paged_attn_decode_merge",
    "pkv_prefill_workspace_bytes",
    "pkv_paged_attn_prefill_window",
    "pkv_order_moves",
    "pkv_copy_cells_plan_words",
    "pkv_copy_cells_plan",
    "pkv_copy_cells_stage_bytes",
    "pkv_copy_cells_apply",
    "pkv_copy_cells_workspace_bytes",
    "pkv_kv_copy_cells",
    "pkv_kv_store",
    "pkv_pool_create",
    "pkv_pool_destroy",
    "pkv_pool_free_blocks",
    "pkv_pool_can_allocate",
    "pkv_pool_refcount",
    "pkv_pool_seq_len",
    "pkv_pool_fork",
    "pkv_pool_remove",
    "pkv_pool_prepare_writes",
    "pkv_pool_defrag",
    "pkv_pool_export",
    "pkv_cow_apply",
    "pkv_int4_blob_bytes",
    "pkv_int4_encode",
    "pkv_int4_decode",
    "pkv_resolve_rows",
    "pkv_last_error",
    "pkv_version",
)


class PkvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


class Shape(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("n_pool_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("q_fmt", ctypes.c_int32),
        ("k_fmt", ctypes.c_int32),
        ("v_fmt", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
        ("split_tokens", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_table_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SH = ctypes.POINTER(Shape)
    sig = {
        "pkv_row_bytes": (I64, [I32, I32, I32]),
        "pkv_decode_workspace_bytes": (SZ, [SH, I32, I32]),
        "pkv_decode_split_tokens": (I32, [SH, I32, I32]),
        "pkv_paged_attn_decode": (I32, [SH, P, P, P, P, P, I32, I32, P, P, P, P, SZ, P]),
        "pkv_paged_attn_decode_partials": (I32, [SH, P, P, P, P, P, I32, I32, P, P, SZ, P]),
        "pkv_paged_attn_decode_merge": (I32, [SH, P, I32, I32, P, P, P, P, SZ, P]),
        "pkv_paged_attn_decode_noalloc": (I32, [SH, P, P, P, P, P, I32, I32, P, P, P, P]),
        "pkv_prefill_workspace_bytes": (SZ, [SH, I32, I32, I32, I32]),
        "pkv_paged_attn_prefill_window": (I32, [SH, I32, I32, P, P, P, P, P, P, P, I32, I32, P, P, P, P, SZ, P]),
        "pkv_order_moves": (I32, [P, I32, P, P]),
        "pkv_copy_cells_workspace_bytes": (SZ, [P, I32, I64, I64]),
        "pkv_copy_cells_plan_words": (I64, [P, I32]),
        "pkv_copy_cells_plan": (I32, [P, I32, I64, P, I64, P]),
        "pkv_copy_cells_stage_bytes": (SZ, [P, I64, I64]),
        "pkv_copy_cells_apply": (I32, [P, P, I32, I32, I32, I64, I64, P, P, P, SZ, P]),
        "pkv_kv_copy_cells": (I32, [P, P, I32, I32, I32, I64, I64, P, I32, P, SZ, P]),
        "pkv_kv_store": (I32, [SH, I32, I32, P, P, P, P, P, P, P, P, P]),
        "pkv_pool_create": (I32, [I32, I32, I32, I32, I32, ctypes.POINTER(P)]),
        "pkv_pool_destroy": (None, [P]),
        "pkv_pool_free_blocks": (I32, [P]),
        "pkv_pool_can_allocate": (I32, [P, I32]),
        "pkv_pool_refcount": (I32, [P, I32]),
        "pkv_pool_seq_len": (I32, [P, I32]),
        "pkv_pool_fork": (I32, [P, I32, I32, I32]),
        "pkv_pool_remove": (I32, [P, I32, I32, I32]),
        "pkv_pool_prepare_writes": (I32, [P, I32, P, P, P, P, I32, P]),
        "pkv_pool_defrag": (I32, [P, I32, P, I32, P]),
        "pkv_pool_export": (I32, [P, P, P]),
        "pkv_cow_apply": (I32, [P, P, I32, I64, I64, P, I32, P, I64, P]),
        "pkv_int4_blob_bytes": (I64, [I64]),
        "pkv_int4_encode": (I32, [P, I32, I32, I64, P, I32, P, I64, P]),
        "pkv_int4_decode": (I32, [P, I64, I32, P, I32, I32, I64, P, P]),
        "pkv_resolve_rows": (I32, [SH, I32, P, P, P, P, I32, I32, P, I32, P, P]),
        "pkv_last_error": (ctypes.c_char_p, []),
        "pkv_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(status: int):
    if status != 0:
        raise PkvError(status, lib().pkv_last_error().decode())


def last_error() -> str:
    return lib().pkv_last_error().decode()


def version() -> str:
    return lib().pkv_version().decode()


# ---------------------------------------------------------------------------
# marshalling helpers


def _torch():
    import torch

    return torch


def _ptr(t) -> Optional[int]:
    """Device address of a tensor argument (kernels dereference it)."""
    if t is None:
        return None
    if t.device.type != "cuda":
        raise TypeError(f"expected a GPU tensor, got one on {t.device}")
    return t.data_ptr()


def _on_one_gpu(*tensors):
    """Every given tensor lives on the same GPU (None entries are skipped):
    a host pointer or another GPU's memory handed to a kernel would fault."""
    dev = None
    for t in tensors:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise TypeError(f"expected GPU tensors, got one on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise TypeError(f"tensors on {dev} and {t.device}: all must be on one GPU")


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _fmt_of(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.uint8:
        return Q8_0
    raise TypeError(f"no KV format for dtype {t.dtype}")


def _i32(t, name):
    torch = _torch()
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    return t


def row_bytes(fmt: int, n_kv_heads: int, head_dim: int) -> int:
    return int(lib().pkv_row_bytes(fmt, n_kv_heads, head_dim))


def make_shape(q, k_pool, v_pool, block_table, n_seqs: int, scale: float, flags: int = 0,
               split_tokens: int = 0) -> Shape:
    """pkv_shape from the tensors: q [.., Hq, hd]; v_pool [NB, Hkv, bs, hd]."""
    for name, t in (("q", q), ("k_pool", k_pool), ("v_pool", v_pool)):
        if not t.is_contiguous():
            raise TypeError(f"{name} must be contiguous")
    _i32(block_table, "block_table")
    if v_pool.dim() != 4 or k_pool.dim() != 4:
        raise TypeError("pools must be [n_blocks, n_kv_heads, block_size, W]")
    nb, hkv, bs, hd = v_pool.shape
    if tuple(k_pool.shape[:3]) != (nb, hkv, bs):
        raise TypeError("k_pool and v_pool disagree on (n_blocks, n_kv_heads, block_size)")
    kw = row_bytes(_fmt_of(k_pool), 1, hd) // k_pool.element_size()
    if k_pool.shape[3] != kw:
        raise TypeError(f"k_pool rows are {k_pool.shape[3]} wide; head_dim {hd} in its format needs {kw}")
    if q.dim() != 3 or q.shape[-1] != hd:
        raise TypeError(f"q must be [n, n_q_heads, {hd}]")
    if block_table.dim() != 2 or block_table.shape[0] < n_seqs:
        raise TypeError(f"block_table must be [>= {n_seqs}, max_blocks]")
    return Shape(n_seqs=n_seqs, n_q_heads=q.shape[-2], n_kv_heads=hkv, head_dim=hd, block_size=bs,
                 n_pool_blocks=nb, max_blocks_per_seq=block_table.shape[1], q_fmt=_fmt_of(q),
                 k_fmt=_fmt_of(k_pool), v_fmt=_fmt_of(v_pool), scale=scale, flags=flags,
                 split_tokens=split_tokens)


def _sized(t, name: str, numel: int, dtype=None):
    """t (if given) is a contiguous tensor of at least `numel` elements of
    `dtype`: the kernels index it up to there from the call's sizes."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements; the call reads or writes {numel}")


def _window_args(mode: str, window):
    m = MODES[mode]
    if m == WIN_CAUSAL:
        return m, 1, None
    if window is None:
        raise ValueError(f"mode {mode} needs a window tensor")
    _i32(window, "window")
    n_runs = window.shape[1] if m == WIN_KV_MAP else 1
    return m, n_runs, window


def _workspace(nbytes: int, like, workspace):
    torch = _torch()
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=like.device)


# ---------------------------------------------------------------------------
# attention


def decode_workspace_bytes(shape: Shape, mode: str = "causal", n_runs: int = 1) -> int:
    return int(lib().pkv_decode_workspace_bytes(ctypes.byref(shape), MODES[mode], n_runs))


def decode_split_tokens(shape: Shape, mode: str = "causal", n_runs: int = 1) -> int:
    return int(lib().pkv_decode_split_tokens(ctypes.byref(shape), MODES[mode], n_runs))


def paged_attn_decode(q, k_pool, v_pool, block_table, seq_lens, scale: float, mode: str = "causal",
                      window=None, out=None, lse=None, workspace=None, flags: int = 0,
                      split_tokens: int = 0, part: str = "both"):
    """Decode attention (one query per sequence) through the block table.

    q [S, Hq, hd]; pools [NB, Hkv, bs, hd] (K may be uint8 q8_0 [NB, Hkv, bs, seg]);
    block_table int32 [S, MB]; seq_lens int32 [S]; window int32 [S, 2] (span) or
    [S, n_runs, 2] (kv_map).  Returns (out float32 [S, Hq, hd], lse float32 [S, Hq]).
    part = "partials" / "merge" runs one of the two passes (same workspace)."""
    torch = _torch()
    _on_one_gpu(q, k_pool, v_pool, block_table, seq_lens, window, out, lse, workspace)
    S = q.shape[0]
    shape = make_shape(q, k_pool, v_pool, block_table, S, scale, flags, split_tokens)
    _i32(seq_lens, "seq_lens")
    m, n_runs, win = _window_args(mode, window)
    i32, f32 = torch.int32, torch.float32
    _sized(seq_lens, "seq_lens", S, i32)
    _sized(win, "window", S * n_runs * 2, i32)
    _sized(out, "out", S * shape.n_q_heads * shape.head_dim, f32)
    _sized(lse, "lse", S * shape.n_q_heads, f32)
    need = int(lib().pkv_decode_workspace_bytes(ctypes.byref(shape), m, n_runs))
    if need == 0:
        _check(lib().pkv_paged_attn_decode(ctypes.byref(shape), None, None, None, None, None, m, n_runs,
                                           None, None, None, None, 0, None))
    ws = _workspace(need, q, workspace)
    if out is None:
        out = torch.empty((S, shape.n_q_heads, shape.head_dim), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((S, shape.n_q_heads), dtype=torch.float32, device=q.device)
    st = _stream(q)
    L = lib()
    if part == "both":
        _check(L.pkv_paged_attn_decode(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                       _ptr(block_table), _ptr(seq_lens), m, n_runs, _ptr(win),
                                       _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), st))
    elif part == "partials":
        _check(L.pkv_paged_attn_decode_partials(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                                _ptr(block_table), _ptr(seq_lens), m, n_runs, _ptr(win),
                                                _ptr(ws), ws.numel(), st))
    elif part == "merge":
        _check(L.pkv_paged_attn_decode_merge(ctypes.byref(shape), _ptr(seq_lens), m, n_runs, _ptr(win),
                                             _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), st))
    else:
        raise ValueError(part)
    return out, lse


NOALLOC_SCRATCH_BYTES = 64 << 20  # PKV_NOALLOC_SCRATCH_BYTES


def paged_attn_decode_noalloc(q, k_pool, v_pool, block_table, seq_lens, scale: float, out, lse,
                              mode: str = "causal", window=None, flags: int = 0, split_tokens: int = 0):
    """pkv_paged_attn_decode_noalloc: decode with the library's built-in
    device scratch instead of a workspace (the call allocates nothing, so
    out and lse must be given).  Arguments as for paged_attn_decode."""
    torch = _torch()
    _on_one_gpu(q, k_pool, v_pool, block_table, seq_lens, window, out, lse)
    S = q.shape[0]
    shape = make_shape(q, k_pool, v_pool, block_table, S, scale, flags, split_tokens)
    _i32(seq_lens, "seq_lens")
    m, n_runs, win = _window_args(mode, window)
    i32, f32 = torch.int32, torch.float32
    _sized(seq_lens, "seq_lens", S, i32)
    _sized(win, "window", S * n_runs * 2, i32)
    _sized(out, "out", S * shape.n_q_heads * shape.head_dim, f32)
    _sized(lse, "lse", S * shape.n_q_heads, f32)
    _check(lib().pkv_paged_attn_decode_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                               _ptr(block_table), _ptr(seq_lens), m, n_runs, _ptr(win),
                                               _ptr(out), _ptr(lse), _stream(q)))
    return out, lse


def prefill_workspace_bytes(shape: Shape, n_q_total: int, max_q_per_seq: int, mode: str = "kv_map",
                            n_runs: int = 1) -> int:
    return int(lib().pkv_prefill_workspace_bytes(ctypes.byref(shape), n_q_total, max_q_per_seq,
                                                 MODES[mode], n_runs))


def paged_attn_prefill_window(q, cu_q, q_pos, k_pool, v_pool, block_table, seq_lens, scale: float,
                              max_q_per_seq: int, mode: str = "kv_map", window=None, out=None, lse=None,
                              workspace=None, flags: int = 0):
    """Windowed prefill: queries of sequence s are rows cu_q[s]..cu_q[s+1]-1 of q
    [Nq, Hq, hd] at positions q_pos [Nq].  Returns (out [Nq, Hq, hd], lse [Nq, Hq])."""
    torch = _torch()
    _on_one_gpu(q, cu_q, q_pos, k_pool, v_pool, block_table, seq_lens, window, out, lse, workspace)
    S = block_table.shape[0]
    Nq = q.shape[0]
    shape = make_shape(q, k_pool, v_pool, block_table, S, scale, flags)
    for name, t in (("cu_q", cu_q), ("q_pos", q_pos), ("seq_lens", seq_lens)):
        _i32(t, name)
    m, n_runs, win = _window_args(mode, window)
    i32, f32 = torch.int32, torch.float32
    _sized(cu_q, "cu_q", S + 1, i32)
    _sized(q_pos, "q_pos", Nq, i32)
    _sized(seq_lens, "seq_lens", S, i32)
    _sized(win, "window", S * n_runs * 2, i32)
    _sized(out, "out", Nq * shape.n_q_heads * shape.head_dim, f32)
    _sized(lse, "lse", Nq * shape.n_q_heads, f32)
    need = int(lib().pkv_prefill_workspace_bytes(ctypes.byref(shape), Nq, max_q_per_seq, m, n_runs))
    ws = _workspace(need, q, workspace) if need else workspace
    if out is None:
        out = torch.empty((Nq, shape.n_q_heads, shape.head_dim), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((Nq, shape.n_q_heads), dtype=torch.float32, device=q.device)
    _check(lib().pkv_paged_attn_prefill_window(
        ctypes.byref(shape), Nq, max_q_per_seq, _ptr(q), _ptr(cu_q), _ptr(q_pos), _ptr(k_pool), _ptr(v_pool),
        _ptr(block_table), _ptr(seq_lens), m, n_runs, _ptr(win), _ptr(out), _ptr(lse), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(q)))
    return out, lse


def resolve_rows(block_table, seq_lens, block_size: int, n_kv_heads: int, head_dim: int, n_pool_blocks: int,
                 n_cand: int, mode: str = "causal", window=None, cu_q=None, q_pos=None, n_q_heads=None,
                 k_fmt: int = F16, v_fmt: int = F16, q_fmt: int = F16):
    """Pool row read by every (query, window candidate), or -1 (debug export)."""
    torch = _torch()
    _on_one_gpu(block_table, seq_lens, window, cu_q, q_pos)
    S = block_table.shape[0]
    shape = Shape(n_seqs=S, n_q_heads=n_q_heads or n_kv_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
                  block_size=block_size, n_pool_blocks=n_pool_blocks, max_blocks_per_seq=block_table.shape[1],
                  q_fmt=q_fmt, k_fmt=k_fmt, v_fmt=v_fmt, scale=1.0, flags=0, split_tokens=0)
    m, n_runs, win = _window_args(mode, window)
    nq = S if cu_q is None else q_pos.shape[0]
    rows = torch.empty((nq, n_cand), dtype=torch.int32, device=block_table.device)
    _check(lib().pkv_resolve_rows(ctypes.byref(shape), nq, _ptr(cu_q), _ptr(q_pos), _ptr(block_table),
                                  _ptr(seq_lens), m, n_runs, _ptr(win), n_cand, _ptr(rows),
                                  _stream(block_table)))
    return rows


# ---------------------------------------------------------------------------
# moves


def order_moves(moves) -> list:
    """Application order of (src, dst, len) moves (host call)."""
    import numpy as np

    mv = np.ascontiguousarray(np.asarray(moves, dtype=np.int32).reshape(-1, 3))
    n = mv.shape[0]
    order = np.zeros(max(n, 1), dtype=np.int32)
    n_out = ctypes.c_int32(0)
    _check(lib().pkv_order_moves(mv.ctypes.data, n, order.ctypes.data, ctypes.byref(n_out)))
    return order[: n_out.value].tolist()


class CopyPlan(ctypes.Structure):
    """pkv_copy_plan: what pkv_copy_cells_plan wrote (kind 0 nothing, 1
    disjoint runs, 2 staged rows; counts; plan words)."""

    _fields_ = [("kind", ctypes.c_int32), ("n_moves", ctypes.c_int32), ("total_rows", ctypes.c_int32),
                ("n_gather", ctypes.c_int32), ("n_scatter", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("n_words", ctypes.c_int64)]


def _pool_geometry(k_pool, v_pool):
    for t in (k_pool, v_pool):
        if t is not None and (not t.is_contiguous() or t.dim() != 4):
            raise TypeError("pools must be contiguous [n_blocks, n_kv_heads, block_size, W]")
    nb, hkv, bs = k_pool.shape[:3]
    seg_k = k_pool.shape[3] * k_pool.element_size()
    seg_v = 0
    if v_pool is not None:
        if tuple(v_pool.shape[:3]) != (nb, hkv, bs):
            raise ValueError("K and V pools must agree on (n_blocks, n_kv_heads, block_size)")
        seg_v = v_pool.shape[3] * v_pool.element_size()
    return nb, hkv, bs, seg_k, seg_v


def _moves_array(moves):
    import numpy as np

    return np.ascontiguousarray(np.asarray(moves, dtype=np.int32).reshape(-1, 3))


def copy_cells_plan(moves, n_pool_rows: int, pin_memory: bool = True):
    """pkv_copy_cells_plan (host): returns (info, plan), plan a host int32
    tensor (pinned when pin_memory, so it can be uploaded asynchronously)
    whose first info.n_words words are the plan."""
    torch = _torch()
    mv = _moves_array(moves)
    n = mv.shape[0]
    words = int(lib().pkv_copy_cells_plan_words(mv.ctypes.data, n))
    plan = torch.empty(max(words, 1), dtype=torch.int32, pin_memory=pin_memory)
    info = CopyPlan()
    _check(lib().pkv_copy_cells_plan(mv.ctypes.data, n, int(n_pool_rows), plan.data_ptr(), words,
                                     ctypes.byref(info)))
    return info, plan


def copy_cells_stage_bytes(info: CopyPlan, k_pool, v_pool) -> int:
    _, hkv, _, seg_k, seg_v = _pool_geometry(k_pool, v_pool)
    return int(lib().pkv_copy_cells_stage_bytes(ctypes.byref(info), seg_k * hkv, seg_v * hkv))


def copy_cells_apply(k_pool, v_pool, info: CopyPlan, plan, stage=None):
    """pkv_copy_cells_apply (device only, capturable): plan is a device int32
    tensor holding the info.n_words words pkv_copy_cells_plan wrote; stage a
    device uint8 tensor of copy_cells_stage_bytes bytes (kind 2)."""
    torch = _torch()
    _on_one_gpu(k_pool, v_pool, plan, stage)
    nb, hkv, bs, seg_k, seg_v = _pool_geometry(k_pool, v_pool)
    _sized(plan, "plan", int(info.n_words), torch.int32)
    need = int(lib().pkv_copy_cells_stage_bytes(ctypes.byref(info), seg_k * hkv, seg_v * hkv))
    _sized(stage, "stage", need, torch.uint8)
    _check(lib().pkv_copy_cells_apply(_ptr(k_pool), _ptr(v_pool), nb, bs, hkv, seg_k, seg_v, ctypes.byref(info),
                                      _ptr(plan), _ptr(stage), 0 if stage is None else stage.numel(),
                                      _stream(k_pool)))


def kv_copy_cells(k_pool, v_pool, moves, workspace=None):
    """Apply (src, dst, len) row moves (host int32 array [n, 3]) to both pools
    in order_moves order, bit-exact.  Pools are [n_blocks, n_kv_heads,
    block_size, W]; a row is one slot of every kv head.  The plan is made on
    the host into pinned memory, copied to the device asynchronously on the
    current stream (the front of `workspace`, a device uint8 tensor, when
    given) and applied there; nothing waits for the device."""
    torch = _torch()
    _on_one_gpu(k_pool, v_pool, workspace)
    nb, hkv, bs, seg_k, seg_v = _pool_geometry(k_pool, v_pool)
    info, plan_h = copy_cells_plan(moves, nb * bs)
    if info.kind == 0:
        return k_pool, v_pool
    words = int(info.n_words)
    plan_bytes = (words * 4 + 255) // 256 * 256
    stage_bytes = int(lib().pkv_copy_cells_stage_bytes(ctypes.byref(info), seg_k * hkv, seg_v * hkv))
    if workspace is None:
        workspace = torch.empty(plan_bytes + max(stage_bytes, 256), dtype=torch.uint8, device=k_pool.device)
    _sized(workspace, "workspace", plan_bytes + stage_bytes, torch.uint8)
    plan_d = workspace[: words * 4].view(torch.int32)
    plan_d.copy_(plan_h[:words], non_blocking=True)
    stage = workspace[plan_bytes:]
    _check(lib().pkv_copy_cells_apply(_ptr(k_pool), _ptr(v_pool), nb, bs, hkv, seg_k, seg_v, ctypes.byref(info),
                                      _ptr(plan_d), _ptr(stage), stage.numel(), _stream(k_pool)))
    return k_pool, v_pool


def copy_cells_workspace_bytes(moves, k_pool, v_pool) -> int:
    """pkv_copy_cells_workspace_bytes: an upper bound on what kv_copy_cells
    (or pkv_kv_copy_cells) needs for these moves."""
    mv = _moves_array(moves)
    _, hkv, _, seg_k, seg_v = _pool_geometry(k_pool, v_pool)
    return int(lib().pkv_copy_cells_workspace_bytes(mv.ctypes.data, mv.shape[0], seg_k * hkv, seg_v * hkv))


# ---------------------------------------------------------------------------
# store


def kv_store(k_new, v_new, positions, k_pool, v_pool, block_table, seq_ids=None, skipped=None):
    """Write token t's rows k_new[t], v_new[t] ([n_tok, n_kv_heads, head_dim],
    float32 or float16) into pool row table[s][p // bs] * bs + p % bs of each
    pool (s = seq_ids[t], or t when seq_ids is None; p = positions[t]),
    converted to the pool's format (q8_0 through the store quantizer).
    v_new and v_pool may both be None.  Tokens without a destination are
    left out and counted into ``skipped`` (a device int32 tensor of one
    element, cleared by the caller) when it is given."""
    torch = _torch()
    _on_one_gpu(k_new, v_new, positions, k_pool, v_pool, block_table, seq_ids, skipped)
    if k_new.dtype not in (torch.float32, torch.float16):
        raise TypeError("k_new must be float32 or float16")
    if (v_new is None) != (v_pool is None):
        raise ValueError("v_new and v_pool go together")
    for name, t in (("k_new", k_new), ("v_new", v_new), ("k_pool", k_pool), ("v_pool", v_pool)):
        if t is not None and not t.is_contiguous():
            raise TypeError(f"{name} must be contiguous")
    if v_new is not None and (v_new.dtype != k_new.dtype or v_new.shape != k_new.shape):
        raise TypeError("v_new must match k_new in dtype and shape")
    if k_new.dim() != 3 or k_pool.dim() != 4:
        raise TypeError("k_new is [n_tok, n_kv_heads, head_dim]; pools are [n_blocks, n_kv_heads, block_size, W]")
    n_tok, hkv, hd = k_new.shape
    _sized(positions, "positions", n_tok, torch.int32)
    _sized(seq_ids, "seq_ids", n_tok, torch.int32)
    _sized(skipped, "skipped", 1, torch.int32)
    nb, phkv, bs = k_pool.shape[:3]
    if phkv != hkv:
        raise ValueError("k_new and k_pool disagree on n_kv_heads")
    if v_pool is not None and tuple(v_pool.shape[:3]) != (nb, hkv, bs):
        raise ValueError("K and V pools must agree on (n_blocks, n_kv_heads, block_size)")
    _i32(block_table, "block_table")
    _i32(positions, "positions")
    if positions.numel() != n_tok:
        raise ValueError("positions must have one entry per token")
    if seq_ids is not None:
        _i32(seq_ids, "seq_ids")
        if seq_ids.numel() != n_tok:
            raise ValueError("seq_ids must have one entry per token")
    if skipped is not None:
        _i32(skipped, "skipped")
    kf = _fmt_of(k_pool)
    vf = _fmt_of(v_pool) if v_pool is not None else F16
    for fmt, pool in ((kf, k_pool), (vf, v_pool)):
        if pool is None:
            continue
        if pool.shape[3] * pool.element_size() != row_bytes(fmt, 1, hd):
            raise ValueError(f"pool width {pool.shape[3]} does not hold head_dim {hd} in its format")
    sh = Shape(n_seqs=block_table.shape[0], n_q_heads=hkv, n_kv_heads=hkv, head_dim=hd, block_size=bs,
               n_pool_blocks=nb, max_blocks_per_seq=block_table.shape[1], q_fmt=F32, k_fmt=kf, v_fmt=vf,
               scale=1.0, flags=0, split_tokens=0)
    src = F32 if k_new.dtype == torch.float32 else F16
    _check(lib().pkv_kv_store(ctypes.byref(sh), n_tok, src, _ptr(k_new), _ptr(v_new), _ptr(seq_ids),
                              _ptr(positions), _ptr(block_table), _ptr(k_pool), _ptr(v_pool), _ptr(skipped),
                              _stream(k_pool)))
    return k_pool, v_pool


# ---------------------------------------------------------------------------
# copy-on-write block pool


class BlockPool:
    """Host block pool with reference counts (the library's pkv_block_pool):
    fork shares blocks, prepare_writes makes the blocks a write touches
    private and returns the block copies that must run first."""

    def __init__(self, n_blocks: int, n_seqs: int, max_blocks_per_seq: int, block_size: int, watermark: int = 0):
        self._h = ctypes.c_void_p()
        _check(lib().pkv_pool_create(n_blocks, n_seqs, max_blocks_per_seq, block_size, watermark,
                                     ctypes.byref(self._h)))
        self.n_blocks, self.n_seqs, self.max_blocks, self.block_size = n_blocks, n_seqs, max_blocks_per_seq, block_size

    def close(self):
        if self._h:
            lib().pkv_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass

    def free_blocks(self) -> int:
        return int(lib().pkv_pool_free_blocks(self._h))

    def can_allocate(self, n: int) -> bool:
        return bool(lib().pkv_pool_can_allocate(self._h, n))

    def refcount(self, block: int) -> int:
        return int(lib().pkv_pool_refcount(self._h, block))

    def seq_len(self, seq: int) -> int:
        return int(lib().pkv_pool_seq_len(self._h, seq))

    def fork(self, src: int, dst: int, n_tokens: int = -1):
        _check(lib().pkv_pool_fork(self._h, src, dst, n_tokens))

    def remove(self, seq: int, p0: int, p1: int):
        _check(lib().pkv_pool_remove(self._h, seq, p0, p1))

    def prepare_writes(self, seqs, p0s, counts):
        """Host int32 arrays; returns the ops int32 numpy array [n, 3] =
        (block to copy or -1, new block, table entry index), one per table
        entry the writes change, for cow_apply."""
        import numpy as np

        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        p0s = np.ascontiguousarray(p0s, dtype=np.int32)
        counts = np.ascontiguousarray(counts, dtype=np.int32)
        n = len(seqs)
        if len(p0s) != n or len(counts) != n:
            raise ValueError("seqs, p0s and counts must have equal lengths")
        # a write of c tokens touches at most c // bs + 2 logical blocks
        cap = 2 * n + int(counts.sum(dtype=np.int64)) // self.block_size + 1 if n else 1
        cap = max(cap, 1)
        if getattr(self, "_ops", None) is None or self._ops.shape[0] < cap:
            self._ops = np.zeros((cap, 3), dtype=np.int32)
            self._nc = ctypes.c_int32(0)
        _check(lib().pkv_pool_prepare_writes(self._h, n, seqs.ctypes.data, p0s.ctypes.data, counts.ctypes.data,
                                             self._ops.ctypes.data, cap, ctypes.byref(self._nc)))
        return self._ops[: self._nc.value].copy()

    def defrag(self, need: int = -1):
        """Free the top `need` block ids (need < 0: every free block) by
        moving the live blocks there into the lowest free blocks; returns
        the row moves int32 [n, 3] (src_row, dst_row, len) for kv_copy_cells.
        The pool's tables already follow; re-export them to the device."""
        import numpy as np

        cap = max(1, self.n_blocks - self.free_blocks())
        out = np.zeros((cap, 3), dtype=np.int32)
        nm = ctypes.c_int32(0)
        _check(lib().pkv_pool_defrag(self._h, need, out.ctypes.data, cap, ctypes.byref(nm)))
        return out[: nm.value].copy()

    def export(self):
        """(table int32 [n_seqs, max_blocks], lengths int32 [n_seqs]) on the host."""
        import numpy as np

        table = np.zeros((self.n_seqs, self.max_blocks), dtype=np.int32)
        lens = np.zeros(self.n_seqs, dtype=np.int32)
        _check(lib().pkv_pool_export(self._h, table.ctypes.data, lens.ctypes.data))
        return table, lens


def cow_apply(k_pool, v_pool, ops, table=None):
    """Apply BlockPool.prepare_writes ops on the device: copy each op's
    source block (if any) to its new block in both pools and, if a device
    table is given (int32 [n_seqs, max_blocks]), patch its entries.  ops is
    a device int32 tensor [n, 3] or a host array (uploaded first)."""
    torch = _torch()
    _on_one_gpu(k_pool, v_pool, table, ops if isinstance(ops, torch.Tensor) else None)
    if not isinstance(ops, torch.Tensor):
        import numpy as np

        ops = torch.from_numpy(np.ascontiguousarray(ops, dtype=np.int32).reshape(-1, 3)).to(k_pool.device)
    _i32(ops, "ops")
    for t in (k_pool, v_pool):
        if t is not None and not t.is_contiguous():
            raise TypeError("pools must be contiguous")
    if table is not None:
        _i32(table, "table")
    nb = k_pool.shape[0]
    if v_pool is not None and v_pool.shape[0] != nb:
        raise ValueError("K and V pools must have the same number of blocks")
    kb = k_pool[0].numel() * k_pool.element_size()
    vb = v_pool[0].numel() * v_pool.element_size() if v_pool is not None else 0
    _check(lib().pkv_cow_apply(_ptr(k_pool), _ptr(v_pool), nb, kb, vb, _ptr(ops), ops.shape[0], _ptr(table),
                               table.numel() if table is not None else 0, _stream(k_pool)))
    return k_pool, v_pool


# ---------------------------------------------------------------------------
# int4 cold-block codec


def int4_blob_bytes(n_elts: int) -> int:
    return int(lib().pkv_int4_blob_bytes(n_elts))


def _int4_geometry(pool):
    if pool.dtype not in (_torch().float16, _torch().float32) or not pool.is_contiguous():
        raise TypeError("the int4 codec works on contiguous float16 or float32 pools")
    return pool.shape[0], pool[0].numel(), _fmt_of(pool)


def int4_encode(pool, blocks, blobs=None):
    """Encode pool blocks (device int32 ids [n]) into blobs [n, stride]
    (uint8, stride = blob bytes rounded up to 16; allocated if not given)."""
    torch = _torch()
    _on_one_gpu(pool, blocks, blobs)
    _i32(blocks, "blocks")
    nb, elems, fmt = _int4_geometry(pool)
    n = blocks.numel()
    if blobs is None:
        stride = (int4_blob_bytes(elems) + 15) // 16 * 16
        blobs = torch.zeros((n, stride), dtype=torch.uint8, device=pool.device)
    if blobs.dim() != 2 or blobs.shape[0] != n or not blobs.is_contiguous():
        raise TypeError("blobs must be a contiguous [n, stride] uint8 tensor")
    _check(lib().pkv_int4_encode(_ptr(pool), fmt, nb, elems, _ptr(blocks), n, _ptr(blobs), blobs.shape[1],
                                 _stream(pool)))
    return blobs


def int4_decode(blobs, pool, blocks):
    """Decode blobs [n, stride] into the listed pool blocks (device int32 [n])."""
    _on_one_gpu(blobs, pool, blocks)
    _i32(blocks, "blocks")
    nb, elems, fmt = _int4_geometry(pool)
    n = blocks.numel()
    if blobs.dim() != 2 or blobs.shape[0] != n or not blobs.is_contiguous():
        raise TypeError("blobs must be a contiguous [n, stride] uint8 tensor")
    _check(lib().pkv_int4_decode(_ptr(blobs), blobs.shape[1], n, _ptr(pool), fmt, nb, elems, _ptr(blocks),
                                 _stream(pool)))
    return pool
