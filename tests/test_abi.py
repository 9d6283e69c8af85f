"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and its host-only logic (row widths, order_moves, workspace sizes,
validation before any launch) is right.  No kernel runs here."""

import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

import oracle
import paged_kv_cache_table_amd as pkv
from workloads import gen as wgen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")

pytestmark = pytest.mark.skipif(not os.path.exists(pkv.LIB_PATH), reason="libpkv.so not built")


def declared_functions():
    src = open(os.path.join(ROOT, "include", "pkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(pkv.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = pkv.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH], capture_output=True, text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared_functions():
        assert name in syms, name
    assert pkv.version().startswith("pkv")


def test_row_bytes_golden():
    with open(os.path.join(GOLDEN, "q8_0_row_bytes.json")) as f:
        for c in json.load(f)["cases"]:
            assert pkv.row_bytes(pkv.Q8_0, c["n_kv_heads"], c["head_dim"]) == c["row_bytes"]
            assert pkv.row_bytes(pkv.Q8_0, 1, c["head_dim"]) == c["segment_bytes"]
    assert pkv.row_bytes(pkv.F16, 8, 128) == 2048
    assert pkv.row_bytes(pkv.F32, 2, 64) == 512
    assert pkv.row_bytes(pkv.Q8_0, 1, 48) == 0
    assert pkv.row_bytes(7, 1, 64) == 0


def test_order_moves_golden_and_random():
    with open(os.path.join(GOLDEN, "order_moves_worked.json")) as f:
        g = json.load(f)
    assert pkv.order_moves(g["moves"]) == g["order"]
    rng = np.random.default_rng(3)
    for _ in range(300):
        n = int(rng.integers(0, 40))
        mv = np.stack([rng.integers(0, 30, n), rng.integers(0, 30, n), rng.integers(-1, 6, n)], 1)
        assert pkv.order_moves(mv) == oracle.order_moves(mv)
    ms = wgen.make_moves(seed=55, n_moves=10000)
    assert pkv.order_moves(ms.moves) == oracle.order_moves(ms.moves)
    for _ in range(200):  # negative rows (order_moves takes any int32) and runs of equal keys
        n = int(rng.integers(1, 50))
        mv = np.stack([rng.integers(-4, 4, n), rng.integers(-4, 4, n), rng.integers(-1, 3, n)], 1)
        assert pkv.order_moves(mv) == oracle.order_moves(mv)


def _shape(**kw):
    base = dict(n_seqs=2, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16, n_pool_blocks=64,
                max_blocks_per_seq=16, q_fmt=pkv.F16, k_fmt=pkv.F16, v_fmt=pkv.F16, scale=0.1, flags=0,
                split_tokens=0)
    base.update(kw)
    return pkv.Shape(**base)


def test_dispatch_table_golden():
    with open(os.path.join(GOLDEN, "dispatch_tuples.json")) as f:
        g = json.load(f)
    L = pkv.lib()
    for hd, bs in g["supported_head_block"]:
        sh = _shape(head_dim=hd, block_size=bs)
        assert L.pkv_decode_workspace_bytes(ctypes.byref(sh), 0, 1) > 0, (hd, bs)
    for hd, bs in g["refused_head_block"]:
        sh = _shape(head_dim=hd, block_size=bs)
        assert L.pkv_decode_workspace_bytes(ctypes.byref(sh), 0, 1) == 0, (hd, bs)


FAKE = 0x10000  # never dereferenced: every case below is refused before any launch


def _decode(sh, mode=0, n_runs=1, window=FAKE, ws=FAKE, ws_bytes=1 << 40):
    return pkv.lib().pkv_paged_attn_decode(ctypes.byref(sh), FAKE, FAKE, FAKE, FAKE, FAKE, mode, n_runs,
                                           window, FAKE, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(head_dim=96), 2, "(96, 16)"),
    (dict(block_size=32, head_dim=64), 2, "(64, 32)"),
    (dict(n_q_heads=10, n_kv_heads=2), 2, "group 5"),
    (dict(n_q_heads=9, n_kv_heads=2), 1, "multiple"),
    (dict(k_fmt=7), 1, "unknown KV format"),
    (dict(q_fmt=pkv.F32, k_fmt=pkv.F16, v_fmt=pkv.F16), 2, "(f32, f16, f16)"),
    (dict(v_fmt=pkv.Q8_0), 2, "(f16, f16, q8_0)"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(n_pool_blocks=0), 1, "n_pool_blocks"),
    (dict(split_tokens=24), 1, "split_tokens"),
])
def test_refusals_name_the_problem(kw, status, needle):
    st = _decode(_shape(**kw))
    assert st == status
    assert needle in pkv.last_error()


def test_window_and_workspace_refusals():
    sh = _shape()
    assert _decode(sh, mode=2, n_runs=9) == 1 and "runs" in pkv.last_error()
    assert _decode(sh, mode=1, window=None) == 1 and "window" in pkv.last_error()
    assert _decode(sh, mode=5) == 1
    need = pkv.decode_workspace_bytes(sh)
    assert _decode(sh, ws_bytes=need - 1) == 3 and str(need) in pkv.last_error()
    assert _decode(sh, ws=None) == 3
    assert _decode(sh, ws=FAKE + 8, ws_bytes=need) == 3 and "aligned" in pkv.last_error()


def test_decode_workspace_size_formula():
    sh = _shape(n_seqs=64, n_q_heads=32, n_kv_heads=8, max_blocks_per_seq=2048, split_tokens=512)
    assert pkv.decode_split_tokens(_shape(n_seqs=64, n_q_heads=32, n_kv_heads=8, max_blocks_per_seq=2048)) == 1024
    # the largest split that still gives >= 6144 possible items: 32 x 3 x 8192 / 128
    assert pkv.decode_split_tokens(_shape(n_seqs=32, n_q_heads=9, n_kv_heads=3, head_dim=64, max_blocks_per_seq=512)) == 128
    def up(x):
        return (x + 255) // 256 * 256

    def need(runs):
        # partial rows: one per split slot, plus the extra pieces of the cut
        # slots (a planned call: 64 x 64 slots x 8 kv heads > 8192 units;
        # 512-position splits -> 2 pieces of 256; cut slots per sequence =
        # ceil(4096 / (2 pieces x 8 kv heads x 64 seqs)) = 4, capped at 2);
        # then the work list (16 bytes per item, at most one per row), 16
        # bytes per sequence for its places in the list, the unit count and
        # the error word
        nspl = 2048 * 16 // 512
        rows = 64 * nspl * runs + 64 * 2 * (2 - 1)
        return up(rows * 32 * 128 * 4) + up(rows * 32 * 2 * 4) + up(rows * 16) + up(64 * 16) + 256 + 256

    assert pkv.decode_workspace_bytes(sh) == need(1)
    assert pkv.decode_workspace_bytes(sh, "kv_map", 4) == need(4)
    # a call with at most 8192 units (4 x 32 slots x 8 kv heads here) skips
    # the plan and cuts nothing: one row per slot
    small = _shape(n_seqs=4, n_q_heads=32, n_kv_heads=8, max_blocks_per_seq=2048, split_tokens=1024)
    rows = 4 * 32
    assert pkv.decode_workspace_bytes(small) == up(rows * 32 * 128 * 4) + up(rows * 32 * 2 * 4) + up(rows * 16) + up(4 * 16) + 512


def test_copy_cells_refuses_out_of_range_moves():
    L = pkv.lib()
    mv = np.array([[0, 5, 3], [10, 98, 4]], dtype=np.int32)
    # 25 blocks x 4 slots = 100 rows, 2 kv heads of 32-byte segments
    st = L.pkv_kv_copy_cells(FAKE, FAKE, 25, 4, 2, 32, 32, mv.ctypes.data, 2, FAKE, 1 << 30, None)
    assert st == 1 and "move 1" in pkv.last_error()
    st = L.pkv_kv_copy_cells(FAKE, FAKE, 25, 4, 2, 30, 32, mv.ctypes.data, 1, FAKE, 1 << 30, None)
    assert st == 1 and "seg_bytes_k" in pkv.last_error()
    st = L.pkv_kv_copy_cells(FAKE, FAKE, 25, 0, 2, 32, 32, mv.ctypes.data, 1, FAKE, 1 << 30, None)
    assert st == 1 and "block_size" in pkv.last_error()
    # no effective move: nothing to do, nothing touched
    mv0 = np.array([[3, 3, 5], [1, 9, 0]], dtype=np.int32)
    assert L.pkv_kv_copy_cells(FAKE, FAKE, 25, 4, 2, 32, 32, mv0.ctypes.data, 2, None, 0, None) == 0


def test_copy_cells_workspace_bound():
    ms = wgen.make_moves(seed=55, n_moves=1000)
    L = pkv.lib()
    need = L.pkv_copy_cells_workspace_bytes(ms.moves.ctypes.data, 1000, 4096, 4096)
    rows = int(ms.moves[ms.moves[:, 0] != ms.moves[:, 1], 2].sum())
    assert need >= rows * 2 * 4096


def test_resolve_refusals():
    L = pkv.lib()
    sh = _shape()
    st = L.pkv_resolve_rows(ctypes.byref(sh), 3, None, None, FAKE, FAKE, 0, 1, None, 10, FAKE, None)
    assert st == 1 and "n_q_total == n_seqs" in pkv.last_error()
    st = L.pkv_resolve_rows(ctypes.byref(sh), 2, FAKE, None, FAKE, FAKE, 0, 1, None, 10, FAKE, None)
    assert st == 1


def test_copy_cells_workspace_for_disjoint_moves_is_small():
    """Moves whose destinations touch no source need no stage: the workspace
    holds only the moves and their prefix sums."""
    import ctypes

    mv = np.array([[0, 100, 10], [200, 20, 30], [50, 300, 5]], dtype=np.int32)
    small = pkv.lib().pkv_copy_cells_workspace_bytes(mv.ctypes.data, 3, 4096, 4096)
    assert small <= 512
    overlapping = np.array([[0, 5, 10], [200, 20, 30]], dtype=np.int32)  # 0..9 -> 5..14 overlaps itself
    big = pkv.lib().pkv_copy_cells_workspace_bytes(overlapping.ctypes.data, 2, 4096, 4096)
    assert big >= 40 * 4096


def _disjoint_brute(mv):
    """No destination row is written twice and no destination row is read."""
    dst, src = [], []
    for a, b, n in mv.tolist():
        if n <= 0 or a == b:
            continue
        dst += range(b, b + n)
        src += range(a, a + n)
    return len(dst) == len(set(dst)) and not (set(dst) & set(src))


def test_copy_cells_disjoint_check():
    """The workspace is the small one exactly when the moves are disjoint,
    for dense and sparse move sets (some disjoint by construction), checked
    against a row-by-row brute force."""
    rng = np.random.default_rng(9)
    seen = {True: 0, False: 0}
    for t in range(400):
        n = int(rng.integers(1, 12))
        span = 200 if t % 2 else 1 << 22  # dense, then sparse over a wide row range
        mv = np.stack([rng.integers(0, span, n), rng.integers(0, span, n), rng.integers(-1, 9, n)], 1)
        if t % 4 == 1:  # disjoint by construction: destinations above every source
            mv[:, 1] = span + 16 * np.arange(n)
            mv[:, 2] = np.clip(mv[:, 2], 0, 16)
        mv = mv.astype(np.int32)
        m = int(np.sum((mv[:, 2] > 0) & (mv[:, 0] != mv[:, 1])))
        small_bound = (3 * m + m + 1) * 4 // 256 * 256 + 512
        ws = pkv.lib().pkv_copy_cells_workspace_bytes(mv.ctypes.data, n, 4096, 4096)
        want = _disjoint_brute(mv)
        assert (ws <= small_bound) == want or m == 0, (t, mv.tolist(), ws)
        seen[want] += 1
    assert seen[True] > 50 and seen[False] > 50


def test_binding_refuses_host_tensors():
    """Tensors that are not on a GPU are refused before anything reaches
    the library (a kernel handed a host pointer would fault)."""
    import torch

    q = torch.zeros((2, 8, 128), dtype=torch.float16)
    k = torch.zeros((4, 2, 16, 128), dtype=torch.float16)
    table = torch.zeros((2, 4), dtype=torch.int32)
    lens = torch.ones(2, dtype=torch.int32)
    with pytest.raises(TypeError, match="GPU"):
        pkv.paged_attn_decode(q, k, k, table, lens, 0.1)
    with pytest.raises(TypeError, match="GPU"):
        pkv.kv_copy_cells(k, k, np.array([[0, 16, 4]], dtype=np.int32))
    with pytest.raises(TypeError, match="GPU"):
        pkv.kv_store(torch.zeros((1, 2, 128)), torch.zeros((1, 2, 128)), torch.zeros(1, dtype=torch.int32),
                     k.float(), k.float(), table)
    with pytest.raises(TypeError, match="GPU"):
        pkv.int4_encode(k, torch.zeros(1, dtype=torch.int32))
    with pytest.raises(TypeError, match="GPU"):
        pkv.cow_apply(k, k, np.zeros((1, 3), dtype=np.int32), table)
    with pytest.raises(TypeError, match="GPU"):
        pkv.paged_attn_prefill_window(q, torch.tensor([0, 1, 2], dtype=torch.int32), torch.zeros(2, dtype=torch.int32),
                                      k, k, table, lens, 0.1, 1, mode="causal")
