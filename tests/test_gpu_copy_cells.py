"""copy_cells on the GPU: bit-exact against the oracle's sequential memmoves."""

import json
import os

import numpy as np
import pytest

import oracle
import paged_kv_cache_table_amd as pkv
from workloads import gen as wgen

from gpu_util import log

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_pool(rng, blocks, hkv, bs, width, dtype):
    import torch

    a = rng.integers(0, 256, size=(blocks, hkv, bs, width), dtype=np.uint8)
    t = torch.from_numpy(a)
    if dtype != "u8":
        t = t.view(getattr(torch, dtype))
    return t


def test_golden_example_on_gpu():
    import torch

    with open(os.path.join(GOLDEN, "order_moves_worked.json")) as f:
        g = json.load(f)
    # 30 rows = 15 blocks of 2 slots, 3 kv heads: every segment holds its row id
    ids = torch.arange(g["n_rows"], dtype=torch.int32).reshape(15, 1, 2, 1).repeat(1, 3, 1, 4)
    k = ids.clone().cuda()
    v = (ids * 3).clone().cuda()
    pkv.kv_copy_cells(k, v, g["moves"])
    for h in range(3):
        assert k[:, h, :, 0].reshape(-1).cpu().tolist() == g["final_rows"]
        assert (v[:, h, :, 1] // 3).reshape(-1).cpu().tolist() == g["final_rows"]


@pytest.mark.parametrize("seed", range(6))
def test_random_moves_bit_exact(seed):
    import torch

    rng = np.random.default_rng(seed)
    blocks, bs = 64, 16
    n_rows = blocks * bs
    kh = _rand_pool(rng, blocks, 4, bs, 512 if seed % 2 else 136, "u8")
    vh = _rand_pool(rng, blocks, 4, bs, 256, "float16" if seed % 3 else "u8")
    ms = wgen.make_moves(seed=seed, n_moves=200 + 100 * seed, n_rows=n_rows, region=n_rows // 2,
                         max_len=16 + seed)
    k, v = kh.cuda(), vh.cuda()
    ref = [kh.numpy().copy(), vh.numpy().copy()]
    oracle.copy_cells(ref, ms.moves)
    pkv.kv_copy_cells(k, v, ms.moves)
    assert np.array_equal(k.cpu().numpy().view(np.uint8), ref[0].view(np.uint8))
    assert np.array_equal(v.cpu().numpy().view(np.uint8), ref[1].view(np.uint8))


def test_single_pool_and_narrow_rows():
    import torch

    rng = np.random.default_rng(5)
    kh = _rand_pool(rng, 10, 3, 16, 12, "u8")  # 12-byte segments: 4-byte copies
    ms = wgen.make_moves(seed=5, n_moves=300, n_rows=160, region=150, max_len=9)
    ref = [kh.numpy().copy()]
    oracle.copy_cells(ref, ms.moves)
    k = kh.cuda()
    pkv.kv_copy_cells(k, None, ms.moves)
    assert np.array_equal(k.cpu().numpy(), ref[0])


def test_refused_moves_leave_pools_untouched():
    import torch

    k = torch.arange(64 * 16, dtype=torch.float32, device="cuda").reshape(64, 1, 16, 1)
    before = k.clone()
    with pytest.raises(pkv.PkvError):
        pkv.kv_copy_cells(k, None, [[0, 10, 4], [1020, 5, 8]])
    assert torch.equal(k, before)


def _pattern(rows, heads, width_words, salt):
    """int32 words that are a function of (row, kv head, column) only:
    [len(rows), heads, width_words]."""
    import torch

    r = rows.long()[:, None, None]
    h = torch.arange(heads, dtype=torch.int64, device=rows.device)[None, :, None]
    c = torch.arange(width_words, dtype=torch.int64, device=rows.device)[None, None, :]
    x = (r * 0x9E3779B1 + h * 0x27D4EB2F + c * 0x85EBCA77 + salt) & 0xFFFFFFFF
    return (x - (x >= 2 ** 31).long() * 2 ** 32).to(torch.int32)


def _fill(pool, salt, chunk_blocks=4096):
    import torch

    nb, hkv, bs, width = pool.shape
    for b0 in range(0, nb, chunk_blocks):
        b1 = min(nb, b0 + chunk_blocks)
        rows = torch.arange(b0 * bs, b1 * bs, device=pool.device)
        pool[b0:b1] = _pattern(rows, hkv, width, salt).reshape(b1 - b0, bs, hkv, width).permute(0, 2, 1, 3)


def _check(pool, prov, salt, chunk_blocks=4096):
    nb, hkv, bs, width = pool.shape
    for b0 in range(0, nb, chunk_blocks):
        b1 = min(nb, b0 + chunk_blocks)
        exp = _pattern(prov[b0 * bs : b1 * bs], hkv, width, salt).reshape(b1 - b0, bs, hkv, width)
        assert bool((pool[b0:b1] == exp.permute(0, 2, 1, 3)).all()), f"blocks {b0}.."


def test_full_size_10k_overlapping_moves():
    """10,000 random overlapping row moves on K and V pools of 2^17 blocks x
    16 slots x 8 kv heads x 512 bytes (2^21 rows of 4096 bytes), every
    segment holding a pattern of its own row and kv head: afterwards each row
    must hold the pattern of the row the oracle's provenance names."""
    import torch

    w = wgen.make(5)
    ms = wgen.make_moves(seed=55)
    n_rows = w.n_pool_blocks * w.block_size
    assert n_rows == ms.n_rows
    width = w.head_dim * 2 // 4
    log(f"copy_cells: {len(ms.moves)} moves on 2 x {n_rows} rows x {w.row_bytes('k')} B")
    k = torch.empty((w.n_pool_blocks, w.n_kv_heads, w.block_size, width), dtype=torch.int32, device="cuda")
    v = torch.empty_like(k)
    _fill(k, 1)
    _fill(v, 2)
    pkv.kv_copy_cells(k, v, ms.moves)
    prov = torch.from_numpy(oracle.provenance(n_rows, ms.moves)).cuda()
    changed = int((prov != torch.arange(n_rows, device="cuda")).sum())
    log(f"  {changed} rows changed")
    _check(k, prov, 1)
    _check(v, prov, 2)


def _disjoint_moves(rng, n_moves, n_rows, max_len):
    """Random moves whose destinations overlap neither each other nor any
    source: 2 * n_moves disjoint intervals, each length used twice, each
    pair split into a source and a destination in random direction."""
    lens = rng.integers(1, max_len + 1, size=n_moves)
    slots = rng.permutation(np.repeat(np.arange(n_moves), 2))
    gaps = rng.integers(0, 3, size=2 * n_moves)
    assert int(lens.sum()) * 2 + int(gaps.sum()) <= n_rows
    starts, pos = {}, 0
    for k, m in enumerate(slots):
        pos += int(gaps[k])
        starts.setdefault(int(m), []).append(pos)
        pos += int(lens[m])
    moves = []
    for m in range(n_moves):
        a, b = starts[m]
        if rng.random() < 0.5:
            a, b = b, a
        moves.append((a, b, int(lens[m])))
    return np.array(moves, dtype=np.int32)


@pytest.mark.parametrize("seed", range(4))
def test_disjoint_moves_bit_exact(seed):
    """Move sets where no destination touches a source take the one-pass
    run copy; bytes must equal the oracle's sequential memmoves."""
    rng = np.random.default_rng(300 + seed)
    blocks, bs = 64, [16, 7, 32, 1][seed]
    n_rows = blocks * bs
    kh = _rand_pool(rng, blocks, 3, bs, [512, 68, 136, 36][seed], "u8")
    vh = _rand_pool(rng, blocks, 3, bs, 256, "float16")
    max_len = max(1, min(32, n_rows // 64))
    moves = _disjoint_moves(rng, max(4, n_rows // (4 * max_len + 8)), n_rows, max_len)
    k, v = kh.cuda(), vh.cuda()
    ref = [kh.numpy().copy(), vh.numpy().copy()]
    oracle.copy_cells(ref, moves)
    pkv.kv_copy_cells(k, v, moves)
    assert np.array_equal(k.cpu().numpy().view(np.uint8), ref[0].view(np.uint8))
    assert np.array_equal(v.cpu().numpy().view(np.uint8), ref[1].view(np.uint8))


def test_back_to_back_calls_without_synchronizing():
    """Five move sets applied by five calls with no synchronize in between
    (overlapping and disjoint sets, so both device paths run): each plan is
    uploaded asynchronously from pinned memory that torch's host allocator
    keeps until its copy has run, so a plan buffer reused too early would
    show here.  Bit-exact against the oracle applying the sets in turn."""
    import torch

    rng = np.random.default_rng(90)
    blocks, bs = 128, 16
    n_rows = blocks * bs
    kh = _rand_pool(rng, blocks, 4, bs, 256, "u8")
    vh = _rand_pool(rng, blocks, 4, bs, 128, "float16")
    k, v = kh.cuda(), vh.cuda()
    ref = [kh.numpy().copy(), vh.numpy().copy()]
    sets = []
    for i in range(5):
        if i % 2:
            sets.append(_disjoint_moves(rng, 40 + 10 * i, n_rows, 12))  # <= 2 x 70 x 12 + 140 rows
        else:
            sets.append(wgen.make_moves(seed=200 + i, n_moves=300 + 50 * i, n_rows=n_rows,
                                        region=n_rows // 2, max_len=20).moves)
    for mv in sets:
        oracle.copy_cells(ref, mv)
        pkv.kv_copy_cells(k, v, mv)
    torch.cuda.synchronize()
    assert np.array_equal(k.cpu().numpy().view(np.uint8), ref[0].view(np.uint8))
    assert np.array_equal(v.cpu().numpy().view(np.uint8), ref[1].view(np.uint8))


def test_concurrent_calls_from_two_threads():
    """Two host threads apply their own move sets to their own pools at the
    same time (each on its own stream); the host plan holds no state, so the
    threads share nothing.  Each pool bit-exact against the oracle."""
    import threading

    import torch

    rng = np.random.default_rng(91)
    blocks, bs = 96, 16
    n_rows = blocks * bs
    jobs = []
    for j in range(2):
        kh = _rand_pool(rng, blocks, 2, bs, 512, "u8")
        vh = _rand_pool(rng, blocks, 2, bs, 256, "u8")
        mvs = [wgen.make_moves(seed=300 + 10 * j + i, n_moves=250, n_rows=n_rows, region=n_rows // 2,
                               max_len=16).moves for i in range(4)]
        ref = [kh.numpy().copy(), vh.numpy().copy()]
        for mv in mvs:
            oracle.copy_cells(ref, mv)
        jobs.append({"k": kh.cuda(), "v": vh.cuda(), "moves": mvs, "ref": ref, "err": None})
    torch.cuda.synchronize()

    def run(job):
        try:
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                for mv in job["moves"]:
                    pkv.kv_copy_cells(job["k"], job["v"], mv)
            st.synchronize()
        except Exception as e:  # reported by the main thread
            job["err"] = e

    threads = [threading.Thread(target=run, args=(job,)) for job in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    for job in jobs:
        assert job["err"] is None, job["err"]
        assert np.array_equal(job["k"].cpu().numpy(), job["ref"][0])
        assert np.array_equal(job["v"].cpu().numpy(), job["ref"][1])


@pytest.mark.parametrize("kind", ["staged rows", "disjoint runs"])
def test_apply_captured_in_a_graph(kind):
    """pkv_copy_cells_apply launches kernels only, so it is captured into a
    HIP graph once (plan made and uploaded before the capture) and every
    replay moves the rows again: after replay i the pools equal the oracle
    applying the moves i times.  Eager work and synchronizations run
    between the replays."""
    import torch

    rng = np.random.default_rng(95 if kind == "staged rows" else 96)
    blocks, bs = 96, 16
    n_rows = blocks * bs
    kh = _rand_pool(rng, blocks, 4, bs, 256, "u8")
    vh = _rand_pool(rng, blocks, 4, bs, 128, "float16")
    if kind == "staged rows":
        mv = wgen.make_moves(seed=97, n_moves=300, n_rows=n_rows, region=n_rows // 2, max_len=16).moves
    else:
        mv = _disjoint_moves(rng, 50, n_rows, 12)
    k, v = kh.cuda(), vh.cuda()
    info, plan_h = pkv.copy_cells_plan(mv, n_rows)
    assert info.kind == (2 if kind == "staged rows" else 1)
    plan_d = plan_h[: info.n_words].cuda()
    stage = torch.empty(max(pkv.copy_cells_stage_bytes(info, k, v), 256), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pkv.copy_cells_apply(k, v, info, plan_d, stage)
    torch.cuda.synchronize()
    # capturing does not run the kernels: the pools are unchanged
    assert np.array_equal(k.cpu().numpy(), kh.numpy())
    ref = [kh.numpy().copy(), vh.numpy().copy()]
    junk = torch.zeros(1 << 20, device="cuda")
    for i in range(3):
        g.replay()
        junk.add_(1.0)  # eager work between replays
        torch.cuda.synchronize()
        oracle.copy_cells(ref, mv)
        assert np.array_equal(k.cpu().numpy().view(np.uint8), ref[0].view(np.uint8)), f"replay {i}"
        assert np.array_equal(v.cpu().numpy().view(np.uint8), ref[1].view(np.uint8)), f"replay {i}"
    log(f"  {kind}: {info.n_words} plan words, three replays bit-exact")


def test_one_call_c_entry_point():
    """pkv_kv_copy_cells (plan, upload and apply in one C call, through
    ctypes) gives the oracle's bytes for an overlapping and a disjoint set."""
    import ctypes

    import torch

    rng = np.random.default_rng(98)
    blocks, bs, hkv = 64, 16, 2
    n_rows = blocks * bs
    kh = _rand_pool(rng, blocks, hkv, bs, 136, "u8")
    vh = _rand_pool(rng, blocks, hkv, bs, 64, "float16")
    k, v = kh.cuda(), vh.cuda()
    ref = [kh.numpy().copy(), vh.numpy().copy()]
    L = pkv.lib()
    for mv in (wgen.make_moves(seed=99, n_moves=200, n_rows=n_rows, region=n_rows // 2, max_len=16).moves,
               _disjoint_moves(rng, 30, n_rows, 8)):
        mv = np.ascontiguousarray(mv.astype(np.int32))
        oracle.copy_cells(ref, mv)
        # K segments are 136 bytes, V segments 64 bytes (32 halves)
        need = L.pkv_copy_cells_workspace_bytes(mv.ctypes.data, mv.shape[0], 136 * hkv, 64 * hkv)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        st = L.pkv_kv_copy_cells(k.data_ptr(), v.data_ptr(), blocks, bs, hkv, 136, 64, mv.ctypes.data,
                                 mv.shape[0], ws.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
        assert st == 0, pkv.last_error()
    torch.cuda.synchronize()
    assert np.array_equal(k.cpu().numpy(), ref[0])
    assert np.array_equal(v.cpu().numpy().view(np.uint8), ref[1].view(np.uint8))
