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


def _rand_pool(rng, blocks, bs, width, dtype):
    import torch

    a = rng.integers(0, 256, size=(blocks, bs, width), dtype=np.uint8)
    t = torch.from_numpy(a)
    if dtype != "u8":
        t = t.view(getattr(torch, dtype))
    return t


def test_golden_example_on_gpu():
    import torch

    with open(os.path.join(GOLDEN, "order_moves_worked.json")) as f:
        g = json.load(f)
    ids = torch.arange(g["n_rows"], dtype=torch.int32).reshape(g["n_rows"], 1, 1).repeat(1, 1, 4)
    k = ids.clone().cuda()
    v = (ids * 3).clone().cuda()
    pkv.kv_copy_cells(k, v, g["moves"])
    assert k[:, 0, 0].cpu().tolist() == g["final_rows"]
    assert (v[:, 0, 0] // 3).cpu().tolist() == g["final_rows"]


@pytest.mark.parametrize("seed", range(6))
def test_random_moves_bit_exact(seed):
    import torch

    rng = np.random.default_rng(seed)
    blocks, bs = 64, 16
    n_rows = blocks * bs
    kh = _rand_pool(rng, blocks, bs, 2048 if seed % 2 else 1088, "u8")
    vh = _rand_pool(rng, blocks, bs, 1024, "float16" if seed % 3 else "u8")
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
    kh = _rand_pool(rng, 10, 16, 12, "u8")  # 12-byte rows: 4-byte copies
    ms = wgen.make_moves(seed=5, n_moves=300, n_rows=160, region=150, max_len=9)
    ref = [kh.numpy().copy()]
    oracle.copy_cells(ref, ms.moves)
    k = kh.cuda()
    pkv.kv_copy_cells(k, None, ms.moves)
    assert np.array_equal(k.cpu().numpy(), ref[0])


def test_refused_moves_leave_pools_untouched():
    import torch

    k = torch.arange(64 * 16, dtype=torch.float32, device="cuda").reshape(64, 16, 1)
    before = k.clone()
    with pytest.raises(pkv.PkvError):
        pkv.kv_copy_cells(k, None, [[0, 10, 4], [1020, 5, 8]])
    assert torch.equal(k, before)


def _row_pattern(n_rows, width_words, device, salt, chunk=1 << 17):
    """int32 rows whose words are a function of (row, column) only."""
    import torch

    out = torch.empty((n_rows, width_words), dtype=torch.int32, device=device)
    c = torch.arange(width_words, dtype=torch.int64, device=device)[None, :]
    for r0 in range(0, n_rows, chunk):
        r = torch.arange(r0, min(n_rows, r0 + chunk), dtype=torch.int64, device=device)[:, None]
        x = (r * 0x9E3779B1 + c * 0x85EBCA77 + salt) & 0xFFFFFFFF
        out[r0 : r0 + r.shape[0]] = (x - (x >= 2 ** 31).long() * 2 ** 32).to(torch.int32)
    return out


def _check_rows(t, prov, salt, chunk=1 << 17):
    n_rows, width = t.shape
    for r0 in range(0, n_rows, chunk):
        p = prov[r0 : r0 + chunk]
        exp = _row_pattern_rows(p, width, salt)
        assert bool((t[r0 : r0 + chunk] == exp).all()), f"rows {r0}.."


def _row_pattern_rows(rows, width_words, salt):
    import torch

    c = torch.arange(width_words, dtype=torch.int64, device=rows.device)[None, :]
    x = (rows.long()[:, None] * 0x9E3779B1 + c * 0x85EBCA77 + salt) & 0xFFFFFFFF
    return (x - (x >= 2 ** 31).long() * 2 ** 32).to(torch.int32)


def test_full_size_10k_overlapping_moves():
    """10,000 random overlapping row moves on two pools of 2^21 rows x 4096
    bytes, every row holding a pattern of its own index: afterwards each row
    must hold the pattern of the row the oracle's provenance names."""
    import torch

    w = wgen.make(5)
    ms = wgen.make_moves(seed=55)
    n_rows = w.n_pool_blocks * w.block_size
    assert n_rows == ms.n_rows
    width = w.row_bytes("k") // 4
    log(f"copy_cells: {len(ms.moves)} moves on 2 x {n_rows} rows x {width * 4} B")
    k = _row_pattern(n_rows, width, "cuda", 1)
    v = _row_pattern(n_rows, width, "cuda", 2)
    pkv.kv_copy_cells(k.view(w.n_pool_blocks, w.block_size, width), v.view(w.n_pool_blocks, w.block_size, width),
                      ms.moves)
    prov = torch.from_numpy(oracle.provenance(n_rows, ms.moves)).cuda()
    changed = int((prov != torch.arange(n_rows, device="cuda")).sum())
    log(f"  {changed} rows changed")
    for t, salt in ((k, 1), (v, 2)):
        _check_rows(t, prov, salt)
