"""KV store with the q8_0 quantizer on the GPU: bit-exact against the oracle.

Every case fills the pools with random bytes first, so the comparison of
the whole pools also checks that no byte outside the named rows changed."""

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
NP_DT = {"f32": np.float32, "f16": np.float16, "q8_0": np.uint8}


def _rand_pool(rng, st, fmt):
    width_bytes = oracle.seg_bytes(fmt, st.head_dim)
    raw = rng.integers(0, 256, size=(st.n_pool_blocks, st.n_kv_heads, st.block_size, width_bytes), dtype=np.uint8)
    return raw.view(NP_DT[fmt])


def _run(st, k_new, v_new, with_v=True, seq_ids=True, seed=0):
    """Store on the GPU and in the oracle from the same bytes; returns
    (gpu K, gpu V, skipped), (oracle K, oracle V, skipped)."""
    import torch

    rng = np.random.default_rng(seed)
    kp = _rand_pool(rng, st, st.k_fmt)
    vp = _rand_pool(rng, st, st.v_fmt) if with_v else None
    dk = torch.from_numpy(kp.copy()).cuda()
    dv = torch.from_numpy(vp.copy()).cuda() if with_v else None
    skipped = torch.zeros(1, dtype=torch.int32, device="cuda")
    table = torch.from_numpy(st.block_table).cuda()
    pos = torch.from_numpy(st.pos).cuda()
    sid = torch.from_numpy(st.seq_ids).cuda() if seq_ids else None
    pkv.kv_store(k_new.cuda(), v_new.cuda() if with_v else None, pos, dk, dv, table, seq_ids=sid,
                 skipped=skipped)
    torch.cuda.synchronize()
    ids = st.seq_ids if seq_ids else np.arange(st.n_tok, dtype=np.int32)
    rk, rv, rs = oracle.store_rows(kp, vp, st.k_fmt, st.v_fmt, k_new.float().numpy(),
                                   v_new.float().numpy() if with_v else None, ids, st.pos, st.block_table)
    got_v = dv.cpu().numpy() if with_v else None
    return (dk.cpu().numpy(), got_v, int(skipped.item())), (rk, rv, rs)


def _same_bytes(a, b):
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def _check(got, ref, what):
    (gk, gv, gs), (rk, rv, rs) = got, ref
    assert gs == rs, f"{what}: skipped {gs} != {rs}"
    assert _same_bytes(gk, rk), f"{what}: K pool differs in {np.count_nonzero(gk.view(np.uint8) != rk.view(np.uint8))} bytes"
    if rv is not None:
        assert _same_bytes(gv, rv), f"{what}: V pool differs in {np.count_nonzero(gv.view(np.uint8) != rv.view(np.uint8))} bytes"


@pytest.mark.parametrize("hd", [32, 64, 128, 256])
@pytest.mark.parametrize("src", ["f32", "f16"])
@pytest.mark.parametrize("kfmt,vfmt", [("q8_0", "f16"), ("q8_0", "f32"), ("f16", "f16"), ("f32", "f32"),
                                       ("f16", "q8_0"), ("q8_0", "q8_0")])
def test_store_formats_bit_exact(hd, src, kfmt, vfmt):
    st = wgen.make_store(seed=hd + len(kfmt) * 7 + (src == "f32"), n_seqs=6, n_kv_heads=3, head_dim=hd,
                         block_size=16, n_pool_blocks=80, max_blocks=9, tok=(1, 70), src_fmt=src,
                         k_fmt=kfmt, v_fmt=vfmt)
    log(f"store hd {hd} src {src} K {kfmt} V {vfmt}: {st.n_tok} tokens")
    k, v = wgen.store_values(st)
    _check(*_run(st, k, v), f"hd{hd} {src} {kfmt}/{vfmt}")


@pytest.mark.parametrize("bs", [1, 5, 16, 32])
def test_store_block_sizes_and_ragged_counts(bs):
    st = wgen.make_store(seed=40 + bs, n_seqs=9, n_kv_heads=8, head_dim=128, block_size=bs,
                         n_pool_blocks=9 * (200 // bs + 2), max_blocks=200 // bs + 2, tok=(1, 190),
                         src_fmt="f16", k_fmt="q8_0", v_fmt="f16")
    log(f"store bs {bs}: {st.n_tok} tokens")
    k, v = wgen.store_values(st)
    _check(*_run(st, k, v), f"bs {bs}")


def test_store_skips_tokens_without_a_row():
    st = wgen.make_store(seed=5, n_seqs=8, n_kv_heads=2, head_dim=64, block_size=16, n_pool_blocks=120,
                         max_blocks=12, tok=(20, 100), src_fmt="f32", k_fmt="q8_0", v_fmt="f16", hole_frac=0.2)
    st.block_table[1, 3] = 120          # past the pool
    st.block_table[2, 0] = -7           # negative, not the sentinel
    n = st.n_tok
    st.seq_ids[n // 5] = 8              # sequence past n_seqs
    st.seq_ids[n // 4] = -1
    st.pos[n // 3] = -3                 # negative position
    st.pos[n // 2] = 12 * 16            # past the table
    log(f"store with holes and bad destinations: {n} tokens")
    k, v = wgen.store_values(st)
    got, ref = _run(st, k, v)
    assert ref[2] > 4
    _check(got, ref, "skips")


def test_store_decode_append_without_seq_ids():
    """One token per sequence at its current length (token t = sequence t)."""
    rng = np.random.default_rng(8)
    st = wgen.make_store(seed=8, n_seqs=64, n_kv_heads=8, head_dim=128, block_size=16, n_pool_blocks=64 * 40,
                         max_blocks=40, tok=(1, 1), src_fmt="f16", k_fmt="q8_0", v_fmt="f16", shuffle=False)
    st.pos = rng.integers(0, 40 * 16, size=64).astype(np.int32)
    log("store: decode append, 64 sequences")
    k, v = wgen.store_values(st)
    _check(*_run(st, k, v, seq_ids=False), "append")


def test_store_k_only():
    st = wgen.make_store(seed=9, n_seqs=4, n_kv_heads=4, head_dim=256, block_size=16, n_pool_blocks=40,
                         max_blocks=8, tok=(30, 100), src_fmt="f32", k_fmt="q8_0", v_fmt="f16")
    k, v = wgen.store_values(st)
    _check(*_run(st, k, v, with_v=False), "K only")


def _edge_rows(st):
    """Source rows whose q8_0 blocks are the hand-worked blocks, blocks on
    and beside code ties, tiny magnitudes (subnormal and flushed f16
    scales, binary32 subnormal inputs) and zeros."""
    import torch

    with open(os.path.join(GOLDEN, "q8_0_store_worked.json")) as f:
        cases = json.load(f)["cases"]
    worked = []
    for c in cases:
        x = np.zeros(32, dtype=np.float32)
        for i, val in c["x"].items():
            x[int(i)] = np.float32(float.fromhex(val))
        worked.append(x)
    rng = np.random.default_rng(77)
    blocks = list(worked)
    for _ in range(200):  # code ties: (k + 1/2) d, one binary32 step either side
        amax = np.float32(rng.uniform(0.05, 4.0))
        d = np.float32(amax / np.float32(127))
        x = ((rng.integers(-126, 126, size=32) + 0.5) * np.float64(d)).astype(np.float32)
        step = rng.integers(-1, 2, size=32)
        x = np.where(step > 0, np.nextafter(x, np.float32(np.inf)),
                     np.where(step < 0, np.nextafter(x, np.float32(-np.inf)), x)).astype(np.float32)
        x[0] = amax
        blocks.append(x)
    for e in range(-40, -14):  # scales from normal down through subnormal f16 and zero
        blocks.append((rng.standard_normal(32) * 2.0 ** e).astype(np.float32))
    blocks.append((rng.standard_normal(32) * 1e-41).astype(np.float32))  # binary32 subnormals
    blocks.append(np.zeros(32, dtype=np.float32))
    flat = np.concatenate(blocks)
    per_tok = st.n_kv_heads * st.head_dim
    need = st.n_tok * per_tok
    flat = np.resize(flat, need).astype(np.float32)
    return torch.from_numpy(flat.reshape(st.n_tok, st.n_kv_heads, st.head_dim).copy())


def test_store_quantizer_edge_values():
    st = wgen.make_store(seed=12, n_seqs=10, n_kv_heads=2, head_dim=128, block_size=16, n_pool_blocks=200,
                         max_blocks=20, tok=(5, 30), src_fmt="f32", k_fmt="q8_0", v_fmt="q8_0")
    k = _edge_rows(st)
    v = k.flip(0).contiguous()
    log(f"store quantizer edge values: {st.n_tok} tokens")
    _check(*_run(st, k, v), "edge values")


def test_store_empty_and_refusals():
    import torch

    st = wgen.make_store(seed=13, n_seqs=2, n_kv_heads=2, head_dim=64, block_size=16, n_pool_blocks=10,
                         max_blocks=4, tok=(3, 9), src_fmt="f16", k_fmt="q8_0", v_fmt="f16")
    k, v = wgen.store_values(st)
    kp = torch.full((10, 2, 16, 68), 7, dtype=torch.uint8, device="cuda")
    vp = torch.full((10, 2, 16, 64), 7.0, dtype=torch.float16, device="cuda")
    table = torch.from_numpy(st.block_table).cuda()
    # zero tokens: nothing written
    pkv.kv_store(k[:0].cuda(), v[:0].cuda(), torch.zeros(0, dtype=torch.int32, device="cuda"), kp, vp, table,
                 seq_ids=torch.zeros(0, dtype=torch.int32, device="cuda"))
    # head_dim 96 is outside the store's dispatch
    k96 = torch.zeros((3, 2, 96), dtype=torch.float16, device="cuda")
    kp96 = torch.zeros((10, 2, 16, 104), dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PkvError) as ei:
        pkv.kv_store(k96, None, torch.zeros(3, dtype=torch.int32, device="cuda"), kp96, None, table)
    assert ei.value.status == 2 and "head_dim" in ei.value.message
    # more tokens than sequences without seq_ids
    with pytest.raises(pkv.PkvError) as ei:
        pkv.kv_store(k.cuda(), v.cuda(), torch.from_numpy(st.pos).cuda(), kp, vp, table)
    assert ei.value.status == 1
    torch.cuda.synchronize()
    assert torch.all(kp == 7) and torch.all(vp == 7.0)


def test_store_then_decode_reads_the_stored_rows():
    """Fill workload-2-like pools through the store from f32 rows, then run
    decode attention on them: pools equal the oracle's store bit for bit and
    attention matches the oracle on those pools."""
    import torch

    w = wgen.make_custom(seed=31, n_seqs=6, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                         fmts=("f16", "q8_0", "f16"), ctx=(30, 400), hole_frac=0.1)
    st = wgen.store_of_workload(w, src_fmt="f32")
    k_new, v_new = wgen.store_values(st)
    got, ref = _run(st, k_new, v_new)
    _check(got, ref, "store of a decode workload")
    gk, gv = torch.from_numpy(got[0]).cuda(), torch.from_numpy(got[1]).cuda()
    q = torch.randn((w.n_seqs, 8, 128), generator=torch.Generator().manual_seed(3)).half()
    out, lse = pkv.paged_attn_decode(q.cuda(), gk, gv, torch.from_numpy(w.block_table).cuda(),
                                     torch.from_numpy(w.seq_lens.astype(np.int32)).cuda(), w.scale)
    ro, rl = oracle.paged_decode(q.numpy(), ref[0], ref[1], "q8_0", "f16", w.block_table, w.seq_lens,
                                 16, 2, 128, w.scale)
    err = float(np.abs(out.cpu().numpy() - ro).max())
    log(f"  decode over stored pools: max-abs {err:.3g}")
    assert err <= 2e-3
    assert np.abs(lse.cpu().numpy() - rl).max() <= 2e-3


def test_store_workload4_full_size_sampled():
    """The bench's store: every position of the 16 windowed-prefill
    sequences (f16 rows into the q8_0 K and f16 V pools).  Sampled tokens
    are checked bit for bit against the oracle's encoding; the pool bytes
    of a sample of unreferenced blocks must keep their fill."""
    import torch

    w = wgen.make(4)
    st = wgen.store_of_workload(w, src_fmt="f16")
    log(f"full-size store: {st.n_tok} tokens into {st.n_pool_blocks} blocks")
    k_new, v_new = wgen.store_values(st, "cuda")
    kp = torch.full((st.n_pool_blocks, 8, 32, 136), 0xA5, dtype=torch.uint8, device="cuda")
    vp = torch.full((st.n_pool_blocks, 8, 32, 128), 3.0, dtype=torch.float16, device="cuda")
    skipped = torch.zeros(1, dtype=torch.int32, device="cuda")
    pkv.kv_store(k_new, v_new, torch.from_numpy(st.pos).cuda(), kp, vp, torch.from_numpy(st.block_table).cuda(),
                 seq_ids=torch.from_numpy(st.seq_ids).cuda(), skipped=skipped)
    torch.cuda.synchronize()
    assert int(skipped.item()) == 0
    rng = np.random.default_rng(4)
    toks = np.sort(rng.choice(st.n_tok, size=2000, replace=False))
    rows = oracle.destination_rows(st.seq_ids[toks], st.pos[toks], st.block_table, st.n_pool_blocks, 32)
    assert np.all(rows >= 0)
    kx = k_new[torch.from_numpy(toks).cuda()].float().cpu().numpy()
    vx = v_new[torch.from_numpy(toks).cuda()].float().cpu().numpy()
    blk = torch.from_numpy(rows // 32).cuda()
    slot = torch.from_numpy(rows % 32).cuda()
    got_k = kp[blk, :, slot].cpu().numpy()
    got_v = vp[blk, :, slot].cpu().numpy()
    assert np.array_equal(got_k, oracle.encode_rows(kx, "q8_0"))
    assert np.array_equal(got_v.view(np.uint16), oracle.encode_rows(vx, "f16").view(np.uint16))
    used = np.zeros(st.n_pool_blocks, dtype=bool)
    used[st.block_table[st.block_table >= 0]] = True
    free = np.nonzero(~used)[0][:64]
    if len(free):
        fb = torch.from_numpy(free).cuda()
        assert torch.all(kp[fb] == 0xA5) and torch.all(vp[fb] == 3.0)
