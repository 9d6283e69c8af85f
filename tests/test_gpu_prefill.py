"""Windowed prefill (matrix-core path) on the GPU against the CPU oracle.

Tolerance: max-abs 2e-3 on out and lse for f16 / q8_0 inputs with f32
accumulation (P is rounded to f16 before the PV product, as the
matrix-core contraction takes f16 operands)."""

import numpy as np
import pytest

import paged_kv_cache_table_amd as pkv
from workloads import gen as wgen

from gpu_util import Dev, compare, log, tol_of

pytestmark = pytest.mark.gpu


def _run(w, **kw):
    d = Dev(w)
    out, lse = d.prefill(**kw)
    ro, rl = d.oracle()
    return d, out.cpu().numpy(), lse.cpu().numpy(), ro, rl


@pytest.mark.parametrize("mode", [None, "span", "kv_map_only"])
def test_prefill_workload4_small(mode):
    w = wgen.make(4, small=True, mode=mode)
    log(f"prefill workload 4 small ({w.mode}, {w.n_seqs} seqs, {w.n_queries} queries)")
    d, out, lse, ro, rl = _run(w)
    compare(out, lse, ro, rl, tol_of(w), f"w4 {w.mode}")


@pytest.mark.parametrize("hd,bs", [(64, 16), (128, 16), (256, 16), (128, 32)])
@pytest.mark.parametrize("g", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("kfmt", ["f16", "q8_0"])
def test_prefill_dispatch_tuples(hd, bs, g, kfmt):
    w = wgen.make_custom(seed=hd + bs + 10 * g + (kfmt == "q8_0"), n_seqs=3, n_q_heads=2 * g, n_kv_heads=2,
                         head_dim=hd, block_size=bs, fmts=("f16", kfmt, "f16"), ctx=(1, 150), kind="prefill",
                         q_per_seq=(1, 40), mode="causal")
    log(f"prefill hd {hd} bs {bs} g {g} K {kfmt}")
    d, out, lse, ro, rl = _run(w)
    compare(out, lse, ro, rl, tol_of(w), f"hd{hd} bs{bs} g{g} {kfmt}")


@pytest.mark.parametrize("mode", ["causal", "span", "kv_map"])
@pytest.mark.parametrize("kfmt", ["f16", "q8_0"])
def test_prefill_windows(mode, kfmt):
    w = wgen.make_custom(seed=77, n_seqs=7, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=32,
                         fmts=("f16", kfmt, "f16"), ctx=(1, 600), mode=mode, n_runs=5, kind="prefill",
                         q_per_seq=(1, 90), hole_frac=0.1)
    log(f"prefill window {mode} K {kfmt}: {w.n_queries} queries")
    d, out, lse, ro, rl = _run(w)
    compare(out, lse, ro, rl, tol_of(w), f"{mode} {kfmt}")


def test_prefill_degenerate():
    import torch

    w = wgen.make_custom(seed=21, n_seqs=5, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                         ctx=(20, 120), mode="span", kind="prefill", q_per_seq=(1, 10), hole_frac=0.0)
    w.window[0] = (5, 5)                        # empty window: every query sees nothing
    w.window[1] = (-50, 10 ** 6)                # clipped to [0, seq_len)
    w.block_table[2, :] = -1                    # all holes
    w.window[3] = (int(w.seq_lens[3]) - 1, int(w.seq_lens[3]))  # only the last position
    d = Dev(w)
    out, lse = d.prefill()
    ro, rl = d.oracle()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for s in (0, 2):
        rows = slice(w.cu_q[s], w.cu_q[s + 1])
        assert np.all(o[rows] == 0) and np.all(np.isneginf(l[rows]))
    compare(o, l, ro, rl, tol_of(w), "degenerate")


def test_prefill_rows_past_max_q_are_untouched():
    import torch

    w = wgen.make_custom(seed=22, n_seqs=3, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                         ctx=(60, 120), kind="prefill", q_per_seq=(20, 30), hole_frac=0.0)
    d = Dev(w)
    out = torch.full((w.n_queries, 8, 128), 7.0, device="cuda")
    lse = torch.full((w.n_queries, 8), 7.0, device="cuda")
    pkv.paged_attn_prefill_window(d.q, d.cu_q, d.q_pos, d.k, d.v, d.table, d.lens, w.scale, 10,
                                  mode="causal", out=out, lse=lse)
    ro, rl = d.oracle()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for s in range(w.n_seqs):
        a, b = int(w.cu_q[s]), int(w.cu_q[s + 1])
        compare(o[a : a + 10], l[a : a + 10], ro[a : a + 10], rl[a : a + 10], tol_of(w), f"seq {s} first 10")
        assert np.all(o[a + 10 : b] == 7.0) and np.all(l[a + 10 : b] == 7.0)


@pytest.mark.parametrize("hd,bs", [(64, 16), (128, 16), (256, 16), (128, 32)])
@pytest.mark.parametrize("kfmt", ["f32", "q8_0"])
@pytest.mark.parametrize("g", [1, 4, 8])
def test_prefill_f32_formats(hd, bs, kfmt, g):
    """f32 queries with f32 or q8_0 K and f32 V: every product and sum in
    f32, held to 1e-5 against the oracle."""
    w = wgen.make_custom(seed=hd + bs + 7 * g + (kfmt == "q8_0"), n_seqs=4, n_q_heads=2 * g, n_kv_heads=2,
                         head_dim=hd, block_size=bs, fmts=("f32", kfmt, "f32"), ctx=(1, 300), kind="prefill",
                         q_per_seq=(1, 40), mode="causal", hole_frac=0.05)
    log(f"f32 prefill hd {hd} bs {bs} g {g} K {kfmt}")
    d, out, lse, ro, rl = _run(w)
    compare(out, lse, ro, rl, 1e-5, f"f32 hd{hd} bs{bs} g{g} {kfmt}")


@pytest.mark.parametrize("mode", ["span", "kv_map"])
@pytest.mark.parametrize("kfmt", ["f32", "q8_0"])
def test_prefill_f32_windows_and_degenerate(mode, kfmt):
    w = wgen.make_custom(seed=55, n_seqs=6, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=32,
                         fmts=("f32", kfmt, "f32"), ctx=(1, 500), mode=mode, n_runs=5, kind="prefill",
                         q_per_seq=(1, 50), hole_frac=0.1)
    if mode == "span":
        w.window[0] = (5, 5)  # empty window
    else:
        w.kv_map[0] = 0       # no runs
    w.block_table[1, :] = -1  # all holes
    d, out, lse, ro, rl = _run(w)
    for s in (0, 1):
        rows = slice(w.cu_q[s], w.cu_q[s + 1])
        assert np.all(out[rows] == 0) and np.all(np.isneginf(lse[rows]))
    compare(out, lse, ro, rl, 1e-5, f"f32 {mode} {kfmt}")


def test_prefill_f32_rows_past_max_q_are_untouched():
    import torch

    w = wgen.make_custom(seed=56, n_seqs=3, n_q_heads=8, n_kv_heads=2, head_dim=64, block_size=16,
                         fmts=("f32", "f32", "f32"), ctx=(60, 120), kind="prefill", q_per_seq=(20, 30),
                         hole_frac=0.0)
    d = Dev(w)
    out = torch.full((w.n_queries, 8, 64), 7.0, device="cuda")
    lse = torch.full((w.n_queries, 8), 7.0, device="cuda")
    pkv.paged_attn_prefill_window(d.q, d.cu_q, d.q_pos, d.k, d.v, d.table, d.lens, w.scale, 10,
                                  mode="causal", out=out, lse=lse)
    ro, rl = d.oracle()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for s in range(w.n_seqs):
        a, b = int(w.cu_q[s]), int(w.cu_q[s + 1])
        compare(o[a : a + 10], l[a : a + 10], ro[a : a + 10], rl[a : a + 10], 1e-5, f"f32 seq {s} first 10")
        assert np.all(o[a + 10 : b] == 7.0) and np.all(l[a + 10 : b] == 7.0)


def test_prefill_matches_decode_for_last_queries():
    """A prefill query at position seq_len - 1 sees what decode sees."""
    w = wgen.make_custom(seed=24, n_seqs=6, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
                         ctx=(100, 900), kind="prefill", q_per_seq=(1, 1), hole_frac=0.05)
    w.q_pos = (w.seq_lens - 1).astype(np.int32)
    d = Dev(w)
    po, pl = d.prefill()
    import paged_kv_cache_table_amd as p2

    do, dl = p2.paged_attn_decode(d.q, d.k, d.v, d.table, d.lens, w.scale)
    err = float((po - do).abs().max())
    log(f"  prefill vs decode at the last position: {err:.3g}")
    assert err <= 2e-3


def test_prefill_workload4_full_size():
    import torch

    w = wgen.make(4)
    log(f"full-size prefill workload 4: {w.n_seqs} seqs x 64 queries, kv_map mode")
    d = Dev(w, gen_on_gpu=True)
    out, lse = d.prefill()
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    seqs = list(range(w.n_seqs))  # every sequence: the span half and the multi-run half
    ro, rl, rows = d.oracle(seqs)
    compare(o[rows], l[rows], ro, rl, tol_of(w), "w4 full size")


def test_prefill_more_sequences_than_the_order_sort_holds():
    """4,100 short sequences: more than the order kernel sorts (4,096), so
    the sequences keep their own order; results still match the oracle, and
    decode over the same batch does too."""
    w = wgen.make_custom(seed=41, n_seqs=4100, n_q_heads=4, n_kv_heads=2, head_dim=64, block_size=16,
                         ctx=(1, 40), mode="kv_map", n_runs=2, kind="prefill", q_per_seq=(1, 3), hole_frac=0.0)
    d = Dev(w)
    out, lse = d.prefill()
    ro, rl = d.oracle()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_of(w), "4100 seqs prefill")
    w.kind, w.cu_q, w.q_pos = "decode", None, None
    d = Dev(w)
    out, lse = d.decode()
    ro, rl = d.oracle()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_of(w), "4100 seqs decode")


def test_prefill_hundred_sequences():
    """100 sequences of mixed lengths, sorted longest first by the order
    kernel before the prefill workgroups pick them up; results match the
    oracle."""
    w = wgen.make_custom(seed=43, n_seqs=100, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                         fmts=("f16", "q8_0", "f16"), ctx=(1, 300), mode="kv_map", n_runs=3, kind="prefill",
                         q_per_seq=(1, 8), hole_frac=0.05)
    log(f"prefill 100 seqs: {w.n_queries} queries")
    d, out, lse, ro, rl = _run(w)
    compare(out, lse, ro, rl, tol_of(w), "100 seqs")


def test_prefill_chunk_merge_is_deterministic():
    """Two long sequences x 8 kv heads: each window is cut into many chunks
    whose workgroups finish in no fixed order; the merge kernel combines the
    chunks in chunk order, so repeated calls give the same bits, and match
    the oracle."""
    import torch

    w = wgen.make_custom(seed=31, n_seqs=2, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=32,
                         fmts=("f16", "q8_0", "f16"), ctx=(3000, 6000), mode="kv_map", n_runs=4, kind="prefill",
                         q_per_seq=(40, 64), hole_frac=0.02)
    d = Dev(w)
    outs = [d.prefill() for _ in range(3)]
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])
    ro, rl = d.oracle()
    compare(outs[0][0].cpu().numpy(), outs[0][1].cpu().numpy(), ro, rl, tol_of(w), "many chunks")
