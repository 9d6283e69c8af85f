"""Paged decode on the GPU against the CPU oracle (through the C ABI).

Tolerances (from the stated acceptance bar): max-abs 1e-5 for f32 inputs,
2e-3 for f16 / q8_0 inputs with f32 accumulation; block-table indexing and
the resolver bit-exact."""

import math

import numpy as np
import pytest

import oracle
import paged_kv_cache_table_amd as pkv
from workloads import gen as wgen

from gpu_util import Dev, compare, log, tol_of

pytestmark = pytest.mark.gpu


def _run(w, **kw):
    d = Dev(w)
    out, lse = d.decode(**kw)
    ro, rl = d.oracle()
    return d, out.cpu().numpy(), lse.cpu().numpy(), ro, rl


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_decode_workloads_small(cfg):
    w = wgen.make(cfg, small=True)
    log(f"decode workload {cfg} ({w.name})")
    d, out, lse, ro, rl = _run(w)
    compare(out, lse, ro, rl, tol_of(w), w.name)


@pytest.mark.parametrize("hd,bs", [(64, 16), (128, 16), (256, 16), (128, 32)])
@pytest.mark.parametrize("g", [1, 2, 3, 4, 8])
def test_decode_dispatch_tuples(hd, bs, g):
    w = wgen.make_custom(seed=hd * 100 + bs * 10 + g, n_seqs=5, n_q_heads=2 * g, n_kv_heads=2, head_dim=hd,
                         block_size=bs, ctx=(1, 5 * bs + 7))
    log(f"decode hd {hd} bs {bs} g {g}")
    d, out, lse, ro, rl = _run(w)
    compare(out, lse, ro, rl, tol_of(w), f"hd{hd} bs{bs} g{g}")


@pytest.mark.parametrize("fmts", [("f32", "f32", "f32"), ("f16", "q8_0", "f16"), ("f32", "q8_0", "f32")])
@pytest.mark.parametrize("hd,bs", [(64, 16), (128, 32), (256, 16)])
def test_decode_formats(fmts, hd, bs):
    w = wgen.make_custom(seed=7 + hd + bs, n_seqs=6, n_q_heads=8, n_kv_heads=2, head_dim=hd, block_size=bs,
                         fmts=fmts, ctx=(1, 200))
    log(f"decode formats {fmts} hd {hd} bs {bs}")
    d, out, lse, ro, rl = _run(w)
    compare(out, lse, ro, rl, tol_of(w), f"{fmts} hd{hd}")


@pytest.mark.parametrize("mode", ["span", "kv_map"])
@pytest.mark.parametrize("fmts", [("f16", "f16", "f16"), ("f16", "q8_0", "f16"), ("f32", "f32", "f32")])
def test_decode_windows(mode, fmts):
    w = wgen.make_custom(seed=31, n_seqs=12, n_q_heads=12, n_kv_heads=3, head_dim=128, block_size=16,
                         fmts=fmts, ctx=(1, 700), mode=mode, n_runs=5)
    log(f"decode window {mode} {fmts}")
    d, out, lse, ro, rl = _run(w)
    compare(out, lse, ro, rl, tol_of(w), f"{mode} {fmts}")


def test_decode_windowed_prefill_workload_as_decode():
    # workload 4's q8_0 pool and kv_map windows, read by one decode query per sequence
    w = wgen.make(4, small=True)
    w.kind, w.cu_q, w.q_pos = "decode", None, None
    log("decode on workload 4 (small) structure")
    d, out, lse, ro, rl = _run(w)
    compare(out, lse, ro, rl, tol_of(w), "w4-as-decode")


@pytest.mark.parametrize("split", [64, 128, 256, 512, 1024])
def test_decode_split_sizes(split):
    w = wgen.make_custom(seed=5, n_seqs=4, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
                         ctx=(900, 2000))
    log(f"decode split {split}")
    d, out, lse, ro, rl = _run(w, split_tokens=split)
    compare(out, lse, ro, rl, tol_of(w), f"split {split}")


@pytest.mark.parametrize("mode,fmts", [
    ("causal", ("f16", "f16", "f16")), ("causal", ("f16", "q8_0", "f16")), ("causal", ("f32", "f32", "f32")),
    ("span", ("f16", "f16", "f16")), ("span", ("f16", "q8_0", "f16")), ("span", ("f32", "f32", "f32")),
    ("kv_map", ("f16", "f16", "f16")), ("kv_map", ("f16", "q8_0", "f16")), ("kv_map", ("f32", "f32", "f32")),
    ("kv_map8", ("f16", "f16", "f16")), ("degenerate", ("f16", "f16", "f16"))])
def test_decode_cut_slots(mode, fmts):
    """A planned call (64 sequences x 32 possible 1024-position slots x 8 kv
    heads > 8192 units): the work list skips the empty slots, and each
    sequence's last two full slots are cut into four 256-position pieces
    (ceil(4096 / (4 x 8 x 64)) = 2), next to whole and partial slots, holes
    and windows; "kv_map8" uses the most runs a kv_map may have, and
    "degenerate" adds empty sequences, windows and tables.
    Against the oracle; the fused call equals partials + merge on a
    workspace full of garbage."""
    import torch

    wmode = "kv_map" if mode in ("degenerate", "kv_map8") else mode
    w = wgen.make_custom(seed=77, n_seqs=64, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
                         fmts=fmts, ctx=(1500, 6000), mode=wmode, n_runs=8 if mode == "kv_map8" else 3,
                         max_blocks=2048)
    if mode == "degenerate":
        w.seq_lens[0] = 0                 # empty sequence
        w.kv_map[1] = 0                   # no runs
        w.block_table[2, :] = -1          # all holes
        w.kv_map[3, :, 1] = -4            # negative lengths: unused runs
    log(f"decode cut slots {mode} {fmts}")
    d = Dev(w)
    n_runs = 1 if wmode != "kv_map" else w.kv_map.shape[1]
    shape = pkv.make_shape(d.q, d.k, d.v, d.table, w.n_seqs, w.scale, 0, 1024)
    ws = torch.full((pkv.decode_workspace_bytes(shape, wmode, n_runs),), 0xAB, dtype=torch.uint8, device="cuda")
    out, lse = d.decode(split_tokens=1024, workspace=ws)
    d.decode(split_tokens=1024, part="partials", workspace=ws)
    out2, lse2 = d.decode(split_tokens=1024, part="merge", workspace=ws)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    ro, rl = d.oracle()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_of(w), f"cut {mode} {fmts}")


@pytest.mark.parametrize("case", ["w3", "kv_map_holes", "degenerate"])
def test_one_call_equals_partials_then_merge(case):
    """One call equals the two-call route (partials, then merge) bit for bit,
    also on a dirty workspace, on repeat calls and on sequences with no
    visible position (out 0, lse -inf)."""
    import torch

    if case == "w3":
        w = wgen.make(3, small=True)
    else:
        w = wgen.make_custom(seed=91, n_seqs=9, n_q_heads=16, n_kv_heads=4, head_dim=128, block_size=16,
                             ctx=(0, 700), mode="kv_map", n_runs=5, hole_frac=0.2)
        if case == "degenerate":
            w.kv_map[0] = 0                 # no runs: empty window
            w.block_table[1, :] = -1        # all holes
            w.seq_lens[2] = 0               # empty sequence
    d = Dev(w)
    ws = torch.empty(pkv.decode_workspace_bytes(pkv.make_shape(d.q, d.k, d.v, d.table, w.n_seqs, w.scale),
                                                w.mode, 1 if w.mode != "kv_map" else w.kv_map.shape[1]),
                     dtype=torch.uint8, device="cuda")
    ws.fill_(0xAB)  # nothing may depend on the workspace's previous contents
    out1, lse1 = d.decode(workspace=ws)
    out1b, lse1b = d.decode(workspace=ws)
    d.decode(part="partials", workspace=ws)
    out2, lse2 = d.decode(part="merge", workspace=ws)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    assert torch.equal(out1, out1b) and torch.equal(lse1, lse1b)
    if case == "degenerate":
        assert torch.all(out1[:3] == 0) and torch.all(torch.isneginf(lse1[:3]))
    if case != "w3":
        ro, rl = d.oracle()
        compare(out1.cpu().numpy(), lse1.cpu().numpy(), ro, rl, tol_of(w), case)


def test_determinism_and_block_permutation_invariance():
    """Bitwise: the same call twice, and the same data with its blocks moved
    to other physical ids (table rewritten to follow)."""
    import torch

    w = wgen.make(2, small=True)
    d = Dev(w)
    o1, l1 = d.decode()
    o2, l2 = d.decode()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    rng = np.random.default_rng(0)
    perm = rng.permutation(w.n_pool_blocks)  # old block b -> new block perm[b]
    inv = np.argsort(perm)
    k2 = d.k[torch.from_numpy(inv).cuda()].contiguous()
    v2 = d.v[torch.from_numpy(inv).cuda()].contiguous()
    t = w.block_table
    t2 = np.where(t >= 0, perm[np.maximum(t, 0)], -1).astype(np.int32)
    o3, l3 = pkv.paged_attn_decode(d.q, k2, v2, torch.from_numpy(t2).cuda(), d.lens, w.scale)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_one_hot_row_ids():
    """One visible slot per sequence and V rows holding their own row id: the
    output is the row id exactly, so a wrong table lookup shows directly."""
    import torch

    w = wgen.make_custom(seed=9, n_seqs=40, n_q_heads=4, n_kv_heads=2, head_dim=64, block_size=16,
                         fmts=("f32", "f32", "f32"), ctx=(1, 400), hole_frac=0.0, mode="span")
    rng = np.random.default_rng(1)
    t = np.array([int(rng.integers(0, int(L))) for L in w.seq_lens])
    w.window = np.stack([t, t + 1], 1).astype(np.int32)
    d = Dev(w)
    n_rows = w.n_pool_blocks * w.block_size
    rowid = torch.arange(n_rows, dtype=torch.float32, device="cuda").reshape(w.n_pool_blocks, 1, w.block_size, 1)
    v = rowid.expand(w.n_pool_blocks, w.n_kv_heads, w.block_size, w.head_dim).contiguous()
    out, lse = pkv.paged_attn_decode(d.q, d.k, v, d.table, d.lens, w.scale, mode="span", window=d.window)
    rows = np.array([oracle.physical_row(w.block_table[s], np.array([t[s]]), w.block_size)[0]
                     for s in range(w.n_seqs)])
    got = out.cpu().numpy()
    assert np.array_equal(got, np.broadcast_to(rows[:, None, None].astype(np.float32), got.shape))


def test_resolver_bit_exact():
    import torch

    for mode in ("causal", "span", "kv_map"):
        w = wgen.make_custom(seed=3, n_seqs=9, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                             ctx=(1, 300), mode=mode, n_runs=6, kind="prefill")
        d = Dev(w)
        n_cand = w.max_blocks_per_seq * w.block_size + 5
        rows = pkv.resolve_rows(d.table, d.lens, w.block_size, w.n_kv_heads, w.head_dim, w.n_pool_blocks,
                                n_cand, mode=mode, window=d.window, cu_q=d.cu_q, q_pos=d.q_pos)
        ref = oracle.resolve_rows(mode, w.block_table, w.seq_lens, w.block_size, w.q_seq(), w.q_pos, n_cand,
                                  w.window, w.kv_map)
        assert np.array_equal(rows.cpu().numpy(), ref), mode
        # decode form: query at seq_len - 1
        rows = pkv.resolve_rows(d.table, d.lens, w.block_size, w.n_kv_heads, w.head_dim, w.n_pool_blocks,
                                n_cand, mode=mode, window=d.window)
        ref = oracle.resolve_rows(mode, w.block_table, w.seq_lens, w.block_size, np.arange(w.n_seqs),
                                  w.seq_lens - 1, n_cand, w.window, w.kv_map)
        assert np.array_equal(rows.cpu().numpy(), ref), mode
        log(f"  resolver {mode}: bit-exact over {rows.numel()} entries")


def test_degenerate_cases():
    import torch

    w = wgen.make_custom(seed=12, n_seqs=6, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                         ctx=(20, 100), mode="span", hole_frac=0.0)
    w.seq_lens[0] = 0                     # empty sequence
    w.block_table[1, :] = -1              # every block a hole
    w.window[2] = (50, 50)                # empty span
    w.window[3] = (-100, 10 ** 6)         # span far outside: clipped to [0, seq_len)
    w.window[4] = (int(w.seq_lens[4]) - 1, int(w.seq_lens[4]))  # only the last token
    d = Dev(w)
    out, lse = d.decode()
    ro, rl = d.oracle()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    for s in (0, 1, 2):
        assert np.all(o[s] == 0) and np.all(np.isneginf(l[s]))
    compare(o, l, ro, rl, tol_of(w), "degenerate")
    # no sequences at all
    e, el = pkv.paged_attn_decode(d.q[:0], d.k, d.v, d.table[:0], d.lens[:0], w.scale)
    assert e.shape == (0, 8, 128)


def test_seq_len_beyond_table_is_clamped():
    import torch

    w = wgen.make_custom(seed=13, n_seqs=3, n_q_heads=4, n_kv_heads=1, head_dim=64, block_size=16,
                         ctx=(64, 64), hole_frac=0.0, max_blocks=4)
    d = Dev(w)
    o1, l1 = d.decode()
    o2, l2 = pkv.paged_attn_decode(d.q, d.k, d.v, d.table, torch.full_like(d.lens, 10 ** 6), w.scale)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_refused_call_leaves_outputs_untouched():
    import torch

    w = wgen.make(2, small=True)
    d = Dev(w)
    out = torch.full((w.n_seqs, w.n_q_heads, w.head_dim), 7.0, device="cuda")
    lse = torch.full((w.n_seqs, w.n_q_heads), 7.0, device="cuda")
    with pytest.raises(pkv.PkvError) as ei:
        pkv.paged_attn_decode(d.q, d.k, d.v, d.table, d.lens, w.scale, out=out, lse=lse, split_tokens=24)
    assert ei.value.status == 1
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PkvError) as ei:
        pkv.paged_attn_decode(d.q, d.k, d.v, d.table, d.lens, w.scale, out=out, lse=lse, workspace=small)
    assert ei.value.status == 3
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)


def test_checked_mode_reports_bad_block_ids():
    import torch

    w = wgen.make(2, small=True)
    d = Dev(w)
    ref, rl = d.decode()
    bad = d.table.clone()
    t = w.block_table.copy()
    s, b = 0, 0
    t[s, b] = -1
    bad[s, b] = w.n_pool_blocks + 5  # out of range: read as a hole, reported when checked
    with pytest.raises(pkv.PkvError) as ei:
        pkv.paged_attn_decode(d.q, d.k, d.v, bad, d.lens, w.scale, flags=pkv.FLAG_CHECKED)
    assert ei.value.status == 1 and "1 block-table" in ei.value.message, ei.value.message
    o_unchecked, l_unchecked = pkv.paged_attn_decode(d.q, d.k, d.v, bad, d.lens, w.scale)
    o_hole, l_hole = pkv.paged_attn_decode(d.q, d.k, d.v, torch.from_numpy(t).cuda(), d.lens, w.scale)
    assert torch.equal(o_unchecked, o_hole)
    # a clean table passes checked mode with the same result
    oc, lc = pkv.paged_attn_decode(d.q, d.k, d.v, d.table, d.lens, w.scale, flags=pkv.FLAG_CHECKED)
    assert torch.equal(oc, ref)


@pytest.mark.parametrize("cfg,n_sample", [(2, 32), (3, 64), (5, 8)])
def test_decode_full_size(cfg, n_sample):
    """Full-size workload in the launch configuration the benchmark times;
    the oracle checks every sequence (the long-context batch: 8 of
    131,072 tokens), and every output is checked for properties that hold
    at any size."""
    import torch

    w = wgen.make(cfg)
    log(f"full-size decode workload {cfg} ({w.name}): generating on the GPU")
    d = Dev(w, gen_on_gpu=True)
    out, lse = d.decode()
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    l = lse.cpu().numpy()
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    rng = np.random.default_rng(cfg)
    seqs = sorted(rng.choice(w.n_seqs, size=n_sample, replace=False).tolist())
    if cfg == 3:
        seqs = sorted(set(seqs) | {0, 1})  # two forks of one group share their prefix
    log(f"  oracle on {len(seqs)} of {w.n_seqs} sequences")
    ro, rl, rows = d.oracle(seqs)
    compare(o[rows], l[rows], ro, rl, tol_of(w), f"{w.name} sampled")


def test_binding_refuses_undersized_arguments():
    """Outputs, lengths, windows and pools that are smaller than the call's
    sizes say are refused before any launch."""
    import torch

    w = wgen.make_custom(seed=4, n_seqs=3, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16, ctx=(10, 60))
    d = Dev(w)
    S, H, hd = w.n_seqs, w.n_q_heads, w.head_dim
    cases = [
        dict(out=torch.empty((S, H, hd - 1), dtype=torch.float32, device="cuda")),
        dict(out=torch.empty((S, H, hd), dtype=torch.float16, device="cuda")),
        dict(lse=torch.empty((S, H - 1), dtype=torch.float32, device="cuda")),
    ]
    for kw in cases:
        with pytest.raises((TypeError, ValueError)):
            d.decode(**kw)
    with pytest.raises(ValueError):
        pkv.paged_attn_decode(d.q, d.k, d.v, d.table, d.lens[:2].contiguous(), w.scale)
    with pytest.raises(ValueError):
        pkv.paged_attn_decode(d.q, d.k, d.v, d.table, d.lens, w.scale, mode="span",
                              window=torch.zeros((S - 1, 2), dtype=torch.int32, device="cuda"))
    with pytest.raises(TypeError):
        pkv.paged_attn_decode(d.q, d.k[..., :64].contiguous(), d.v, d.table, d.lens, w.scale)
    with pytest.raises(TypeError):
        pkv.paged_attn_decode(d.q[..., :64].contiguous(), d.k, d.v, d.table, d.lens, w.scale)
    out, lse = d.decode()  # the well-formed call still works
    ro, rl = d.oracle()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_of(w), "after refusals")


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_kv_map_at_the_run_limit(kind):
    """Eight runs per sequence (the most a kv_map may hold; runs overlap, stick
    out of the sequence or are empty) through decode, prefill and the
    resolver against the oracle; nine runs are refused."""
    import torch

    w = wgen.make_custom(seed=88, n_seqs=7, n_q_heads=8, n_kv_heads=2, head_dim=128, block_size=16,
                         fmts=("f16", "q8_0", "f16"), ctx=(1, 800), mode="kv_map", n_runs=8, kind=kind,
                         hole_frac=0.1)
    assert w.kv_map.shape[1] == 8
    d = Dev(w)
    out, lse = d.decode() if kind == "decode" else d.prefill()
    ro, rl = d.oracle()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_of(w), f"{kind} 8 runs")
    n_cand = int(np.max(np.sum(np.maximum(w.kv_map[:, :, 1], 0), axis=1))) + 3
    kw = {} if kind == "decode" else dict(cu_q=d.cu_q, q_pos=d.q_pos)
    rows = pkv.resolve_rows(d.table, d.lens, w.block_size, w.n_kv_heads, w.head_dim, w.n_pool_blocks, n_cand,
                            mode="kv_map", window=d.window, k_fmt=pkv.Q8_0, **kw)
    qs, qp = (np.arange(w.n_seqs), w.seq_lens - 1) if kind == "decode" else (w.q_seq(), w.q_pos)
    ref = oracle.resolve_rows("kv_map", w.block_table, w.seq_lens, w.block_size, qs, qp, n_cand, w.window,
                              w.kv_map)
    assert np.array_equal(rows.cpu().numpy(), ref)
    nine = torch.zeros((w.n_seqs, 9, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PkvError):
        if kind == "decode":
            pkv.paged_attn_decode(d.q, d.k, d.v, d.table, d.lens, w.scale, mode="kv_map", window=nine)
        else:
            pkv.paged_attn_prefill_window(d.q, d.cu_q, d.q_pos, d.k, d.v, d.table, d.lens, w.scale,
                                          int(np.max(np.diff(w.cu_q))), mode="kv_map", window=nine)


@pytest.mark.parametrize("mode", ["causal", "kv_map"])
def test_in_kernel_plan_equals_plan_pass(mode):
    """Planned calls over at most 256 sequences derive the work list inside
    the split kernel; larger ones write it with the plan pass first.  The
    same 200 sequences, once alone (in-kernel list) and once as the first
    200 of 300 (plan pass; same split size and cut slots), give bitwise
    equal results, and both match the oracle."""
    import torch

    w = wgen.make_custom(seed=404, n_seqs=300, n_q_heads=16, n_kv_heads=8, head_dim=128, block_size=16,
                         ctx=(1500, 6000), mode=mode, n_runs=3, hole_frac=0.05)
    d = Dev(w)
    win = d.window
    kw = dict(mode=w.mode, split_tokens=1024)
    out_all, lse_all = pkv.paged_attn_decode(d.q, d.k, d.v, d.table, d.lens, w.scale, window=win, **kw)
    n = 200
    out_sub, lse_sub = pkv.paged_attn_decode(d.q[:n], d.k, d.v, d.table[:n], d.lens[:n], w.scale,
                                             window=None if win is None else win[:n], **kw)
    assert torch.equal(out_sub, out_all[:n]) and torch.equal(lse_sub, lse_all[:n])
    ro, rl = d.oracle()
    compare(out_all.cpu().numpy(), lse_all.cpu().numpy(), ro, rl, tol_of(w), f"300 seqs {mode}")
