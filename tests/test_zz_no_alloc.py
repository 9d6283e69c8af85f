"""pkv_paged_attn_decode_noalloc (decode with the library's built-in device
scratch, for callers that cannot allocate) against pkv_paged_attn_decode
with a caller workspace: two calls in a row on one GPU, the second with a
smaller input, each bitwise equal to the workspace call and within the
oracle's tolerance; a call that needs more than the scratch is refused
before anything runs."""

import numpy as np
import pytest

import paged_kv_cache_table_amd as pkv
from workloads import gen as wgen

from gpu_util import Dev, compare, log, tol_of

pytestmark = pytest.mark.gpu


def _noalloc_vs_workspace(w, what):
    import torch

    d = Dev(w)
    ref_out, ref_lse = d.decode()
    S, H, hd = w.n_seqs, w.n_q_heads, w.head_dim
    out = torch.full((S, H, hd), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((S, H), float("nan"), dtype=torch.float32, device="cuda")
    pkv.paged_attn_decode_noalloc(d.q, d.k, d.v, d.table, d.lens, w.scale, out, lse, mode=w.mode,
                                  window=d.window)
    torch.cuda.synchronize()
    log(f"  {what}: {S} seqs, workspace call needs "
        f"{pkv.decode_workspace_bytes(pkv.make_shape(d.q, d.k, d.v, d.table, S, w.scale), w.mode, 1 if w.mode != 'kv_map' else w.kv_map.shape[1])} bytes")
    assert torch.equal(out, ref_out), f"{what}: out differs from the workspace call"
    assert torch.equal(lse, ref_lse), f"{what}: lse differs from the workspace call"
    ro, rl = d.oracle()
    compare(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, tol_of(w), what)


def test_noalloc_decode_two_calls_second_smaller():
    # first call: 100 sequences, planned path (work list and cut slots)
    w1 = wgen.make_custom(seed=71, n_seqs=100, n_q_heads=16, n_kv_heads=8, head_dim=128, block_size=16,
                          ctx=(1, 3000), hole_frac=0.05)
    _noalloc_vs_workspace(w1, "no-alloc decode, 100 seqs")
    # second call: fewer sequences, another geometry and a span window
    w2 = wgen.make_custom(seed=72, n_seqs=7, n_q_heads=9, n_kv_heads=3, head_dim=64, block_size=16,
                          ctx=(1, 700), mode="span", hole_frac=0.05)
    _noalloc_vs_workspace(w2, "no-alloc decode, 7 seqs, span")


def test_noalloc_refuses_more_than_the_scratch():
    import torch

    S, MB, Hq, Hkv, hd, bs = 256, 65536, 8, 8, 64, 16
    q = torch.zeros((S, Hq, hd), dtype=torch.float16, device="cuda")
    k = torch.zeros((4, Hkv, bs, hd), dtype=torch.float16, device="cuda")
    v = torch.zeros_like(k)
    table = torch.full((S, MB), -1, dtype=torch.int32, device="cuda")
    lens = torch.zeros((S,), dtype=torch.int32, device="cuda")
    shape = pkv.make_shape(q, k, v, table, S, 0.125)
    assert pkv.decode_workspace_bytes(shape) > pkv.NOALLOC_SCRATCH_BYTES
    out = torch.full((S, Hq, hd), 7.0, device="cuda")
    lse = torch.full((S, Hq), 7.0, device="cuda")
    with pytest.raises(pkv.PkvError) as ei:
        pkv.paged_attn_decode_noalloc(q, k, v, table, lens, 0.125, out, lse)
    assert ei.value.status == 3 and "scratch" in ei.value.message
    torch.cuda.synchronize()
    assert torch.all(out == 7.0) and torch.all(lse == 7.0)
