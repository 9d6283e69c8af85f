"""Decode, windowed prefill and the store captured into a HIP graph (torch's
graph API over the library's launches) and replayed: every replay, with
eager work and synchronizations between replays, must give bitwise the
result of the eager call.  None of these calls synchronizes, allocates or
records a memset (checked mode does synchronize and is not captured)."""

import numpy as np
import pytest

import paged_kv_cache_table_amd as pkv
from workloads import gen as wgen

from gpu_util import Dev, log

pytestmark = pytest.mark.gpu


def _capture(fn):
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture, as the graph API asks
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("kind", ["direct", "planned"])
def test_decode_graph_replays_equal_eager(kind):
    """direct: a small call (one workgroup per possible slot); planned: 64
    sequences x 32 possible 1024-position slots x 8 kv heads, so the call
    lists its work items (cut slots included) inside the graph."""
    import torch

    if kind == "direct":
        w = wgen.make_custom(seed=17, n_seqs=9, n_q_heads=16, n_kv_heads=4, head_dim=128, block_size=16,
                             ctx=(1, 900), mode="kv_map", n_runs=4, hole_frac=0.1)
        split = 0
    else:
        w = wgen.make_custom(seed=18, n_seqs=64, n_q_heads=32, n_kv_heads=8, head_dim=128, block_size=16,
                             ctx=(1500, 6000), mode="kv_map", n_runs=4, hole_frac=0.1, max_blocks=2048)
        split = 1024
    d = Dev(w)
    want_o, want_l = d.decode(split_tokens=split)
    shape = pkv.make_shape(d.q, d.k, d.v, d.table, w.n_seqs, w.scale, 0, split)
    ws = torch.empty(pkv.decode_workspace_bytes(shape, "kv_map", w.kv_map.shape[1]), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(want_o)
    lse = torch.empty_like(want_l)
    g = _capture(lambda: d.decode(out=out, lse=lse, workspace=ws, split_tokens=split))
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        other_o, _ = d.decode(split_tokens=split)  # eager work between replays, on its own buffers
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_o) and torch.equal(lse, want_l), f"replay {i}"
        assert torch.equal(other_o, want_o)
    log("  decode: 4 replays equal the eager call")


def test_prefill_graph_replays_equal_eager():
    import torch

    w = wgen.make(4, small=True)
    d = Dev(w)
    want_o, want_l = d.prefill()
    shape = pkv.make_shape(d.q, d.k, d.v, d.table, w.n_seqs, w.scale)
    max_q = int(np.max(np.diff(w.cu_q)))
    need = pkv.prefill_workspace_bytes(shape, d.q.shape[0], max_q, "kv_map", w.kv_map.shape[1])
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(want_o)
    lse = torch.empty_like(want_l)
    g = _capture(lambda: d.prefill(out=out, lse=lse, workspace=ws))
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        other_o, _ = d.prefill()  # eager work between replays, on its own buffers
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, want_o) and torch.equal(lse, want_l), f"replay {i}"
        assert torch.equal(other_o, want_o)
    log("  prefill: 4 replays equal the eager call")


def test_store_graph_replays_equal_eager():
    import torch

    st = wgen.make_store(seed=8, n_seqs=6, n_kv_heads=4, head_dim=128, block_size=16, n_pool_blocks=96,
                         max_blocks=12, k_fmt="q8_0", v_fmt="f16", src_fmt="f16")
    k_new, v_new = wgen.store_values(st, "cuda")
    kw = wgen.pool_width("q8_0", st.head_dim)
    table = torch.from_numpy(st.block_table).cuda()
    pos = torch.from_numpy(st.pos).cuda()
    sid = torch.from_numpy(st.seq_ids).cuda()

    def pools():
        return (torch.zeros((st.n_pool_blocks, st.n_kv_heads, st.block_size, kw), dtype=torch.uint8, device="cuda"),
                torch.zeros((st.n_pool_blocks, st.n_kv_heads, st.block_size, st.head_dim), dtype=torch.float16,
                            device="cuda"))

    ke, ve = pools()
    pkv.kv_store(k_new, v_new, pos, ke, ve, table, seq_ids=sid)
    kg, vg = pools()
    g = _capture(lambda: pkv.kv_store(k_new, v_new, pos, kg, vg, table, seq_ids=sid))
    for i in range(3):
        kg.zero_()  # back to the eager call's starting pools (zeros), so a replay that wrote nothing shows
        vg.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(kg, ke) and torch.equal(vg.view(torch.int16), ve.view(torch.int16)), f"replay {i}"
    log("  store: 3 replays equal the eager call")
