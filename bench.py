"""Benchmark of the paged-attention hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload decode3]

Default workload: decode on the 7B-class batch (64 sequences in 16 groups of
4 copy-on-write forks sharing a 2048-token prefix, 32 q / 8 kv heads,
head_dim 128, block 16, f16 K/V, 4096..32768 tokens each).  A step is one
pkv_paged_attn_decode call (split and log-sum-exp merge kernels; a plan
kernel first when the call plans more than 256 sequences) over the batch,
with all inputs resident in HBM.  Prints one JSON line:

* value: effective KV bandwidth = logical K/V bytes the queries attend to
  (B_log: every visible token x kv head, K and V rows) / step time;
* hbm_frac_step: B_uniq / step time / 8 TB/s, with B_uniq the call's
  distinct bytes (each physical K/V row once, q, table entries, seq_lens,
  out and lse, and the split partials written and read back);
* pct_of_device_copy: the same rate against a plain device copy measured in
  the same run;
* roofline: the split kernel's algorithmic bytes / the average duration of
  the call's partials half (the split kernel, and the plan kernel when there
  is one) from HIP events on the stream it runs on, against the 8 TB/s HBM
  peak;
* cpu_baseline: the float64 CPU oracle timed on a bounded sample of the same
  workload on this host, with the host's core counts and CPU model.

Other workloads (for the record; the default is the headline): decode1,
decode2, decode5, prefill4 (--prefill-k f16: the same batch with f16 K),
copy5b, store4, cow3, defrag3, int4; and calib, a plain device copy of
known size used to scale the HBM byte counters.

Counter summary (turns two rocprofv3 --pmc runs, FETCH_SIZE then WRITE_SIZE,
of a workload and of the calibration copy into bytes per launch):

    python bench.py --pmc-summary WORKLOAD KERNEL FETCH.csv WRITE.csv CAL_FETCH.csv CAL_WRITE.csv
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
CALIB_BYTES = 4 << 30  # bytes read and bytes written by one calibration copy
# Counter summaries per workload: the committed file and the sources that
# determine the measured kernel's code; a summary only applies while their
# hash is unchanged.
_CSRC = "paged_kv_cache_table_amd/csrc/"
TRAFFIC = {
    "decode3": ("profiles/decode_split_7b_class.traffic.json",
                (_CSRC + "pkv_internal.hpp", _CSRC + "decode_impl.hpp", _CSRC + "decode_f16.hip")),
    "decode2": ("profiles/decode_split_smollm_class.traffic.json",
                (_CSRC + "pkv_internal.hpp", _CSRC + "decode_impl.hpp", _CSRC + "decode_f16.hip")),
    "store4": ("profiles/store_w4.traffic.json",
               (_CSRC + "pkv_internal.hpp", _CSRC + "store.hip")),
    "prefill4": ("profiles/prefill_window_w4.traffic.json",
                 (_CSRC + "pkv_internal.hpp", _CSRC + "prefill.hip")),
}
MFMA_F16_PEAK_TFLOPS = 2500.0
METRIC = "paged decode attention: effective KV GB/s (% HBM peak) + queries/s"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def decode_bytes(w):
    """(B_log, B_uniq_kv, visible tokens per seq) for a causal decode batch."""
    bs = w.block_size
    row_k = w.row_bytes("k") // w.n_kv_heads
    row_v = w.row_bytes("v") // w.n_kv_heads
    b_log = 0
    vis = []
    uniq = set()
    for s in range(w.n_seqs):
        L = int(w.seq_lens[s])
        nb = (L + bs - 1) // bs
        ids = w.block_table[s, :nb]
        n = 0
        for b in range(nb):
            if ids[b] < 0:
                continue
            cnt = min(bs, L - b * bs)
            n += cnt
            uniq.add((int(ids[b]), cnt))
        vis.append(n)
        b_log += n * w.n_kv_heads * (row_k + row_v)
    # a shared block is read by every fork; count its rows once (the longest use)
    best = {}
    for blk, cnt in uniq:
        best[blk] = max(best.get(blk, 0), cnt)
    b_uniq = sum(best.values()) * w.n_kv_heads * (row_k + row_v)
    return b_log, b_uniq, vis


def host_cpu_info():
    """Host CPU facts for the baseline: logical CPUs, CPUs this process may
    use, physical cores and the model name (from lscpu)."""
    info = {"host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0))}
    try:
        import psutil

        info["physical_cores"] = psutil.cpu_count(logical=False)
    except Exception:  # pragma: no cover
        info["physical_cores"] = None
    model = None
    try:
        import subprocess

        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
            if line.startswith("Core(s) per socket:") and info["physical_cores"] is None:
                info["cores_per_socket"] = int(line.split(":", 1)[1])
    except Exception:  # pragma: no cover
        pass
    info["cpu_model"] = model
    return info


def cpu_baseline_decode(w, d, budget_s=12.0):
    """Time the oracle on whole sequences of the workload until budget_s."""
    import oracle
    from workloads import gen as wgen

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    b_log, _, vis = decode_bytes(w)
    per_tok = b_log / max(1, sum(vis))
    done_bytes = 0.0
    t_total = 0.0
    seqs = []
    for s in range(w.n_seqs):
        sub, kh, vh = wgen.host_subset(w, [s], d["k"], d["v"])
        qh = d["q"][s : s + 1].cpu().numpy()
        t0 = time.perf_counter()
        oracle.paged_decode(qh, kh, vh, w.k_fmt, w.v_fmt, sub.block_table, sub.seq_lens, w.block_size,
                            w.n_kv_heads, w.head_dim, w.scale)
        t_total += time.perf_counter() - t0
        done_bytes += vis[s] * per_tok
        seqs.append(s)
        if t_total >= budget_s:
            break
    res = {
        "value": round(done_bytes / t_total / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"float64 numpy oracle on {len(seqs)} of {w.n_seqs} sequences "
                  f"({sum(vis[s] for s in seqs)} visible tokens, {t_total:.1f} s; excludes host copies); "
                  f"cores = BLAS threads the oracle's products ran on",
        "queries_per_s": round(len(seqs) / t_total, 4),
    }
    res.update(host_cpu_info())
    return res


def sources_hash(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(workload):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed counter summary, or None if absent or taken on other kernel
    sources."""
    path, sources = TRAFFIC[workload]
    try:
        with open(os.path.join(ROOT, path)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256") != sources_hash(sources):
        return None
    return t.get("traffic_bytes_per_launch")


def _pmc_mean(path, kernel_substr, counter):
    vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
            if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter]
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel_substr!r} in {path}")
    return sum(vals) / len(vals), len(vals)


def pmc_summary(workload, kernel, fetch_csv, write_csv, cal_fetch_csv, cal_write_csv):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of `kernel`, each scaled by
    the factor that maps the same counter to the known bytes of the
    calibration copy.  `kernel` may name several kernels joined by '+' (the
    launches of one call): their per-dispatch means are added."""
    f_kib = w_kib = 0.0
    nf = nw = 0
    for k in kernel.split("+"):
        f, n1 = _pmc_mean(fetch_csv, k, "FETCH_SIZE")
        w_, n2 = _pmc_mean(write_csv, k, "WRITE_SIZE")
        f_kib, w_kib, nf, nw = f_kib + f, w_kib + w_, max(nf, n1), max(nw, n2)
    cf_kib, _ = _pmc_mean(cal_fetch_csv, "copy", "FETCH_SIZE")
    cw_kib, _ = _pmc_mean(cal_write_csv, "copy", "WRITE_SIZE")
    f_scale = CALIB_BYTES / (cf_kib * 1024)
    w_scale = CALIB_BYTES / (cw_kib * 1024)
    out = {
        "workload": workload,
        "kernel": kernel,
        "sources_sha256": sources_hash(TRAFFIC[workload][1]),
        "fetch_kib_per_dispatch": round(f_kib, 1), "fetch_dispatches": nf,
        "write_kib_per_dispatch": round(w_kib, 1), "write_dispatches": nw,
        "calib_fetch_kib": round(cf_kib, 1), "calib_write_kib": round(cw_kib, 1),
        "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
        "traffic_bytes_per_launch": int(f_kib * 1024 * f_scale + w_kib * 1024 * w_scale),
    }
    print(json.dumps(out, indent=2))
    return 0


class ColdCache:
    """Evicts L2 and the 256 MB Infinity Cache between timed steps by reading
    a 1 GiB buffer (filled once): the caches end up holding clean lines, so
    no write-back of unrelated dirty data lands inside the timed region."""

    def __init__(self):
        import torch

        self.buf = torch.ones(1 << 27, dtype=torch.int64, device="cuda")

    def __call__(self):
        self.buf.sum()


def run_calib(args):
    import torch

    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    return {"workload": "calib", "bytes_read": CALIB_BYTES, "bytes_written": CALIB_BYTES,
            "ms_per_copy": round(ms, 4), "GBps_read_plus_write": round(2 * CALIB_BYTES / (ms * 1e-3) / 1e9, 1)}


def decode_partial_rows(w, split, planned_units_min=4 * 2048):
    """Partial rows a decode call writes (and its merge reads): one per
    non-empty split slot of each sequence, plus the extra pieces of the slots
    a planned call cuts (each sequence's last min(2, ceil(4096 / (pieces x
    kv heads x seqs))) full slots, cut into pieces of >= 256 positions).
    Causal windows; this mirrors the split rule of the library's decode."""
    bs, S, hkv = w.block_size, w.n_seqs, w.n_kv_heads
    nspl = -(-w.max_blocks_per_seq * bs // split)
    planned = S * nspl * hkv > planned_units_min
    nsub = max(1, min(4, split // 256))
    fine = -(-(-(-split // nsub)) // bs) * bs
    while nsub > 1 and (nsub - 1) * fine >= split:
        nsub -= 1
    fine_per_seq = 0
    if planned and nsub > 1:
        fine_per_seq = min(2, -(-4096 // (nsub * hkv * S)), nspl)
    rows = 0
    for L in w.seq_lens:
        L = int(L)
        rows += -(-L // split) + min(fine_per_seq, L // split) * (nsub - 1)
    return rows


def run_decode(cfg, args):
    """Decode headline: one fused pkv_paged_attn_decode call (split + merge
    kernels, and a plan kernel first when the call plans more than 256
    sequences) per step.  Three passes over the same inputs after the
    warm-up: one call at a time between HIP events on the stream the library
    launches on (event_ms); the two halves of the call (partials = split
    kernel, after the plan kernel if any, then merge) between events, for
    the dominant-kernel roofline; and last,
    back to back by wall clock (ms_per_step, value)."""
    import torch

    import paged_kv_cache_table_amd as pkv
    from workloads import gen as wgen

    w = wgen.make(cfg)
    log(f"[bench] workload {cfg}: {w.name}; generating inputs on the GPU")
    q, k, v = wgen.materialize(w, "cuda")
    table = torch.from_numpy(w.block_table).cuda()
    lens = torch.from_numpy(w.seq_lens.astype(np.int32)).cuda()
    shape = pkv.make_shape(q, k, v, table, w.n_seqs, w.scale, split_tokens=args.split)
    ws = torch.empty(pkv.decode_workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    out = torch.empty((w.n_seqs, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.n_seqs, w.n_q_heads), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(part="both"):
        pkv.paged_attn_decode(q, k, v, table, lens, w.scale, out=out, lse=lse, workspace=ws,
                              split_tokens=args.split, part=part)

    # host-side byte counts first, so that the timed passes follow the
    # warm-up directly (an idle GPU clocks down)
    b_log, b_uniq_kv, vis = decode_bytes(w)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # A batch whose K/V fit in the 256 MB Infinity Cache would be timed from
    # the cache: evict before every timed step and time each step with events
    # (the eviction itself stays outside); the warm figure is kept, labelled.
    cold = b_uniq_kv < (1 << 30)
    flush = ColdCache() if cold else None
    log(f"[bench] timing {args.steps} steps" + (" (caches evicted before each)" if cold else ""))
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # pass 1: one fused call per step between events
    call_ms = []
    for _ in range(args.steps):
        if cold:
            flush()
        e = [ev(), ev()]
        e[0].record(stream)
        call()
        e[1].record(stream)
        if cold:
            torch.cuda.synchronize()
        call_ms.append(e)
    torch.cuda.synchronize()
    call_ms = [e[0].elapsed_time(e[1]) for e in call_ms]
    # pass 2: the two halves of the call
    halves = []
    for _ in range(args.steps):
        if cold:
            flush()
        e = [ev(), ev(), ev()]
        e[0].record(stream)
        call("partials")
        e[1].record(stream)
        call("merge")
        e[2].record(stream)
        if cold:
            torch.cuda.synchronize()
        halves.append(e)
    torch.cuda.synchronize()
    # pass 3: back to back, wall clock (no events in the stream), last, so
    # that it runs at the clocks of a GPU that has been busy
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    part_ms = [e[0].elapsed_time(e[1]) for e in halves]
    merge_ms = [e[1].elapsed_time(e[2]) for e in halves]
    ms = float(np.mean(call_ms)) if cold else wall_ms

    # algorithmic bytes of the whole call (B_uniq): distinct K/V rows, q, the
    # table entries and seq_lens read, out and lse written, and the split
    # partials written by the split kernel and read by the merge
    G, hd = w.group, w.head_dim
    split = pkv.decode_split_tokens(shape)
    rows = decode_partial_rows(w, split)
    q_bytes = q.numel() * q.element_size()
    table_bytes = sum((int(L) + w.block_size - 1) // w.block_size for L in w.seq_lens) * 4
    lens_bytes = 4 * w.n_seqs
    out_bytes = out.numel() * 4 + lse.numel() * 4
    part_bytes = rows * w.n_q_heads * (hd + 2) * 4
    b_uniq = b_uniq_kv + q_bytes + table_bytes + lens_bytes + out_bytes + 2 * part_bytes
    # the split kernel's own bytes: K/V, q, table, seq_lens, partials written
    alg_split = b_uniq_kv + q_bytes + table_bytes + lens_bytes + part_bytes
    part_avg = float(np.mean(part_ms))
    achieved = alg_split / (part_avg * 1e-3) / 1e9
    copy = measure_copy_GBps()
    step_gbs = b_uniq / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(b_log / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.k_fmt,
        "data": "synthetic",
        "config": {
            "workload": f"{w.name} decode: {w.n_seqs} seqs, {w.n_q_heads} q / {w.n_kv_heads} kv heads, "
                        f"head_dim {w.head_dim}, block {w.block_size}, {w.k_fmt} K/V, "
                        f"ctx {int(w.seq_lens.min())}-{int(w.seq_lens.max())}",
            "seqs": w.n_seqs,
            "visible_tokens": int(sum(vis)),
            "B_log_bytes": int(b_log),
            "B_uniq_bytes": int(b_uniq),
            "B_uniq_parts": {"kv": int(b_uniq_kv), "q": q_bytes, "table": table_bytes, "seq_lens": lens_bytes,
                             "out_lse": out_bytes, "partials_written_and_read": 2 * part_bytes},
            "split_tokens": int(split),
            "partial_rows": int(rows),
        },
        "step": "one pkv_paged_attn_decode call (split + merge kernels; a plan kernel first when the call plans more than 256 sequences)",
        "timing": ("HIP events per call, caches evicted before each call" if cold
                   else "wall clock over back-to-back calls"),
        "queries_per_s": round(w.n_seqs / (ms * 1e-3), 1),
        # the headline fraction: B_uniq of the whole call / step time / 8 TB/s
        "hbm_frac_step": round(step_gbs / HBM_PEAK_GBS, 4),
        "uniq_GBps_step": round(step_gbs, 1),
        "hbm_frac_call_median": round(b_uniq / (float(np.median(call_ms)) * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "pct_of_device_copy": round(100 * step_gbs / copy["GBps_read_plus_write"], 1),
        "device_copy": copy,
        "event_ms": {"call_median": round(float(np.median(call_ms)), 5),
                     "call_mean": round(float(np.mean(call_ms)), 5),
                     "call_p10": round(float(np.percentile(call_ms, 10)), 5),
                     "call_p90": round(float(np.percentile(call_ms, 90)), 5),
                     "wall_back_to_back": round(wall_ms, 5),
                     "partials_mean": round(part_avg, 5),
                     "merge_mean": round(float(np.mean(merge_ms)), 5)},
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_split_kernel",
            # events bracket the partials half of the call: the one-workgroup
            # plan kernel (when the call is planned) and the split kernel
            "timed": "decode partials call (decode_split_kernel; a decode_plan_kernel first above 256 sequences), HIP events",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(f"decode{cfg}") if f"decode{cfg}" in TRAFFIC and not args.split else None,
            "algorithmic_bytes": int(alg_split),
        },
    }
    if cold:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            call()
        torch.cuda.synchronize()
        warm_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        res["warm_unflushed"] = {"ms_per_step": round(warm_ms, 5),
                                 "GBps_B_log": round(b_log / (warm_ms * 1e-3) / 1e9, 2)}
    return res, w, {"q": q, "k": k, "v": v}


def measure_copy_GBps(nbytes=1 << 30, reps=10):
    """A plain device-to-device copy of `nbytes` on the same GPU, timed with
    HIP events: read + write bytes per second (the secondary reference for
    the decode figure)."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return {"bytes": 2 * nbytes, "ms": round(ms, 4), "GBps_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def prefill_work(w, dev):
    """(flops, unique K/V bytes, visible (query, position) pairs) of a prefill
    batch, counted from the library's own resolver (parity-tested bit-exact):
    per visible pair and q head 4*hd flops (q.k and p.v); bytes count each
    distinct pool row read once, K and V, all kv heads."""
    import torch

    import paged_kv_cache_table_amd as pkv

    runs = w.kv_map
    n_cand = int(np.max(np.sum(np.maximum(runs[:, :, 1], 0), axis=1)))
    rows = pkv.resolve_rows(dev["table"], dev["lens"], w.block_size, w.n_kv_heads, w.head_dim, w.n_pool_blocks,
                            n_cand, mode="kv_map", window=dev["win"], cu_q=dev["cu_q"], q_pos=dev["q_pos"],
                            n_q_heads=w.n_q_heads, k_fmt=pkv.Q8_0 if w.k_fmt == "q8_0" else pkv.F16)
    pairs = int((rows >= 0).sum())
    uniq = int(torch.unique(rows[rows >= 0]).numel())
    flops = pairs * w.n_q_heads * 4 * w.head_dim
    kv_bytes = uniq * (w.row_bytes("k") + w.row_bytes("v"))
    return flops, kv_bytes, pairs


def run_prefill(args):
    import torch

    import paged_kv_cache_table_amd as pkv
    from workloads import gen as wgen

    w = wgen.make(4)
    kfmt = getattr(args, "prefill_k", "q8_0")
    if kfmt != w.k_fmt:
        # the same batch with K stored in another format (what the q8_0 K
        # format costs the kernel); inputs are regenerated in that format
        w.k_fmt = kfmt
    log(f"[bench] workload 4: {w.name}, K {w.k_fmt}; generating inputs on the GPU")
    q, k, v = wgen.materialize(w, "cuda")
    dev = {n: torch.from_numpy(np.ascontiguousarray(x).astype(np.int32)).cuda()
           for n, x in (("table", w.block_table), ("lens", w.seq_lens), ("cu_q", w.cu_q), ("q_pos", w.q_pos),
                        ("win", w.kv_map))}
    max_q = int(np.max(np.diff(w.cu_q)))
    out = torch.empty((w.n_queries, w.n_q_heads, w.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.n_queries, w.n_q_heads), dtype=torch.float32, device="cuda")
    flush = ColdCache()  # the whole input (0.16 GB of K/V) would otherwise sit in the 256 MB cache

    def call():
        pkv.paged_attn_prefill_window(q, dev["cu_q"], dev["q_pos"], k, v, dev["table"], dev["lens"], w.scale, max_q,
                                      mode="kv_map", window=dev["win"], out=out, lse=lse)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(args.steps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.mean(times))
    # warm figure, labelled: the same calls back to back, inputs left in the caches
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    for _ in range(args.steps):
        call()
    w1.record(stream)
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1) / args.steps
    flops, kv_bytes, pairs = prefill_work(w, dev)
    tflops = flops / (ms * 1e-3) / 1e12
    io_bytes = kv_bytes + q.numel() * 2 + out.numel() * 4 + lse.numel() * 4
    return {
        "metric": "windowed prefill: TFLOP/s (% MFMA f16 peak) and HBM GB/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"f16 (K {w.k_fmt})", "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.n_seqs} seqs x {max_q} queries, 32 q / 8 kv heads, hd 128, block 32, "
                               f"K {w.k_fmt}, V f16; half one span, half 4 runs; causal in window; cache flushed per step",
                   "visible_pairs": pairs, "flops": flops, "kv_bytes": kv_bytes},
        "roofline": {"bound": "mfma", "kernel": "prefill_order_kernel + prefill_kernel + prefill_merge_kernel (one call)",
                     "achieved": round(tflops, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": stored_traffic("prefill4") if w.k_fmt == "q8_0" else None, "hbm_GBps": round(io_bytes / (ms * 1e-3) / 1e9, 1),
                     "hbm_frac": round(io_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "event_ms": {"median": round(float(np.median(times)), 5), "p10": round(float(np.percentile(times, 10)), 5),
                     "p90": round(float(np.percentile(times, 90)), 5)},
        "warm_unflushed": {"ms_per_call": round(warm_ms, 5),
                           "TFLOPs": round(flops / (warm_ms * 1e-3) / 1e12, 2)},
    }


def run_copy(args):
    """copy_cells on 10,000 random overlapping moves over K and V pools of
    2^17 blocks (8 kv heads x 16 slots x 512 B).  A step is one
    kv_copy_cells call: the host plan (pinned memory), its asynchronous
    upload and the device copies.  value: back-to-back calls, no
    synchronization between them (the host plan of one call overlaps the
    device copies of the one before), wall clock; also reported: one call at
    a time (synchronized), the host plan alone and the device half alone
    (HIP events around pkv_copy_cells_apply with the plan already on the
    device)."""
    import torch

    import paged_kv_cache_table_amd as pkv
    from workloads import gen as wgen

    w = wgen.make(5)
    ms_ = wgen.make_moves(seed=55)
    log("[bench] copy_cells: 10k moves on two 2^21-row pools")
    k = torch.zeros((w.n_pool_blocks, w.n_kv_heads, w.block_size, w.head_dim), dtype=torch.float16, device="cuda")
    v = torch.zeros_like(k)
    changed = int(ms_.moves[:, 2].sum())  # rows the moves name (a row moved twice counts twice)
    row = w.row_bytes("k") + w.row_bytes("v")
    ws = torch.empty(pkv.copy_cells_workspace_bytes(ms_.moves, k, v), dtype=torch.uint8, device="cuda")
    n_rows = w.n_pool_blocks * w.block_size

    def call():
        pkv.kv_copy_cells(k, v, ms_.moves, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    # one call at a time
    t_single = []
    for _ in range(args.steps):
        t0 = time.perf_counter()
        call()
        torch.cuda.synchronize()
        t_single.append(time.perf_counter() - t0)
    # host plan alone
    t_plan = []
    for _ in range(args.steps):
        t0 = time.perf_counter()
        info, plan_h = pkv.copy_cells_plan(ms_.moves, n_rows)
        t_plan.append(time.perf_counter() - t0)
    # device half alone
    plan_d = plan_h[: info.n_words].cuda()
    stage = torch.empty(pkv.copy_cells_stage_bytes(info, k, v), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    dev_ms = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pkv.copy_cells_apply(k, v, info, plan_d, stage)
        e1.record()
        torch.cuda.synchronize()
        dev_ms.append(e0.elapsed_time(e1))
    # back to back, last
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        call()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / args.steps
    moved = 2 * changed * row  # each moved row read once and written once
    dev = float(np.mean(dev_ms))
    dev_bytes = 2 * (info.n_scatter + info.n_gather) * row  # rows read and written by the device half
    return {
        "metric": "copy_cells: rows moved per second (bit-exact, sequential order_moves semantics)",
        "value": round(changed / wall, 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bytes", "data": "synthetic",
        "config": {"workload": "10,000 random overlapping moves (len 1..32) on K and V pools of 2^17 blocks x 16 "
                               "slots x 8 kv heads x 512 B; back-to-back kv_copy_cells calls (host plan + "
                               "asynchronous upload + device copies), wall clock",
                   "moved_rows": changed, "min_bytes": moved, "plan_words": int(info.n_words),
                   "staged_rows": int(info.n_gather), "written_rows": int(info.n_scatter)},
        "GBps_min_bytes_wall": round(moved / wall / 1e9, 2),
        "single_call_ms": round(float(np.mean(t_single)) * 1e3, 4),
        "host_plan_ms": round(float(np.mean(t_plan)) * 1e3, 4),
        "device_ms": round(dev, 4),
        "roofline": {"bound": "hbm", "kernel": "copy_rows_kernel (gather + scatter, both pools)",
                     "achieved": round(dev_bytes / (dev * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dev_bytes / (dev * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None},
    }


def run_store(args):
    """The store that fills the windowed-prefill pools: every position of the
    16 sequences (93,809 tokens), f16 rows into the q8_0 K pool (store
    quantizer) and the f16 V pool, through the block table."""
    import torch

    import paged_kv_cache_table_amd as pkv
    from workloads import gen as wgen

    w = wgen.make(4)
    st = wgen.store_of_workload(w, src_fmt="f16")
    log(f"[bench] store: {st.n_tok} tokens of workload 4 into its q8_0 K / f16 V pools")
    k_new, v_new = wgen.store_values(st, "cuda")
    kp = torch.zeros((st.n_pool_blocks, st.n_kv_heads, st.block_size, wgen.pool_width("q8_0", st.head_dim)),
                     dtype=torch.uint8, device="cuda")
    vp = torch.zeros((st.n_pool_blocks, st.n_kv_heads, st.block_size, st.head_dim), dtype=torch.float16,
                     device="cuda")
    table = torch.from_numpy(st.block_table).cuda()
    pos = torch.from_numpy(st.pos).cuda()
    sid = torch.from_numpy(st.seq_ids).cuda()
    flush = ColdCache()

    def call():
        pkv.kv_store(k_new, v_new, pos, kp, vp, table, seq_ids=sid)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(args.steps):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.mean(times))
    n = st.n_tok
    seg_k = wgen.q8_0_seg_bytes(st.head_dim)
    src_bytes = 2 * n * st.n_kv_heads * st.head_dim * 2            # K and V rows read, f16
    dst_bytes = n * st.n_kv_heads * (seg_k + 2 * st.head_dim)       # q8_0 K and f16 V rows written
    idx_bytes = n * 8                                               # positions and sequence ids
    total = src_bytes + dst_bytes + idx_bytes
    gbs = total / (ms * 1e-3) / 1e9
    return {
        "metric": "KV store (q8_0 K quantizer + f16 V): HBM GB/s (% HBM peak) and tokens/s",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16 -> q8_0 / f16", "data": "synthetic",
        "config": {"workload": f"store of {n} tokens (16 seqs of 2048..8192 positions, 8 kv heads, hd 128, block 32, "
                               "tables from a 2^13-block pool): f16 K rows -> q8_0, f16 V rows -> f16; "
                               "cache flushed per step",
                   "tokens": n, "bytes": total},
        "tokens_per_s": round(n / (ms * 1e-3), 1),
        "roofline": {"bound": "hbm", "kernel": "store_kernel", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": stored_traffic("store4"),
                     "algorithmic_bytes": int(total)},
    }


def run_cow(args):
    """Copy-on-write fork step: 256 parents (7B-class layer shape: 8 kv heads,
    hd 128, block 16, f16 K/V) of 1000..8000 tokens, each forked three times;
    in one step all 1024 sequences append one token.  Every fork whose
    shared last block is partial must copy it first.  Timed per step: host
    planning (prepare_writes), the upload of its ops, cow_apply (block
    copies + device table patches) and the store of the 1024 rows; the
    copy kernel is also timed alone for its roofline."""
    import torch

    import paged_kv_cache_table_amd as pkv

    rng = np.random.default_rng(3)
    n_par, fan, hkv, hd, bs = 256, 4, 8, 128, 16
    n_seqs = n_par * fan
    L = rng.integers(1000, 8001, size=n_par).astype(np.int32)
    max_blocks = 8192 // bs + 2
    n_blocks = int(np.sum((L + bs - 1) // bs)) * 2 + 4096
    log(f"[bench] cow: {n_par} parents x {fan} members, {n_blocks} blocks per pool")
    pool = pkv.BlockPool(n_blocks, n_seqs, max_blocks, bs)
    k = torch.zeros((n_blocks, hkv, bs, hd), dtype=torch.float16, device="cuda")
    v = torch.zeros_like(k)
    table = torch.full((n_seqs, max_blocks), -1, dtype=torch.int32, device="cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    # parents: one prefill store each (fresh blocks only)
    pseqs = np.arange(0, n_seqs, fan, dtype=np.int32)
    ops = pool.prepare_writes(pseqs, np.zeros(n_par, dtype=np.int32), L)
    pkv.cow_apply(k, v, ops, table)
    n_tok = int(L.sum())
    sid = torch.from_numpy(np.repeat(pseqs, L)).cuda()
    pos = torch.from_numpy(np.concatenate([np.arange(x, dtype=np.int32) for x in L])).cuda()
    for lo in range(0, n_tok, 1 << 16):
        hi = min(n_tok, lo + (1 << 16))
        rows = torch.randn((hi - lo, hkv, hd), generator=g, device="cuda").half()
        pkv.kv_store(rows, rows, pos[lo:hi], k, v, table, seq_ids=sid[lo:hi])
    step_rows = torch.randn((n_seqs, hkv, hd), generator=g, device="cuda").half()
    all_seqs = np.arange(n_seqs, dtype=np.int32)
    step_pos_h = np.repeat(L, fan).astype(np.int32)
    step_pos = torch.from_numpy(step_pos_h).cuda()
    step_sid = torch.from_numpy(all_seqs).cuda()
    ones = np.ones(n_seqs, dtype=np.int32)
    ops_host = torch.empty((4 * n_seqs, 3), dtype=torch.int32).pin_memory()
    ops_dev = torch.empty((4 * n_seqs, 3), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def reset():
        """Untimed: drop the members' step tokens and forks, fork again."""
        for p in range(n_par):
            base = fan * p
            pool.remove(base, int(L[p]), int(L[p]) + 1)
            for m in range(1, fan):
                pool.remove(base + m, 0, 1 << 30)
            for m in range(1, fan):
                pool.fork(base, base + m)
        t, _ = pool.export()
        table.copy_(torch.from_numpy(t))
        torch.cuda.synchronize()

    def step(ev=None):
        ops = pool.prepare_writes(all_seqs, step_pos_h, ones)
        n = len(ops)
        ops_host[:n].numpy()[:] = ops
        ops_dev[:n].copy_(ops_host[:n], non_blocking=True)
        if ev is not None:
            ev[0].record(stream)
        pkv.cow_apply(k, v, ops_dev[:n], table)
        if ev is not None:
            ev[1].record(stream)
        pkv.kv_store(step_rows, step_rows, step_pos, k, v, table, seq_ids=step_sid)
        return ops

    for p in range(n_par):
        for m in range(1, fan):
            pool.fork(fan * p, fan * p + m)
    t, _ = pool.export()
    table.copy_(torch.from_numpy(t))
    for _ in range(args.warmup):
        step()
        torch.cuda.synchronize()
        reset()
    walls = []
    n_copies = 0
    for _ in range(args.steps):  # wall clock: host plan + upload + both kernels
        t0 = time.perf_counter()
        ops = step()
        torch.cuda.synchronize()
        walls.append(time.perf_counter() - t0)
        n_copies = int(np.count_nonzero(ops[:, 0] >= 0))
        reset()
    kern, dev = [], []
    for _ in range(args.steps):  # device time: the GPU is kept busy while the host enqueues
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        torch.cuda._sleep(400000)
        step(ev)
        ev[2].record(stream)
        torch.cuda.synchronize()
        kern.append(ev[0].elapsed_time(ev[1]))
        dev.append(ev[0].elapsed_time(ev[2]))
        reset()
    wall = float(np.mean(walls))
    kms = float(np.mean(kern))
    block_bytes = hkv * bs * hd * 2
    copy_bytes = 2 * n_copies * 2 * block_bytes  # K and V blocks, read + written
    gbs = copy_bytes / (kms * 1e-3) / 1e9
    return {
        "metric": "copy-on-write fork step: sequences appended per second (host plan + block copies + store)",
        "value": round(n_seqs / wall, 1), "unit": "sequences/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": f"{n_par} parents of 1000..8000 tokens x {fan} members (8 kv heads, hd 128, block 16, "
                               f"f16 K/V); every member appends one token; wall clock per step",
                   "sequences": n_seqs, "block_copies": n_copies, "copy_bytes": copy_bytes},
        "roofline": {"bound": "hbm", "kernel": "cow_apply_kernel", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel_ms": round(kms, 5)},
        "device_ms_per_step": round(float(np.mean(dev)), 5),
    }


def run_defrag(args):
    """Compaction of a fragmented pool: 64 sequences of 4096..32768 tokens
    (7B-class layer: 8 kv heads, hd 128, block 16, f16 K/V) allocated
    through the block pool, then every other one dropped; defrag(-1) moves
    the live blocks above the live count into the holes below and the row
    moves run through kv_copy_cells.  Timed per step by wall clock: the
    pool's plan, copy_cells' plan and upload, and the device copies."""
    import torch

    import paged_kv_cache_table_amd as pkv

    rng = np.random.default_rng(3)
    n_seqs, hkv, hd, bs = 64, 8, 128, 16
    L = rng.integers(4096, 32769, size=n_seqs).astype(np.int32)
    max_blocks = 32768 // bs
    n_blocks = int(np.sum((L + bs - 1) // bs)) + 1024
    log(f"[bench] defrag: {n_seqs} sequences, {n_blocks} blocks per pool")
    k = torch.empty((n_blocks, hkv, bs, hd), dtype=torch.float16, device="cuda")
    v = torch.empty_like(k)

    def fragmented():
        pool = pkv.BlockPool(n_blocks, n_seqs, max_blocks, bs)
        for s_ in range(n_seqs):
            pool.prepare_writes([s_], [0], [int(L[s_])])
        for s_ in range(0, n_seqs, 2):
            pool.remove(s_, 0, 1 << 30)
        return pool

    row_bytes = 2 * hkv * hd * 2  # K and V rows
    walls, plans, devs = [], [], []
    moved_rows = 0
    for it in range(args.warmup + args.steps):
        pool = fragmented()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        moves = pool.defrag(-1)
        t1 = time.perf_counter()
        e0.record()
        pkv.kv_copy_cells(k, v, moves)
        e1.record()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        if it >= args.warmup:
            walls.append(t2 - t0)
            plans.append(t1 - t0)
            devs.append(e0.elapsed_time(e1))
        moved_rows = int(moves[:, 2].sum())
    wall = float(np.mean(walls))
    dev_ms = float(np.mean(devs))
    moved_bytes = 2 * moved_rows * row_bytes  # each moved row read once and written once
    gbs = moved_bytes / (dev_ms * 1e-3) / 1e9
    return {
        "metric": "defrag: rows moved per second (pool plan + copy_cells plan, upload and copies)",
        "value": round(moved_rows / wall, 1), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(wall * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bytes", "data": "synthetic",
        "config": {"workload": f"{n_seqs} sequences of 4096..32768 tokens (8 kv heads, hd 128, block 16, f16 K/V), "
                               "every other one dropped, then defrag(-1) + kv_copy_cells; wall clock",
                   "moves": int(len(moves)), "moved_rows": moved_rows, "moved_bytes": moved_bytes},
        "pool_plan_ms": round(float(np.mean(plans)) * 1e3, 4),
        "roofline": {"bound": "hbm", "kernel": "copy_rows_kernel (copy_cells: plan upload + copies)",
                     "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "device_ms": round(dev_ms, 5)},
    }


def run_int4(args):
    """int4 cold-block codec on the 7B-class block shape (8 kv heads x 16
    slots x hd 128, f16: 32 KiB per block): encode 16,384 random blocks of a
    2^15-block pool into blobs (f32 scale + 8 KiB of nibbles), then decode
    them into 16,384 other blocks.  Each launch timed with HIP events after
    a cache eviction."""
    import torch

    import paged_kv_cache_table_amd as pkv

    rng = np.random.default_rng(6)
    nb, n = 1 << 15, 16384
    g = torch.Generator(device="cuda")
    g.manual_seed(6)
    pool = torch.randn((nb, 8, 16, 128), generator=g, device="cuda").half()
    perm = rng.permutation(nb)
    src = torch.from_numpy(perm[:n].astype(np.int32)).cuda()
    dst = torch.from_numpy(perm[n : 2 * n].astype(np.int32)).cuda()
    elems = 8 * 16 * 128
    blob = pkv.int4_blob_bytes(elems)
    blobs = torch.zeros((n, (blob + 15) // 16 * 16), dtype=torch.uint8, device="cuda")
    flush = ColdCache()
    stream = torch.cuda.current_stream()
    enc, dec = [], []
    for it in range(args.warmup + args.steps):
        flush()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        pkv.int4_encode(pool, src, blobs)
        e[1].record(stream)
        flush()
        e[2].record(stream)
        pkv.int4_decode(blobs, pool, dst)
        e[3].record(stream)
        torch.cuda.synchronize()
        if it >= args.warmup:
            enc.append(e[0].elapsed_time(e[1]))
            dec.append(e[2].elapsed_time(e[3]))
    enc_ms, dec_ms = float(np.mean(enc)), float(np.mean(dec))
    blk_bytes = elems * 2
    bytes_each = n * (blk_bytes + blob)  # read a block, write a blob (encode) or the reverse (decode)
    enc_gbs = bytes_each / (enc_ms * 1e-3) / 1e9
    dec_gbs = bytes_each / (dec_ms * 1e-3) / 1e9
    return {
        "metric": "int4 cold-block codec: encode HBM GB/s (% HBM peak); decode alongside",
        "value": round(enc_gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(enc_ms + dec_ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16 <-> int4", "data": "synthetic",
        "config": {"workload": f"{n} random blocks of a 2^15-block pool, 8 kv heads x 16 slots x hd 128 f16 "
                               f"(32 KiB) <-> {blob}-byte blobs; encode then decode into other blocks; "
                               "cache evicted before each launch",
                   "blocks": n, "bytes_per_launch": bytes_each},
        "decode_GBps": round(dec_gbs, 1), "encode_ms": round(enc_ms, 5), "decode_ms": round(dec_ms, 5),
        "roofline": {"bound": "hbm", "kernel": "int4_encode_kernel", "achieved": round(enc_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(enc_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None},
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode3",
                    choices=["decode1", "decode2", "decode3", "decode5", "prefill4", "copy5b", "store4", "cow3", "defrag3", "int4", "calib"])
    ap.add_argument("--pmc-summary", nargs=6, metavar=("WORKLOAD", "KERNEL", "FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"))
    ap.add_argument("--split", type=int, default=0, help="decode split size in tokens (0 = automatic)")
    ap.add_argument("--prefill-k", default="q8_0", choices=["q8_0", "f16"],
                    help="K format of the prefill4 batch (q8_0 as the workload states; f16 for comparison)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    args = ap.parse_args(argv)
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary)
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(sequences shard across GPUs with no exchange, so per-GPU throughput is the figure).",
              file=sys.stderr)
        return 2
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.workload == "calib":
        print(json.dumps(run_calib(args)), flush=True)
        return 0
    if args.workload.startswith("decode"):
        res, w, d = run_decode(int(args.workload[-1]), args)
        if not args.no_cpu_baseline:
            log("[bench] timing the CPU oracle on a sample")
            res["cpu_baseline"] = cpu_baseline_decode(w, d, args.cpu_budget)
        else:
            res["cpu_baseline"] = None
    elif args.workload == "prefill4":
        res = run_prefill(args)
    elif args.workload == "store4":
        res = run_store(args)
    elif args.workload == "cow3":
        res = run_cow(args)
    elif args.workload == "defrag3":
        res = run_defrag(args)
    elif args.workload == "int4":
        res = run_int4(args)
    elif args.workload == "copy5b":
        res = run_copy(args)
    else:
        print(f"unknown workload {args.workload}", file=sys.stderr)
        return 2
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
