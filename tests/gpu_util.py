"""Helpers shared by the GPU tests: put a workload on the device, run the
library, run the oracle on the same bytes, compare."""

from __future__ import annotations

import math
import sys

import numpy as np

import oracle
import paged_kv_cache_table_amd as pkv
from workloads import gen as wgen

TOL = {"f32": 1e-5, "f16": 2e-3, "q8_0": 2e-3}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def tol_of(w) -> float:
    return max(TOL[w.q_fmt], TOL[w.k_fmt], TOL[w.v_fmt])


class Dev:
    """A workload's tensors on the GPU (and, when small, on the host)."""

    def __init__(self, w: wgen.Workload, gen_on_gpu: bool = False, host: bool = True):
        import torch

        self.w = w
        dev = "cuda"
        if gen_on_gpu:
            q, k, v = wgen.materialize(w, dev)
            self.qh = self.kh = self.vh = None
        else:
            q, k, v = wgen.materialize(w, "cpu")
            self.qh, self.kh, self.vh = q.numpy(), k.numpy(), v.numpy()
            q, k, v = q.to(dev), k.to(dev), v.to(dev)
        self.q, self.k, self.v = q, k, v
        self.table = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
        self.lens = torch.from_numpy(np.ascontiguousarray(w.seq_lens.astype(np.int32))).to(dev)
        self.window = None
        if w.mode == "span":
            self.window = torch.from_numpy(np.ascontiguousarray(w.window.astype(np.int32))).to(dev)
        elif w.mode == "kv_map":
            self.window = torch.from_numpy(np.ascontiguousarray(w.kv_map.astype(np.int32))).to(dev)
        if w.kind == "prefill":
            self.cu_q = torch.from_numpy(w.cu_q.astype(np.int32)).to(dev)
            self.q_pos = torch.from_numpy(w.q_pos.astype(np.int32)).to(dev)

    def decode(self, **kw):
        return pkv.paged_attn_decode(self.q, self.k, self.v, self.table, self.lens, self.w.scale,
                                     mode=self.w.mode, window=self.window, **kw)

    def prefill(self, **kw):
        w = self.w
        max_q = int(np.max(np.diff(w.cu_q)))
        return pkv.paged_attn_prefill_window(self.q, self.cu_q, self.q_pos, self.k, self.v, self.table,
                                             self.lens, w.scale, max_q, mode=w.mode, window=self.window, **kw)

    def oracle(self, seqs=None):
        w = self.w
        if self.kh is not None:
            return oracle.paged_attention(self.qh, w.q_seq(), w.query_pos(), self.kh, self.vh, w.k_fmt, w.v_fmt,
                                          w.block_table, w.seq_lens, w.block_size, w.n_kv_heads, w.head_dim,
                                          w.scale, w.mode, w.window, w.kv_map, seqs)
        # large pools: copy only the blocks the sampled sequences reference
        sub, kh, vh = wgen.host_subset(w, seqs, self.k, self.v)
        qrows = np.concatenate([np.nonzero(w.q_seq() == s)[0] for s in seqs])
        qh = self.q[qrows].cpu().numpy()
        o, l = oracle.paged_attention(qh, sub.q_seq(), sub.query_pos(), kh, vh, w.k_fmt, w.v_fmt,
                                      sub.block_table, sub.seq_lens, w.block_size, w.n_kv_heads, w.head_dim,
                                      w.scale, sub.mode, sub.window, sub.kv_map)
        return o, l, qrows


def compare(out, lse, ref_out, ref_lse, tol, what=""):
    """Max-abs check of out and lse (lse compared where finite; -inf must
    match exactly)."""
    out = np.asarray(out, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    assert np.all(np.isfinite(out)), f"{what}: non-finite output"
    err = float(np.max(np.abs(out - ref_out))) if out.size else 0.0
    fin = np.isfinite(ref_lse)
    assert np.array_equal(fin, np.isfinite(lse)), f"{what}: lse finiteness differs"
    lerr = float(np.max(np.abs(lse[fin] - ref_lse[fin]))) if fin.any() else 0.0
    log(f"  {what}: max|out-oracle| = {err:.3g}, max|lse-oracle| = {lerr:.3g} (tol {tol:g})")
    assert err <= tol, f"{what}: out error {err} > {tol}"
    assert lerr <= tol, f"{what}: lse error {lerr} > {tol}"
    return err


def default_scale(hd):
    return 1.0 / math.sqrt(hd)
