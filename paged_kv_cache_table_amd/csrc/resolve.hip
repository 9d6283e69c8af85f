// Debug export of the block-table/window resolver: materializes, for each
// query and each candidate of its window enumeration, the pool row read (or
// -1), with the same geometry helpers the attention kernels use.
#include "pkv_internal.hpp"

namespace pkv {

__global__ void resolve_kernel(AttnArgs a, int n_cand, int32_t* rows_out) {
  const int64_t j = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_cand) return;
  const int bs = a.block_size;
  int s = -1;
  int64_t qp = 0;
  if (a.cu_q == nullptr) {
    s = (int)j;
  } else {
    // sequence whose query range [cu_q[s], cu_q[s+1]) holds row j
    int lo = 0, hi = a.n_seqs;  // find the last s with cu_q[s] <= j
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (a.cu_q[mid] <= j) lo = mid; else hi = mid - 1;
    }
    s = lo;
    if (s >= a.n_seqs || a.cu_q[s] > j || j >= a.cu_q[s + 1]) s = -1;
  }
  int32_t row = -1;
  if (s >= 0) {
    const int32_t L = clamp_seq_len(a.seq_lens[s], a.max_blocks, bs);
    qp = a.cu_q == nullptr ? (int64_t)L - 1 : (int64_t)a.q_pos[j];
    const int64_t limit = qp + 1 < L ? qp + 1 : L;
    bool have = false;
    int64_t t = 0;
    if (a.mode == PKV_WIN_CAUSAL) {
      have = i < L;
      t = i;
    } else if (a.mode == PKV_WIN_SPAN) {
      const int64_t lo = a.window[2 * s], hi = a.window[2 * s + 1];
      have = i < hi - lo;
      t = lo + i;
    } else {
      int64_t k = i;
      for (int r = 0; r < a.n_runs && !have; ++r) {
        const int32_t* w = a.window + ((int64_t)s * a.n_runs + r) * 2;
        const int64_t n = w[1];
        if (n <= 0) continue;
        if (k < n) {
          have = true;
          t = (int64_t)w[0] + k;
        } else {
          k -= n;
        }
      }
    }
    if (have && t >= 0 && t < limit) {
      const int32_t id = block_id(a, s, (int32_t)(t / bs));
      if (id >= 0) row = id * bs + (int32_t)(t % bs);
    }
  }
  rows_out[j * n_cand + i] = row;
}

hipError_t launch_resolve(const AttnArgs& a, int bs, int n_cand, int32_t* rows_out, hipStream_t st) {
  (void)bs;
  if (n_cand <= 0 || a.n_q_total <= 0) return hipSuccess;
  const dim3 grid((n_cand + 255) / 256, a.n_q_total);
  hipLaunchKernelGGL(resolve_kernel, grid, dim3(256), 0, st, a, n_cand, rows_out);
  return hipGetLastError();
}

}  // namespace pkv
