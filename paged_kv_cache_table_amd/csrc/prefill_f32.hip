// Windowed prefill for f32 queries (K f32 or q8_0, V f32) through the
// split-K decode kernels: the matrix cores take f16 operands, which cannot
// hold f32 inputs to the 1e-5 these formats are held to, while the decode
// kernels compute every product and sum in f32.  Query j of sequence s sees
// W_s ∩ [0, min(seq_len_s, q_pos_j + 1)) minus holes ("KV Cache Design —
// cells, format, sessions", section 1: windowed prefill, causal inside the
// window), which is exactly what a decode query sees for a sequence of
// length min(seq_len_s, q_pos_j + 1) that shares s's block table and
// window.  So each query becomes one virtual decode sequence: a first pass
// gives it s's table row and window and that length; the decode passes
// compute it; a last pass copies the rows that prefill computes (the first
// max_q_per_seq queries of each sequence) to the caller's out and lse.
#include "pkv_internal.hpp"

namespace pkv {

// Grid (n_q_total), 256 threads: query j's sequence (the s with cu_q[s] <=
// j < cu_q[s + 1], by binary search; every index stays inside the arrays
// whatever cu_q holds), whether prefill computes it (its rank in the
// sequence is below max_q after the same clamping the prefill kernel
// applies), its length, table row and window.
__global__ __launch_bounds__(256) void prefill_expand_kernel(AttnArgs a, int32_t* vtable, int32_t* vlens,
                                                             int32_t* vwin, int32_t win_ints,
                                                             uint8_t* computed) {
  const int32_t j = blockIdx.x;
  const int t = threadIdx.x;
  int32_t lo = 0, hi = a.n_seqs - 1;  // last s with cu_q[s] <= j
  while (lo < hi) {
    const int32_t mid = (lo + hi + 1) >> 1;
    if (a.cu_q[mid] <= j) lo = mid;
    else hi = mid - 1;
  }
  const int s = lo;
  int q0 = a.cu_q[s], q1 = a.cu_q[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > a.n_q_total ? a.n_q_total : q0);
  q1 = q1 < q0 ? q0 : (q1 > a.n_q_total ? a.n_q_total : q1);
  if (q1 > q0 + a.max_q) q1 = q0 + a.max_q;
  const bool on = j >= q0 && j < q1;
  if (t == 0) {
    computed[j] = on ? 1 : 0;
    int64_t len = 0;
    if (on) {
      len = (int64_t)a.q_pos[j] + 1;
      const int32_t L = clamp_seq_len(a.seq_lens[s], a.max_blocks, a.block_size);
      if (len > L) len = L;
      if (len < 0) len = 0;
    }
    vlens[j] = (int32_t)len;
  }
  if (!on) return;
  const int32_t* src = a.table + (int64_t)s * a.max_blocks;
  int32_t* dst = vtable + (int64_t)j * a.max_blocks;
  for (int32_t b = t; b < a.max_blocks; b += 256) dst[b] = src[b];
  if (win_ints && t < win_ints) vwin[(int64_t)j * win_ints + t] = a.window[(int64_t)s * win_ints + t];
}

// Grid (ceil(n_q_total * n_q_heads * head_dim / 1024)), 256 threads, four
// floats each: the computed rows of the decode output to out (and lse).
__global__ __launch_bounds__(256) void prefill_copy_rows_kernel(const float* tmp_out, const float* tmp_lse,
                                                                const uint8_t* computed, float* out, float* lse,
                                                                int64_t row_floats, int64_t n_rows, int32_t hq) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;  // float index; row_floats % 4 == 0
  if (i >= n_rows * row_floats) return;
  const int64_t j = i / row_floats;
  if (!computed[j]) return;
  *(float4*)(out + i) = *(const float4*)(tmp_out + i);
  const int64_t r = i - j * row_floats;  // offset inside the query's row
  if (lse && r % (row_floats / hq) == 0) {
    const int64_t h = r / (row_floats / hq);
    lse[j * hq + h] = tmp_lse[j * hq + h];
  }
}

hipError_t launch_prefill_expand(const AttnArgs& a, int32_t* vtable, int32_t* vlens, int32_t* vwin,
                                 int32_t win_ints, uint8_t* computed, hipStream_t st) {
  if (a.n_q_total <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_expand_kernel, dim3((unsigned)a.n_q_total), dim3(256), 0, st, a, vtable, vlens, vwin,
                     win_ints, computed);
  return hipGetLastError();
}

hipError_t launch_prefill_copy_rows(const float* tmp_out, const float* tmp_lse, const uint8_t* computed,
                                    float* out, float* lse, int64_t n_rows, int32_t hq, int32_t hd,
                                    hipStream_t st) {
  const int64_t row_floats = (int64_t)hq * hd;
  const int64_t blocks = (n_rows * row_floats / 4 + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_copy_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, tmp_out, tmp_lse, computed,
                     out, lse, row_floats, n_rows, hq);
  return hipGetLastError();
}

}  // namespace pkv
