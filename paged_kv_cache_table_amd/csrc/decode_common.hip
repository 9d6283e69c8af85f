// Decode dispatch over format combinations, the plan pass and the merge pass.
#include "decode_impl.hpp"

namespace pkv {

// Exclusive prefix sums over the workgroup of three counters per thread,
// and their totals (1024 threads = 16 waves).
constexpr int kPlanThreads = 1024;
__device__ void block_scan3(const uint32_t (&v)[3], uint32_t (&excl)[3], uint32_t (&tot)[3],
                            uint32_t (*wsum)[kPlanThreads / 64]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t inc[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    inc[c] = v[c];
    for (int dlt = 1; dlt < 64; dlt <<= 1) {
      const uint32_t y = __shfl_up(inc[c], dlt);
      if (lane >= dlt) inc[c] += y;
    }
    if (lane == 63) wsum[c][w] = inc[c];
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    uint32_t before = 0, all = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) {
      const uint32_t x = wsum[c][i];
      if (i < w) before += x;
      all += x;
    }
    excl[c] = before + inc[c] - v[c];
    tot[c] = all;
  }
}

// Active slots of a run [rl, rh) and how many of them it covers completely.
__device__ inline void run_slots(int32_t rl, int32_t rh, int32_t split, uint32_t& nact, uint32_t& nfull) {
  nact = rh > rl ? (uint32_t)((rh - 1) / split - rl / split + 1) : 0u;
  nfull = (uint32_t)full_slots(rl, rh, split);
}

// The work list of a decode call.  A sequence's items are its non-empty
// split slots; the last fine_per_seq slots that a run covers completely
// are cut into nsub pieces of fine_tokens positions.  Which slots exist and
// which are cut depends only on the sequence's own length and window (the
// merge derives the same), so the list order is chosen for speed alone:
// whole full slots, then partial slots, then the pieces, each group in
// sequence order.  One workgroup.  First the sequences, 1024 at a time: a
// block scan of their counts gives each its place in each group (seqinfo;
// kept in LDS, with the lengths, when there are at most 1024 sequences).
// Then every (sequence, slot) pair is placed by its own thread, its rank
// among the sequence's slots of its kind counted from the runs before it.
__global__ __launch_bounds__(kPlanThreads) void decode_plan_kernel(AttnArgs a) {
  __shared__ uint32_t wsum[3][kPlanThreads / 64];
  __shared__ uint32_t carry[3];
  __shared__ uint4 s_info[kPlanThreads];
  __shared__ int32_t s_len[kPlanThreads];
  const bool in_lds = a.n_seqs <= kPlanThreads;
  const int t = threadIdx.x;
  const int32_t split = a.split;
  const uint32_t fps = (uint32_t)a.fine_per_seq;
  if (t < 3) carry[t] = 0u;
  __syncthreads();
  for (int c0 = 0; c0 < a.n_seqs; c0 += kPlanThreads) {
    const int s = c0 + t;
    uint32_t cnt[3] = {0u, 0u, 0u}, first_cut = 0u;
    if (s < a.n_seqs) {
      const int32_t L = clamp_seq_len(a.seq_lens[s], a.max_blocks, a.block_size);
      if (in_lds) s_len[t] = L;
      uint32_t nact = 0, nfull = 0;
      for (int r = 0; r < a.n_runs; ++r) {
        int32_t rl, rh;
        run_range(a, s, r, L, rl, rh);
        uint32_t na, nf;
        run_slots(rl, rh, split, na, nf);
        nact += na;
        nfull += nf;
      }
      const uint32_t ncut = nfull < fps ? nfull : fps;
      first_cut = nfull - ncut;
      cnt[0] = first_cut;
      cnt[1] = nact - nfull;
      cnt[2] = ncut;
    }
    uint32_t base[3], total[3];
    block_scan3(cnt, base, total, wsum);
    if (s < a.n_seqs) {
      const uint4 info = make_uint4(carry[0] + base[0], carry[1] + base[1], carry[2] + base[2], first_cut);
      if (in_lds) s_info[t] = info;
      else a.seqinfo[s] = info;
    }
    __syncthreads();
    if (t < 3) carry[t] += total[t];
    __syncthreads();
  }
  const uint32_t n_whole = carry[0], n_part = carry[1], n_cut = carry[2];
  if (t == 0) a.hdr[0] = (n_whole + n_part + n_cut * (uint32_t)a.nsub) * (uint32_t)a.n_kv_heads;
  uint4* items = const_cast<uint4*>(a.items);
  const int64_t sps = (int64_t)a.n_runs * a.nspl;
  const int64_t n_pairs = (int64_t)a.n_seqs * sps;
  for (int64_t idx = t; idx < n_pairs; idx += kPlanThreads) {
    const int s = (int)(idx / sps);
    const int slot = (int)(idx - (int64_t)s * sps);
    const int r = slot / a.nspl, k = slot - r * a.nspl;
    const int32_t L = in_lds ? s_len[s] : clamp_seq_len(a.seq_lens[s], a.max_blocks, a.block_size);
    int32_t rl, rh;
    run_range(a, s, r, L, rl, rh);
    const int64_t w0 = (int64_t)k * split;
    const int32_t lo = (int32_t)(rl > w0 ? rl : w0);
    const int32_t hi = (int32_t)(rh < w0 + split ? rh : w0 + split);
    if (lo >= hi) continue;
    uint32_t full_before = 0, part_before = 0;  // in the runs before r
    for (int r2 = 0; r2 < r; ++r2) {
      int32_t l2, h2;
      run_range(a, s, r2, L, l2, h2);
      uint32_t na, nf;
      run_slots(l2, h2, split, na, nf);
      full_before += nf;
      part_before += na - nf;
    }
    const int32_t k0 = rl / split;
    const int32_t kf0 = (int32_t)(((int64_t)rl + split - 1) / split), kf1 = rh / split;
    const uint4 info = in_lds ? s_info[s] : a.seqinfo[s];
    const uint32_t first_cut = info.w;
    const int64_t row0 = (int64_t)s * a.rows_per_seq + slot;
    if (hi - lo != split) {
      // a partial slot is the run's first active slot or its last
      const bool k0_partial = k0 < kf0 || k0 >= kf1;
      const uint32_t rank = part_before + (k == k0 ? 0u : (k0_partial ? 1u : 0u));
      const int32_t full_here = k < kf0 ? 0 : (k - kf0 < kf1 - kf0 ? k - kf0 : kf1 - kf0);
      const uint32_t fb = full_before + (uint32_t)(full_here > 0 ? full_here : 0);
      const uint32_t cut_before = fb > first_cut ? fb - first_cut : 0u;
      items[n_whole + info.y + rank] =
          make_uint4((uint32_t)s, (uint32_t)lo, (uint32_t)hi, (uint32_t)(row0 + (int64_t)cut_before * (a.nsub - 1)));
    } else {
      const uint32_t fi = full_before + (uint32_t)(k - kf0);
      if (fi < first_cut) {
        items[info.x + fi] = make_uint4((uint32_t)s, (uint32_t)lo, (uint32_t)hi, (uint32_t)row0);
      } else {
        const uint32_t j = fi - first_cut;
        const uint32_t pos = n_whole + n_part + (info.z + j) * (uint32_t)a.nsub;
        for (int p = 0; p < a.nsub; ++p) {
          const int32_t plo = lo + p * a.fine_tokens;
          const int32_t phi = plo + a.fine_tokens < hi ? plo + a.fine_tokens : hi;
          items[pos + p] = make_uint4((uint32_t)s, (uint32_t)plo, (uint32_t)phi,
                                      (uint32_t)(row0 + (int64_t)j * (a.nsub - 1) + p));
        }
      }
    }
  }
}

hipError_t launch_decode_plan(const AttnArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_decode_split_f32(const AttnArgs&, int, int, int, int64_t, hipStream_t, bool*);
hipError_t launch_decode_split_f16(const AttnArgs&, int, int, int, int64_t, hipStream_t, bool*);
hipError_t launch_decode_split_q8h(const AttnArgs&, int, int, int, int64_t, hipStream_t, bool*);
hipError_t launch_decode_split_q8f(const AttnArgs&, int, int, int, int64_t, hipStream_t, bool*);

hipError_t launch_decode_split(const AttnArgs& a, int combo, int hd, int bs, int g,
                               int64_t max_units, hipStream_t st, bool* found) {
  switch (combo) {
    case kComboF32: return launch_decode_split_f32(a, hd, bs, g, max_units, st, found);
    case kComboF16: return launch_decode_split_f16(a, hd, bs, g, max_units, st, found);
    case kComboQ8H: return launch_decode_split_q8h(a, hd, bs, g, max_units, st, found);
    case kComboQ8F: return launch_decode_split_q8f(a, hd, bs, g, max_units, st, found);
    default: *found = false; return hipSuccess;
  }
}

hipError_t launch_decode_merge(const AttnArgs& a, int hd, hipStream_t st) {
  const dim3 grid((unsigned)((a.n_q_heads * hd + 255) / 256), a.n_seqs);
  const bool small = (int64_t)grid.x * grid.y < 512;  // eight waves share each workgroup's rows
#define PKV_MERGE(HD)                                                                   \
  if (small) hipLaunchKernelGGL((decode_merge_kernel<HD, 8>), grid, dim3(512), 0, st, a); \
  else hipLaunchKernelGGL((decode_merge_kernel<HD, 4>), grid, dim3(256), 0, st, a);
  switch (hd) {
    case 64: PKV_MERGE(64) break;
    case 128: PKV_MERGE(128) break;
    case 256: PKV_MERGE(256) break;
    default: return hipErrorInvalidValue;
  }
#undef PKV_MERGE
  return hipGetLastError();
}

__global__ void zero_words_kernel(int32_t* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_words(int32_t* p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace pkv
