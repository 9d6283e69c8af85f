// Windowed prefill on the matrix cores (gfx950 v_mfma_f32_16x16x32_f16).
//
// What it computes ("KV Cache Design — cells, format, sessions", section 1:
// windows as causal positions, one [lo, hi) range or a map of (cell, len)
// runs, and the fast multi-query windowed prefill; "Tiered KV cache —
// architecture", section "The paged-attention block model": positions read
// through the block table, holes score -inf): for every query j of sequence
// s and q head h, softmax attention over the window positions t of s with
// t < min(seq_len_s, q_pos_j + 1), t not in a hole.
//
// A workgroup (4 waves) takes one kv head and a block of consecutive queries
// of one sequence: 128 rows = (query, q head in the GQA group) pairs, 32 per
// wave in two 16-row tiles.  The window is walked in tiles of 32 positions
// (a tile never crosses a run; runs are not block-aligned, so every position
// resolves its own block).  Each tile is staged in LDS once for the four
// waves: K row-major (f16, or q8_0 codes widened to f16 — exact — plus one
// f32 scale per (position, 32-wide block)), V transposed.  Per tile and row
// tile the wave computes S^T = K Q^T (16x16x32 MFMAs over head_dim), so each
// lane holds eight scores of one row: the running max/sum of that row live
// in the lane and P (f16) is already laid out as the B operand of
// O^T = V^T P^T.  For q8_0 K each 32-wide head_dim block is one MFMA whose
// result is scaled by that position's block scale before it is added
// (the dequantized value scale * code is never rounded to f16).
// Positions outside the run, in a hole or past a row's causal limit get
// score -inf by selection; their staged K/V are zeros.
#include "pkv_internal.hpp"

namespace pkv {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kTileT = 32;      // window positions per tile
constexpr int kPWaves = 4;      // waves per workgroup
constexpr int kRowTiles = 2;    // 16-row tiles per wave
constexpr int kRowsWG = kPWaves * kRowTiles * 16;
constexpr float kEmptyMax = -1e30f;

template <int HD>
struct PrefillSmem {
  _Float16 k[kTileT][HD + 8];      // K tile [position][head_dim]; +8 spreads LDS banks
  _Float16 vt[HD][kTileT + 8];     // V tile transposed [head_dim][position]
  float kscale[kTileT][HD / 32];   // q8_0 block scales
  int32_t id[kTileT];              // physical block of each position, -1 = not visible
  int32_t lim_max;                 // largest causal limit of the workgroup's rows
};

__device__ __forceinline__ float4_t mfma16x16x32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

template <int HD, int BS, int G, bool KQ8>
__global__ __launch_bounds__(256) void prefill_kernel(AttnArgs a) {
  constexpr int KS = HD / 32;   // MFMA k-steps over head_dim
  constexpr int DT = HD / 16;   // 16-wide head_dim tiles of the output
  constexpr int QPB = kRowsWG / G;  // queries per workgroup
  constexpr int CH = HD / 8;        // 16-byte chunks per f16 head row
  __shared__ PrefillSmem<HD> sm;

  const int kvh = blockIdx.x, qb = blockIdx.y, s = blockIdx.z;
  const int t = threadIdx.x, w = t >> 6, l = t & 63, g = l >> 4, n16 = l & 15;
  int q0 = a.cu_q[s], q1 = a.cu_q[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > a.n_q_total ? a.n_q_total : q0);
  q1 = q1 < q0 ? q0 : (q1 > a.n_q_total ? a.n_q_total : q1);
  if (q1 > q0 + a.max_q) q1 = q0 + a.max_q;  // queries past max_q_per_seq are not computed
  const int j0 = q0 + qb * QPB;
  if (j0 >= q1) return;  // whole workgroup: no queries here
  const int j1 = j0 + QPB < q1 ? j0 + QPB : q1;
  const int32_t L = clamp_seq_len(a.seq_lens[s], a.max_blocks, BS);

  // ---- rows of this lane: row tile rt covers rows w*32 + rt*16 + n16
  int jq[kRowTiles], hq[kRowTiles];
  int32_t lim[kRowTiles];
  half8_t qf[kRowTiles][KS];
  if (t == 0) sm.lim_max = 0;
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int rr = w * 32 + rt * 16 + n16;
    jq[rt] = j0 + rr / G;
    hq[rt] = rr % G;
    const bool ok = rr < QPB * G && jq[rt] < j1;
    int64_t lm = 0;
    if (ok) {
      lm = (int64_t)a.q_pos[jq[rt]] + 1;
      if (lm > L) lm = L;
      if (lm < 0) lm = 0;
    }
    lim[rt] = (int32_t)lm;
    const _Float16* qrow = (const _Float16*)a.q + ((int64_t)(ok ? jq[rt] : 0) * a.n_q_heads + kvh * G + hq[rt]) * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      half8_t v = {};
      if (ok) v = *(const half8_t*)(qrow + ks * 32 + g * 8);
      qf[rt][ks] = v;
    }
    if (ok) atomicMax(&sm.lim_max, lim[rt]);
  }
  __syncthreads();
  const int32_t lim_max = sm.lim_max;

  float m[kRowTiles], lsum[kRowTiles];
  float4_t o[kRowTiles][DT];
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    m[rt] = kEmptyMax;
    lsum[rt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  const unsigned char* kbase = a.k_pool + (int64_t)kvh * BS * a.k_seg_bytes;
  const unsigned char* vbase = a.v_pool + (int64_t)kvh * BS * a.v_seg_bytes;
  const bool count_bad = kvh == 0 && qb == 0;

  for (int r = 0; r < a.n_runs; ++r) {
    int32_t ra, rb;
    run_range(a, s, r, L, ra, rb);
    if (rb > lim_max) rb = lim_max;  // no row of this workgroup sees past it
    for (int32_t t0 = ra; t0 < rb; t0 += kTileT) {
      // ---- stage the tile
      __syncthreads();  // previous tile fully consumed
      if (t < kTileT) {
        const int32_t pos = t0 + t;
        int32_t id = -1;
        if (pos < rb) id = block_id(a, s, pos / BS, count_bad);
        sm.id[t] = id;
      }
      __syncthreads();
      // V (f16): 16-byte chunks, written transposed
      for (int c = t; c < kTileT * CH; c += 256) {
        const int p = c / CH, ch = c - p * CH;
        const int32_t id = sm.id[p];
        uint4 x = {0u, 0u, 0u, 0u};
        if (id >= 0) {
          const int32_t pos = t0 + p;
          x = *(const uint4*)(vbase + (int64_t)id * a.v_block_bytes + (int64_t)(pos % BS) * a.v_seg_bytes + ch * 16);
        }
        const _Float16* hx = (const _Float16*)&x;
#pragma unroll
        for (int i = 0; i < 8; ++i) sm.vt[ch * 8 + i][p] = hx[i];
      }
      if constexpr (!KQ8) {
        for (int c = t; c < kTileT * CH; c += 256) {
          const int p = c / CH, ch = c - p * CH;
          const int32_t id = sm.id[p];
          uint4 x = {0u, 0u, 0u, 0u};
          if (id >= 0) {
            const int32_t pos = t0 + p;
            x = *(const uint4*)(kbase + (int64_t)id * a.k_block_bytes + (int64_t)(pos % BS) * a.k_seg_bytes + ch * 16);
          }
          *(uint4*)&sm.k[p][ch * 8] = x;
        }
      } else {
        // one thread per (position, q8_0 block): 34 bytes at a 2-byte aligned
        // offset, read as the nine enclosing dwords of the segment
        for (int c = t; c < kTileT * KS; c += 256) {
          const int p = c / KS, b = c - p * KS;
          const int32_t id = sm.id[p];
          uint32_t wd[9];
#pragma unroll
          for (int i = 0; i < 9; ++i) wd[i] = 0u;
          int sh = 0;
          if (id >= 0) {
            const int32_t pos = t0 + p;
            const int off = 34 * b;
            sh = off & 3;
            const uint32_t* src = (const uint32_t*)(kbase + (int64_t)id * a.k_block_bytes +
                                                    (int64_t)(pos % BS) * a.k_seg_bytes + (off - sh));
#pragma unroll
            for (int i = 0; i < 9; ++i) wd[i] = src[i];
          }
          uint32_t al[9];  // bytes [off, off + 36) of the segment
#pragma unroll
          for (int i = 0; i < 8; ++i) al[i] = __builtin_amdgcn_alignbyte(wd[i + 1], wd[i], sh);
          al[8] = wd[8] >> (8 * sh);
          const float scale = (float)__builtin_bit_cast(_Float16, (unsigned short)(al[0] & 0xFFFFu));
          sm.kscale[p][b] = scale;
          // codes: bytes 2..33 of the block
          _Float16 hv[32];
#pragma unroll
          for (int i = 0; i < 32; ++i) {
            const int byte = 2 + i;
            const uint32_t word = al[byte >> 2];
            hv[i] = (_Float16)(float)(int)(int8_t)(word >> (8 * (byte & 3)));
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) *(half8_t*)&sm.k[p][b * 32 + i * 8] = *(half8_t*)&hv[i * 8];
        }
      }
      __syncthreads();

      // ---- S^T = K Q^T: lane holds positions st*16 + 4g + i of row n16
      float sc[kRowTiles][8];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        float4_t acc[kRowTiles];
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) acc[rt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const half8_t af = *(const half8_t*)&sm.k[st * 16 + n16][ks * 32 + g * 8];
          if constexpr (!KQ8) {
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) acc[rt] = mfma16x16x32(af, qf[rt][ks], acc[rt]);
          } else {
            float scl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) scl[i] = sm.kscale[st * 16 + 4 * g + i][ks];
#pragma unroll
            for (int rt = 0; rt < kRowTiles; ++rt) {
              const float4_t part = mfma16x16x32(af, qf[rt][ks], float4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[rt][i] = fmaf(part[i], scl[i], acc[rt][i]);
            }
          }
        }
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int p = st * 16 + 4 * g + i;
            const bool vis = sm.id[p] >= 0 && t0 + p < lim[rt];
            sc[rt][st * 4 + i] = vis ? acc[rt][i] * a.score_mul : -INFINITY;
          }
      }

      // ---- online softmax per row (the four lane groups hold the same row)
      half8_t pf[kRowTiles];
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) {
        float mx = sc[rt][0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sc[rt][i]);
        mx = fmaxf(mx, shfl_xor(mx, 16));
        mx = fmaxf(mx, shfl_xor(mx, 32));
        const float mn = fmaxf(m[rt], mx);
        const float alpha = fast_exp2(m[rt] - mn);
        if (__builtin_amdgcn_ballot_w64(mn > m[rt])) {
          lsum[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= alpha;
        }
        m[rt] = mn;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = fast_exp2(sc[rt][i] - mn);
          lsum[rt] += p;
          pf[rt][i] = (_Float16)p;
        }
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 16 + n16;
        const half4_t lo4 = *(const half4_t*)&sm.vt[d][4 * g];
        const half4_t hi4 = *(const half4_t*)&sm.vt[d][16 + 4 * g];
        const half8_t vf = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) o[rt][dt] = mfma16x16x32(vf, pf[rt], o[rt][dt]);
      }
    }
  }

  // ---- finish: sum the row's lane groups, normalise, write
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    float ls = lsum[rt];
    ls += shfl_xor(ls, 16);
    ls += shfl_xor(ls, 32);
    const int rr = w * 32 + rt * 16 + n16;
    const bool ok = rr < QPB * G && jq[rt] < j1;
    if (!ok) continue;
    const bool empty = m[rt] == kEmptyMax;
    const float inv = empty ? 0.f : 1.f / ls;
    float* orow = a.out + ((int64_t)jq[rt] * a.n_q_heads + kvh * G + hq[rt]) * HD;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const float4_t v = o[rt][dt] * inv;
      *(float4*)(orow + dt * 16 + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
    }
    if (a.lse && g == 0)
      a.lse[(int64_t)jq[rt] * a.n_q_heads + kvh * G + hq[rt]] =
          empty ? -INFINITY : (m[rt] + __builtin_amdgcn_logf(ls)) * kLn2;
  }
}

size_t prefill_workspace(const AttnArgs& a, int combo, int hd, int bs, int g, bool* found) {
  (void)hd; (void)bs; (void)g;
  *found = combo == kComboF16 || combo == kComboQ8H;
  // no partials: only the checked-mode error word
  return (*found && (a.flags & PKV_FLAG_CHECKED)) ? 256 : 0;
}

hipError_t launch_prefill(const AttnArgs& a, int combo, int hd, int bs, int g, hipStream_t st,
                          bool* found) {
  *found = false;
  if (combo != kComboF16 && combo != kComboQ8H) return hipSuccess;
  const bool q8 = combo == kComboQ8H;
#define PKV_PCASE(HD, BS, G)                                                                     \
  if (hd == HD && bs == BS && g == G) {                                                          \
    const dim3 grid(a.n_kv_heads, (a.max_q + kRowsWG / G - 1) / (kRowsWG / G), a.n_seqs);        \
    if (q8)                                                                                      \
      hipLaunchKernelGGL((prefill_kernel<HD, BS, G, true>), grid, dim3(256), 0, st, a);          \
    else                                                                                         \
      hipLaunchKernelGGL((prefill_kernel<HD, BS, G, false>), grid, dim3(256), 0, st, a);         \
    *found = true;                                                                               \
    return hipGetLastError();                                                                    \
  }
#define PKV_PCASES_G(HD, BS) PKV_PCASE(HD, BS, 1) PKV_PCASE(HD, BS, 2) PKV_PCASE(HD, BS, 3) PKV_PCASE(HD, BS, 4) PKV_PCASE(HD, BS, 8)
  PKV_PCASES_G(64, 16)
  PKV_PCASES_G(128, 16)
  PKV_PCASES_G(256, 16)
  PKV_PCASES_G(128, 32)
#undef PKV_PCASES_G
#undef PKV_PCASE
  return hipSuccess;
}

}  // namespace pkv
