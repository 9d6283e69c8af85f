// Split-K paged decode for gfx950.
//
// What it computes ("Tiered KV cache — architecture", section "The
// paged-attention block model"; "KV cache" (sipllm), section "Problem"):
// for each sequence s and q head h, softmax attention of its one query over
// the positions of its window that lie in [0, seq_len) and are not in a
// hole, reading K/V rows through the block table.
//
// Work item = one wave = (sequence, kv head, split slot).  A split slot is
// the intersection of one window run with an aligned range of `split`
// positions, so its blocks are at most 64 and their ids fit one register.
// Lane layout: each token row of one kv head is spread over LPT = HD/16
// lanes (16 elements per lane), a pass covers TPP = 64/LPT tokens, and a
// 16- or 32-token block takes BS/TPP passes.  The g query heads that share
// the kv head are all computed from the same K/V registers (GQA reads every
// K/V byte once).  Each lane keeps its own running output for its tokens;
// the running max is kept per head for the whole wave, so the end of the
// split only sums lanes (no rescaling), then writes (max, sum, output) for
// the merge.  Scores are kept in the log2 domain (scale * log2 e folded in).
//
// Holes and positions outside [lo, hi) are masked by selection (never by a
// multiply), so NaN in rows that must not be read cannot leak in.
#pragma once

#include "pkv_internal.hpp"

namespace pkv {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

// --------------------------------------------------------------------------
// K paths: lane `sub` of a token computes a partial q.k over its elements.

// q f16, K f16: elements are the 16-byte chunks sub and sub+LPT of the head
// row (so one instruction reads LPT*16 contiguous bytes of each row); the
// dot uses the packed f16 dot with f32 accumulation.
template <int HD, int G>
struct KPathF16 {
  static constexpr int LPT = HD / 16;
  static constexpr int KW = 8;
  static constexpr int64_t kHeadBytes = HD * 2;
  uint32_t q[G][8];

  __device__ void load_q(const void* qbase, int sub) {
    const _Float16* qp = (const _Float16*)qbase;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4* p = (const uint4*)(qp + h * HD);
      uint4 x = p[sub], y = p[sub + LPT];
      q[h][0] = x.x; q[h][1] = x.y; q[h][2] = x.z; q[h][3] = x.w;
      q[h][4] = y.x; q[h][5] = y.y; q[h][6] = y.z; q[h][7] = y.w;
    }
  }
  __device__ __forceinline__ void load_k(const unsigned char* hp, int sub, uint32_t (&w)[KW]) const {
    const uint4* p = (const uint4*)hp;
    uint4 x = p[sub], y = p[sub + LPT];
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
  }
  __device__ __forceinline__ void dot(const uint32_t (&w)[KW], float (&s)[G]) const {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, q[h][i]),
                                     __builtin_bit_cast(half2_t, w[i]), acc, false);
      s[h] = acc;
    }
  }
};

// q f32, K f32: chunks sub + LPT*c (c < 4) of four floats each.
template <int HD, int G>
struct KPathF32 {
  static constexpr int LPT = HD / 16;
  static constexpr int KW = 16;
  static constexpr int64_t kHeadBytes = HD * 4;
  float q[G][16];

  __device__ void load_q(const void* qbase, int sub) {
    const float* qp = (const float*)qbase;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float4* p = (const float4*)(qp + h * HD);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        float4 x = p[sub + LPT * c];
        q[h][4 * c + 0] = x.x; q[h][4 * c + 1] = x.y; q[h][4 * c + 2] = x.z; q[h][4 * c + 3] = x.w;
      }
    }
  }
  __device__ __forceinline__ void load_k(const unsigned char* hp, int sub, uint32_t (&w)[KW]) const {
    const uint4* p = (const uint4*)hp;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 x = p[sub + LPT * c];
      w[4 * c + 0] = x.x; w[4 * c + 1] = x.y; w[4 * c + 2] = x.z; w[4 * c + 3] = x.w;
    }
  }
  __device__ __forceinline__ void dot(const uint32_t (&w)[KW], float (&s)[G]) const {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc = fmaf(q[h][i], __builtin_bit_cast(float, w[i]), acc);
      s[h] = acc;
    }
  }
};

// K q8_0 (q f16 or f32): lane `sub` owns elements [16 sub, 16 sub + 16), one
// half of q8_0 block b = sub/2.  A block is 34 bytes (f16 scale, 32 int8
// codes) so the codes start 2 bytes off a 4-byte boundary for even b: the
// lane reads the enclosing dwords and shifts.  k = scale * code exactly, and
// q.k over the 16 elements is scale * sum(q * code) in f32.
template <int HD, int G, bool QF32>
struct KPathQ8 {
  static constexpr int LPT = HD / 16;
  static constexpr int KW = 6;  // 5 dwords around the codes, 1 with the scale
  static constexpr int64_t kHeadBytes = HD / 32 * 34;
  float q[G][16];
  int code_off, code_shift, scale_off;
  bool scale_hi;

  __device__ void load_q(const void* qbase, int sub) {
    const int b = sub >> 1, half = sub & 1;
    const int cstart = 34 * b + 2 + 16 * half;
    code_shift = cstart & 3;
    code_off = cstart - code_shift;
    const int sstart = 34 * b;
    scale_hi = (sstart & 3) != 0;
    scale_off = sstart & ~3;
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (QF32)
          q[h][i] = ((const float*)qbase)[h * HD + 16 * sub + i];
        else
          q[h][i] = (float)((const _Float16*)qbase)[h * HD + 16 * sub + i];
      }
    }
  }
  __device__ __forceinline__ void load_k(const unsigned char* hp, int sub, uint32_t (&w)[KW]) const {
    const uint32_t* p = (const uint32_t*)(hp + code_off);
    w[0] = p[0]; w[1] = p[1]; w[2] = p[2]; w[3] = p[3];
    // The fifth dword is only needed (and only inside the head segment) when
    // the codes are misaligned, which never happens in the last block.
    w[4] = code_shift ? p[4] : 0u;
    w[5] = *(const uint32_t*)(hp + scale_off);
  }
  __device__ __forceinline__ void dot(const uint32_t (&w)[KW], float (&s)[G]) const {
    uint32_t c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_alignbyte(w[i + 1], w[i], code_shift);
    const float d = scale_hi ? h2f_hi(w[5]) : h2f_lo(w[5]);
    float kv[16];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int k = 0; k < 4; ++k) kv[4 * i + k] = (float)(int)(int8_t)(c[i] >> (8 * k));
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc = fmaf(q[h][i], kv[i], acc);
      s[h] = d * acc;
    }
  }
};

// --------------------------------------------------------------------------
// V paths: lane `sub` of a token holds 16 of the head's values.

template <int HD>
struct VPathF16 {
  static constexpr int LPT = HD / 16;
  static constexpr int VW = 8;
  static constexpr int64_t kHeadBytes = HD * 2;
  __device__ __forceinline__ static void load(const unsigned char* hp, int sub, uint32_t (&w)[VW]) {
    const uint4* p = (const uint4*)hp;
    uint4 x = p[sub], y = p[sub + LPT];
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
  }
  __device__ __forceinline__ static void to_float(const uint32_t (&w)[VW], float (&f)[16]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f[2 * i] = h2f_lo(w[i]);
      f[2 * i + 1] = h2f_hi(w[i]);
    }
  }
  // element e of lane sub is head dimension d
  __device__ __forceinline__ static int dim(int sub, int e) {
    return e < 8 ? 8 * sub + e : 8 * (sub + LPT) + (e - 8);
  }
  static constexpr int kChunks = 2;  // contiguous runs of 8 floats
  __device__ __forceinline__ static int chunk_dim(int sub, int c) { return 8 * (sub + LPT * c); }
  static constexpr int kChunkLen = 8;
};

template <int HD>
struct VPathF32 {
  static constexpr int LPT = HD / 16;
  static constexpr int VW = 16;
  static constexpr int64_t kHeadBytes = HD * 4;
  __device__ __forceinline__ static void load(const unsigned char* hp, int sub, uint32_t (&w)[VW]) {
    const uint4* p = (const uint4*)hp;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 x = p[sub + LPT * c];
      w[4 * c + 0] = x.x; w[4 * c + 1] = x.y; w[4 * c + 2] = x.z; w[4 * c + 3] = x.w;
    }
  }
  __device__ __forceinline__ static void to_float(const uint32_t (&w)[VW], float (&f)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) f[i] = __builtin_bit_cast(float, w[i]);
  }
  static constexpr int kChunks = 4;
  __device__ __forceinline__ static int chunk_dim(int sub, int c) { return 4 * (sub + LPT * c); }
  static constexpr int kChunkLen = 4;
};

template <int HD, int G, int COMBO>
struct Paths;
template <int HD, int G>
struct Paths<HD, G, kComboF32> { using K = KPathF32<HD, G>; using V = VPathF32<HD>; };
template <int HD, int G>
struct Paths<HD, G, kComboF16> { using K = KPathF16<HD, G>; using V = VPathF16<HD>; };
template <int HD, int G>
struct Paths<HD, G, kComboQ8H> { using K = KPathQ8<HD, G, false>; using V = VPathF16<HD>; };
template <int HD, int G>
struct Paths<HD, G, kComboQ8F> { using K = KPathQ8<HD, G, true>; using V = VPathF32<HD>; };

template <int COMBO>
struct QElem { using T = _Float16; };
template <>
struct QElem<kComboF32> { using T = float; };
template <>
struct QElem<kComboQ8F> { using T = float; };

// --------------------------------------------------------------------------

template <int HD, int BS, int G, int COMBO>
__global__ __launch_bounds__(64) void decode_split_kernel(AttnArgs a) {
  using KP = typename Paths<HD, G, COMBO>::K;
  using VP = typename Paths<HD, G, COMBO>::V;
  using QT = typename QElem<COMBO>::T;
  constexpr int LPT = HD / 16;   // lanes per token row
  constexpr int TPP = 64 / LPT;  // tokens per pass
  static_assert(BS % TPP == 0, "block size must be a multiple of tokens per pass");
  constexpr int NP = BS / TPP;            // passes per block
  constexpr int NPU = NP < 2 ? NP : 2;    // passes per pipelined unit
  constexpr int NU = NP / NPU;            // units per block
  constexpr int KW = KP::KW, VW = VP::VW;

  const int slot = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
  const int lane = threadIdx.x, tok = lane / LPT, sub = lane % LPT;
  const int32_t L = clamp_seq_len(a.seq_lens[s], a.max_blocks, BS);
  int32_t lo, hi;
  split_range(a, s, slot, L, lo, hi);
  if (lo >= hi) return;  // this slot is not a work item

  const int32_t jb0 = lo / BS;
  const int32_t nblk = (hi - 1) / BS - jb0 + 1;  // <= 64 by construction
  int32_t myid = -1;
  if (lane < nblk) myid = block_id(a, s, jb0 + lane, kvh == 0);
  const uint64_t mask = __ballot(myid >= 0);

  KP kp;
  const int64_t qoff = ((int64_t)s * a.n_q_heads + (int64_t)kvh * G) * HD;
  kp.load_q((const QT*)a.q + qoff, sub);

  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
  }

  const unsigned char* kbase = a.k_pool + (int64_t)kvh * KP::kHeadBytes;
  const unsigned char* vbase = a.v_pool + (int64_t)kvh * VP::kHeadBytes;
  const int64_t krb = a.k_row_bytes, vrb = a.v_row_bytes;

  struct Unit {
    uint32_t k[NPU][KW];
    uint32_t v[NPU][VW];
  };
  auto load_unit = [&](Unit& U, int j, int u) {
    const int32_t blk = __builtin_amdgcn_readlane(myid, j);
    const int64_t row0 = (int64_t)blk * BS + u * (NPU * TPP) + tok;
#pragma unroll
    for (int p = 0; p < NPU; ++p) {
      const int64_t row = row0 + p * TPP;
      kp.load_k(kbase + row * krb, sub, U.k[p]);
      VP::load(vbase + row * vrb, sub, U.v[p]);
    }
  };
  auto compute = [&](const Unit& U, int j, int u) {
    const int32_t pos0 = (jb0 + j) * BS + u * (NPU * TPP);
    const bool full = pos0 >= lo && pos0 + NPU * TPP <= hi;
    float sc[NPU][G];
#pragma unroll
    for (int p = 0; p < NPU; ++p) {
      kp.dot(U.k[p], sc[p]);
      const int32_t t = pos0 + p * TPP + tok;
      const bool ok = full || (t >= lo && t < hi);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float x = group_sum<LPT>(sc[p][h]) * a.score_mul;
        sc[p][h] = ok ? x : -INFINITY;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int p = 1; p < NPU; ++p) bm = fmaxf(bm, sc[p][h]);
      bm = uniform(strided_max<LPT>(bm));
      if (bm > m[h]) {
        const float alpha = fast_exp2(m[h] - bm);
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[h][e] *= alpha;
        m[h] = bm;
      }
    }
#pragma unroll
    for (int p = 0; p < NPU; ++p) {
      float vf[16];
      VP::to_float(U.v[p], vf);
      if (!full) {
        const int32_t t = pos0 + p * TPP + tok;
        const bool ok = t >= lo && t < hi;
#pragma unroll
        for (int e = 0; e < 16; ++e) vf[e] = ok ? vf[e] : 0.f;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pr = m[h] == -INFINITY ? 0.f : fast_exp2(sc[p][h] - m[h]);
        l[h] += pr;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e]);
      }
    }
  };

  if (mask) {
    int cj = __builtin_ctzll(mask), cu = 0;
    Unit cur;
    load_unit(cur, cj, cu);
    while (true) {
      int nj = cj, nu = cu + 1;
      bool has_next = true;
      if (nu == NU) {
        const uint64_t rest = cj >= 63 ? 0ull : (mask & (~0ull << (cj + 1)));
        if (rest) {
          nj = __builtin_ctzll(rest);
          nu = 0;
        } else {
          has_next = false;
        }
      }
      Unit nxt;
      if (has_next) load_unit(nxt, nj, nu);
      compute(cur, cj, cu);
      if (!has_next) break;
      cur = nxt;
      cj = nj;
      cu = nu;
    }
  }

  // Sum lanes that hold the same elements (all share the wave-wide max).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = strided_sum<LPT>(l[h]);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = strided_sum<LPT>(acc[h][e]);
  }
  const int nslot = a.n_runs * a.nspl;
  const int64_t base = ((int64_t)s * nslot + slot) * a.n_q_heads + (int64_t)kvh * G;
  if (tok == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* o = a.part_o + (base + h) * HD;
#pragma unroll
      for (int c = 0; c < VP::kChunks; ++c) {
        float* dst = o + VP::chunk_dim(sub, c);
#pragma unroll
        for (int i = 0; i < VP::kChunkLen; i += 4)
          *(float4*)(dst + i) = make_float4(acc[h][c * VP::kChunkLen + i], acc[h][c * VP::kChunkLen + i + 1],
                                            acc[h][c * VP::kChunkLen + i + 2], acc[h][c * VP::kChunkLen + i + 3]);
      }
    }
  }
  if (lane < G) {
    // lane h writes head h's (max, sum); values are wave-uniform
    float mm = m[0], ll = l[0];
#pragma unroll
    for (int h = 1; h < G; ++h)
      if (lane == h) { mm = m[h]; ll = l[h]; }
    *(float2*)(a.part_ml + (base + lane) * 2) = make_float2(mm, ll);
  }
}

// Merge the split slots of one (sequence, q head) by log-sum-exp:
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i, lse = (M + log2 L) ln 2.
template <int HD>
__global__ __launch_bounds__(256) void decode_merge_kernel(AttnArgs a) {
  constexpr int NG = 256 / HD;  // slot groups
  const int h = blockIdx.x, s = blockIdx.y, t = threadIdx.x;
  const int nslot = a.n_runs * a.nspl;
  __shared__ float red[256];
  __shared__ float red2[256];
  const int32_t lim = clamp_seq_len(a.seq_lens[s], a.max_blocks, a.block_size);

  float M = -INFINITY;
  for (int slot = t; slot < nslot; slot += 256) {
    int32_t lo, hi;
    split_range(a, s, slot, lim, lo, hi);
    if (lo < hi) M = fmaxf(M, a.part_ml[(((int64_t)s * nslot + slot) * a.n_q_heads + h) * 2]);
  }
  red[t] = M;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] = fmaxf(red[t], red[t + w]);
    __syncthreads();
  }
  M = red[0];
  __syncthreads();

  const int d = t % HD, grp = t / HD;
  float acc = 0.f, lsum = 0.f;
  if (M != -INFINITY) {
    for (int slot = grp; slot < nslot; slot += NG) {
      int32_t lo, hi;
      split_range(a, s, slot, lim, lo, hi);
      if (lo >= hi) continue;
      const int64_t base = ((int64_t)s * nslot + slot) * a.n_q_heads + h;
      const float mi = a.part_ml[base * 2];
      if (mi == -INFINITY) continue;
      const float w = fast_exp2(mi - M);
      acc = fmaf(w, a.part_o[base * HD + d], acc);
      lsum = fmaf(w, a.part_ml[base * 2 + 1], lsum);
    }
  }
  red[t] = acc;
  red2[t] = lsum;
  __syncthreads();
  if (grp == 0) {
    float sa = red[d], sl = red2[d];
#pragma unroll
    for (int g2 = 1; g2 < NG; ++g2) {
      sa += red[g2 * HD + d];
      sl += red2[g2 * HD + d];
    }
    const int64_t o = ((int64_t)s * a.n_q_heads + h) * HD + d;
    if (M == -INFINITY) {
      a.out[o] = 0.f;
      if (a.lse && d == 0) a.lse[(int64_t)s * a.n_q_heads + h] = -INFINITY;
    } else {
      a.out[o] = sa / sl;
      if (a.lse && d == 0) a.lse[(int64_t)s * a.n_q_heads + h] = (M + __builtin_amdgcn_logf(sl)) * kLn2;
    }
  }
}

}  // namespace pkv
