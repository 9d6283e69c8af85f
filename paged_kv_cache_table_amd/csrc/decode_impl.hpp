// Split-K paged decode for gfx950.
//
// What it computes ("Tiered KV cache — architecture", section "The
// paged-attention block model"; "KV cache" (sipllm), section "Problem"):
// for each sequence s and q head h, softmax attention of its one query over
// the positions of its window that lie in [0, seq_len) and are not in a
// hole, reading K/V rows through the block table.
//
// Work unit = (item, kv head), one wave at a time.  An item is a split slot
// (the intersection of one window run with an aligned range of `split`
// positions, so its blocks are at most 64 and their ids fit one register)
// or a piece of one.  For calls with many possible items the plan pass
// lists them without gaps: whole slots first, the pieces of cut slots
// last, so the hardware dispatcher keeps every wave slot busy and the pass
// ends on short units.  Smaller calls skip the plan and launch one
// workgroup per possible slot.
// Lane layout: each token row of one kv head is spread over LPT = HD/16
// lanes (16 elements per lane), a pass covers TPP = 64/LPT tokens, and a
// 16- or 32-token block takes BS/TPP passes.  A pass's K and V rows are
// staged ahead of compute, through an LDS ring filled by HBM->LDS copies
// (head_dim 128) or a register ring (head_dim 64 and 256).  The g query heads that share
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
  static constexpr int kQRegs = G * 8;
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
  static constexpr int kQRegs = G * 16;
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
  static constexpr int kQRegs = G * 16;
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
  // acc += p * v with the f16 -> f32 conversion folded into the FMA
  __device__ __forceinline__ static void fma_acc(const uint32_t (&w)[VW], float p, float (&acc)[16]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      acc[2 * i] = fmaf(p, h2f_lo(w[i]), acc[2 * i]);
      acc[2 * i + 1] = fmaf(p, h2f_hi(w[i]), acc[2 * i + 1]);
    }
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
  __device__ __forceinline__ static void fma_acc(const uint32_t (&w)[VW], float p, float (&acc)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = fmaf(p, __builtin_bit_cast(float, w[i]), acc[i]);
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

// The work list without the plan pass: item `it` of the list the plan pass
// would write (whole full slots, then partial slots, then the pieces of cut
// slots, each group in sequence order; see decode_plan_kernel), derived by
// one wave from the sequences' lengths and windows.  Lane l holds sequences
// l * SPL .. l * SPL + SPL - 1; three wave scans give each lane's place in
// each group; the lane whose range holds `it` names the sequence, and the
// sequence's runs give the slot.  Wave-uniform results.  Returns false when
// `it` is past the list's end.
__device__ inline bool self_plan_item(const AttnArgs& a, uint32_t it, int& s_out, int32_t& lo_out,
                                      int32_t& hi_out, int64_t& row_out) {
  constexpr int SPL = kSelfPlanMaxSeqs / 64;
  const int lane = threadIdx.x & 63;
  const int32_t split = a.split;
  const uint32_t fps = (uint32_t)a.fine_per_seq;
  uint32_t cnt[3][SPL], fcut[SPL];
  uint32_t tot[3] = {0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const int s = lane * SPL + i;
    uint32_t nact = 0, nfull = 0;
    if (s < a.n_seqs) {
      const int32_t L = clamp_seq_len(a.seq_lens[s], a.max_blocks, a.block_size);
      for (int r = 0; r < a.n_runs; ++r) {
        int32_t rl, rh;
        run_range(a, s, r, L, rl, rh);
        nact += rh > rl ? (uint32_t)((rh - 1) / split - rl / split + 1) : 0u;
        nfull += (uint32_t)full_slots(rl, rh, split);
      }
    }
    const uint32_t ncut = nfull < fps ? nfull : fps;
    fcut[i] = nfull - ncut;
    cnt[0][i] = nfull - ncut;
    cnt[1][i] = nact - nfull;
    cnt[2][i] = ncut;
#pragma unroll
    for (int c = 0; c < 3; ++c) tot[c] += cnt[c][i];
  }
  // exclusive prefix over lanes of each group's lane total
  uint32_t excl[3], all[3];
#pragma unroll
  for (int c = 0; c < 3; ++c) {
    uint32_t inc = tot[c];
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t y = (uint32_t)__shfl_up((int)inc, d, 64);
      if (lane >= d) inc += y;
    }
    excl[c] = inc - tot[c];
    all[c] = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
  }
  const uint32_t nsub = (uint32_t)a.nsub;
  int grp;
  uint32_t t;
  if (it < all[0]) {
    grp = 0;
    t = it;
  } else if (it - all[0] < all[1]) {
    grp = 1;
    t = it - all[0];
  } else if ((it - all[0] - all[1]) / nsub < all[2]) {
    grp = 2;
    t = (it - all[0] - all[1]) / nsub;
  } else {
    return false;
  }
  // the lane whose sequences hold rank t of the group, then the sequence
  uint32_t ex_g = grp == 0 ? excl[0] : (grp == 1 ? excl[1] : excl[2]);
  uint32_t tot_g = grp == 0 ? tot[0] : (grp == 1 ? tot[1] : tot[2]);
  const uint64_t above = __ballot(ex_g + tot_g > t);
  const int ln = (int)__builtin_ctzll(above);
  uint32_t rank = t - (uint32_t)__builtin_amdgcn_readlane((int)ex_g, ln);
  int s = ln * SPL;
  uint32_t first_cut = 0;
#pragma unroll
  for (int i = 0; i < SPL; ++i) {
    const uint32_t ci = (uint32_t)__builtin_amdgcn_readlane(
        (int)(grp == 0 ? cnt[0][i] : (grp == 1 ? cnt[1][i] : cnt[2][i])), ln);
    const uint32_t fc = (uint32_t)__builtin_amdgcn_readlane((int)fcut[i], ln);
    if (s == ln * SPL + i) {
      if (rank < ci) {
        first_cut = fc;
      } else {
        rank -= ci;
        ++s;
      }
    }
  }
  s = __builtin_amdgcn_readfirstlane(s);
  rank = (uint32_t)__builtin_amdgcn_readfirstlane((int)rank);
  first_cut = (uint32_t)__builtin_amdgcn_readfirstlane((int)first_cut);
  const int32_t L = clamp_seq_len(a.seq_lens[s], a.max_blocks, a.block_size);
  const int64_t seq_row0 = (int64_t)s * a.rows_per_seq;
  // full slot number fi (in sequence order over the runs): its run and slot
  auto full_slot = [&](uint32_t fi, int& r_o, int32_t& k_o) {
    for (int r = 0; r < a.n_runs; ++r) {
      int32_t rl, rh;
      run_range(a, s, r, L, rl, rh);
      const uint32_t nf = (uint32_t)full_slots(rl, rh, split);
      if (fi < nf) {
        r_o = r;
        k_o = (int32_t)(((int64_t)rl + split - 1) / split) + (int32_t)fi;
        return;
      }
      fi -= nf;
    }
    r_o = 0;
    k_o = 0;
  };
  if (grp == 0) {
    int r;
    int32_t k;
    full_slot(rank, r, k);
    lo_out = k * split;
    hi_out = lo_out + split;
    row_out = seq_row0 + (int64_t)r * a.nspl + k;
  } else if (grp == 2) {
    int r;
    int32_t k;
    full_slot(first_cut + rank, r, k);
    const uint32_t p = (it - all[0] - all[1]) % nsub;
    lo_out = k * split + (int32_t)p * a.fine_tokens;
    const int32_t e = lo_out + a.fine_tokens;
    hi_out = e < k * split + split ? e : k * split + split;
    row_out = seq_row0 + (int64_t)r * a.nspl + k + (int64_t)rank * (nsub - 1) + p;
  } else {
    // the rank-th partial slot: a run's partial slots are its first active
    // slot (when partial) and its last (when partial and not the first)
    uint32_t full_before = 0;
    int32_t kk = 0, rr = 0, plo = 0, phi = 0;
    uint32_t fb_here = 0;
    for (int r = 0; r < a.n_runs; ++r) {
      int32_t rl, rh;
      run_range(a, s, r, L, rl, rh);
      if (rh <= rl) continue;
      const int32_t k0 = rl / split, k1 = (rh - 1) / split;
      const int32_t kf0 = (int32_t)(((int64_t)rl + split - 1) / split), kf1 = rh / split;
      const uint32_t nf = (uint32_t)full_slots(rl, rh, split);
      const bool p0 = k0 < kf0 || k0 >= kf1;
      const bool p1 = k1 != k0 && k1 >= kf1;
      const uint32_t np = (p0 ? 1u : 0u) + (p1 ? 1u : 0u);
      if (rank < np) {
        const bool first = p0 && rank == 0;
        kk = first ? k0 : k1;
        rr = r;
        plo = rl > kk * split ? rl : kk * split;
        phi = rh < kk * split + split ? rh : kk * split + split;
        // full slots of this run before slot kk
        const int32_t fh = kk < kf0 ? 0 : (kk - kf0 < kf1 - kf0 ? kk - kf0 : kf1 - kf0);
        fb_here = full_before + (uint32_t)(fh > 0 ? fh : 0);
        break;
      }
      rank -= np;
      full_before += nf;
    }
    const uint32_t cut_before = fb_here > first_cut ? fb_here - first_cut : 0u;
    lo_out = plo;
    hi_out = phi;
    row_out = seq_row0 + (int64_t)rr * a.nspl + kk + (int64_t)cut_before * (nsub - 1);
  }
  s_out = s;
  return true;
}

// Waves per SIMD and register budget of an instance: three waves (a ring
// of at least two passes next to q, the running outputs and ~24
// temporaries, in ~152 VGPRs) where they fit, else no bound on the waves
// and a ring sized for ~232 VGPRs (two waves per SIMD; the eight-head
// groups need more and run one).  With the work list keeping every wave slot busy, the third wave
// hides the start of each unit better than a deeper ring does (7B-class
// split pass 734-736 against 739-744 us; long context and SmolLM2-like
// batches also a little faster).
template <int HD, int G, int COMBO>
struct SplitRegs {
  using KP = typename Paths<HD, G, COMBO>::K;
  using VP = typename Paths<HD, G, COMBO>::V;
  static constexpr int kBase = KP::kQRegs + 16 * G + 24;
  static constexpr int kUnitRegs = KP::KW + VP::VW;
  static constexpr int kWaves = kBase + 2 * kUnitRegs <= 152 ? 3 : 1;  // launch bound
  static constexpr int kBudget = (kWaves == 3 ? 152 : 232) - kBase;
};

template <int HD, int BS, int G, int COMBO>
__global__ __launch_bounds__(64, (SplitRegs<HD, G, COMBO>::kWaves)) void decode_split_kernel(AttnArgs a) {
  using KP = typename Paths<HD, G, COMBO>::K;
  using VP = typename Paths<HD, G, COMBO>::V;
  using QT = typename QElem<COMBO>::T;
  constexpr int LPT = HD / 16;   // lanes per token row
  constexpr int TPP = 64 / LPT;  // tokens per pass
  static_assert(BS % TPP == 0, "block size must be a multiple of tokens per pass");
  constexpr int NU = BS / TPP;  // passes per block; a pass is the pipelined unit
  constexpr int KW = KP::KW, VW = VP::VW;
  // K/V staging.  head_dim 128 (16-bit and q8_0 rows): an LDS ring of two
  // one-pass units, private to the wave: a pass's K rows and V rows are
  // contiguous in the (block, kv head) tile, so each is copied from HBM into
  // its slot by whole 16-byte lanes (global_load_lds_dwordx4, 1 KiB per
  // instruction) one unit ahead of compute, and the compute reads the lane's
  // own elements from the slot.
  // On the 7B-class batch two slots measured 737-738 us per step back to
  // back (748.5 us for one cold call), three slots 741-742 (748-754), and a
  // ring of the same units in registers 735-736: the three waves per SIMD
  // keep enough bytes in flight, and a deeper ring only adds to them.
  // head_dim 64 and 256: the register ring (the loads themselves run
  // ahead), sized to the instance's register budget; the LDS ring measured
  // the same there (SmolLM2-like 34.0-34.2 against 34.1-34.2 us per call,
  // long context 1466-1467 against 1465-1466 us per step).
  constexpr int KPB = TPP * (int)KP::kHeadBytes;  // K bytes of one pass
  constexpr int VPB = TPP * (int)VP::kHeadBytes;  // V bytes of one pass
  constexpr int KPB16 = (KPB + 15) / 16 * 16;
  constexpr int SLOT = KPB16 + VPB;
  constexpr int NDK = (KPB + 1023) / 1024, NDV = (VPB + 1023) / 1024;
  constexpr int NDMA = NDK + NDV;  // copy instructions per unit
  // the LDS ring where two slots per wave fit the CU's 160 KiB at the
  // instance's occupancy (f32 rows do not)
  constexpr bool kLds = HD == 128 && 4 * SplitRegs<HD, G, COMBO>::kWaves * 2 * SLOT <= 160 * 1024;
  constexpr int kBudget = SplitRegs<HD, G, COMBO>::kBudget;
  constexpr int kRingFit = kBudget / (KW + VW);
  constexpr int RING = kLds ? 2 : (kRingFit < 2 ? 2 : (kRingFit > 8 ? 8 : kRingFit));
  static_assert(!kLds || (RING - 1) * NDMA < 64, "vmcnt range");
  static_assert(KPB % 16 == 0 && VPB % 16 == 0, "a pass copies whole 16-byte pieces");
  __shared__ __attribute__((aligned(16))) unsigned char stage[kLds ? RING : 1][kLds ? SLOT : 16];
  constexpr float kEmpty = -1e30f;  // running max before any visible token

  const int lane = threadIdx.x, tok = lane / LPT, sub = lane % LPT;
  // Planned calls: one workgroup per unit of the list, units item-major
  // (kv head fastest: the Hkv waves that read interleaved slices of the
  // same pool rows start together); the grid is the host's bound on units
  // and the workgroups past the count the plan wrote, all at the end of the
  // grid, leave at once.  Direct calls: grid (kv head, slot, sequence),
  // empty slots leave at once.
  int s, kvh;
  int32_t lo, hi;
  int64_t prow;
  int32_t spec = -1;       // this lane's table entry, read ahead (direct causal calls)
  bool have_spec = false;
  if (a.self_plan) {
    const uint32_t unit = blockIdx.x;
    const uint32_t item = unit / (uint32_t)a.n_kv_heads;
    kvh = (int)(unit - item * (uint32_t)a.n_kv_heads);
    if (!self_plan_item(a, item, s, lo, hi, prow)) return;
    s = __builtin_amdgcn_readfirstlane(s);
    lo = __builtin_amdgcn_readfirstlane(lo);
    hi = __builtin_amdgcn_readfirstlane(hi);
    if (lo >= hi) return;
  } else if (a.items) {
    const uint32_t unit = blockIdx.x;
    if (unit >= a.hdr[0]) return;
    const uint32_t item = unit / (uint32_t)a.n_kv_heads;
    kvh = (int)(unit - item * (uint32_t)a.n_kv_heads);
    const uint4 it = a.items[item];  // (sequence, lo, hi, partial row), lo < hi
    s = (int)__builtin_amdgcn_readfirstlane((int)it.x);
    lo = __builtin_amdgcn_readfirstlane((int)it.y);
    hi = __builtin_amdgcn_readfirstlane((int)it.z);
    prow = (uint32_t)__builtin_amdgcn_readfirstlane((int)it.w);
    // An entry that is not an item of this call (the list is only valid
    // right after the plan pass of the same call) is skipped rather than
    // followed out of bounds: sequence, range within the table and inside
    // one aligned split, and row are all checked.
    if ((uint32_t)s >= (uint32_t)a.n_seqs || lo < 0 || hi <= lo || (int64_t)hi > (int64_t)a.max_blocks * BS ||
        hi - lo > a.split || (hi - 1) / BS - lo / BS >= 64 || prow >= (int64_t)a.n_seqs * a.rows_per_seq)
      return;
  } else {
    kvh = blockIdx.x;
    const int slot = blockIdx.y;
    s = blockIdx.z;
    if (a.mode == PKV_WIN_CAUSAL) {
      // Causal: slot k covers [k split, (k + 1) split) cut at the sequence
      // length, so its table entries do not wait for the length; they are
      // read beside it (entries past the cut are neither used nor checked).
      const int32_t b = slot * (a.split / BS) + lane;
      if (lane < a.split / BS && b < a.max_blocks) spec = a.table[(int64_t)s * a.max_blocks + b];
      have_spec = true;
    }
    split_range(a, s, slot, clamp_seq_len(a.seq_lens[s], a.max_blocks, BS), lo, hi);
    if (lo >= hi) return;  // not a work item
    prow = (int64_t)s * a.rows_per_seq + slot;
  }

  const int32_t jb0 = lo / BS;
  const int32_t nblk = (hi - 1) / BS - jb0 + 1;  // <= 64 by construction
  int32_t myid = -1;
  if (have_spec) {
    // the entry read ahead, checked as block_id checks it (slot k starts at
    // block jb0 = k split / BS, so lane i holds block jb0 + i)
    if (lane < nblk) {
      myid = spec;
      if (myid < 0 || myid >= a.n_pool_blocks) {
        if (kvh == 0 && myid != PKV_INVALID_BLOCK_ID && (a.flags & PKV_FLAG_CHECKED) && a.err) atomicAdd(a.err, 1);
        myid = -1;
      }
    }
  } else if (lane < nblk) {
    myid = block_id(a, s, jb0 + lane, kvh == 0);
  }
  // q is read while the block ids are in flight
  KP kp;
  const int64_t qoff = ((int64_t)s * a.n_q_heads + (int64_t)kvh * G) * HD;
  kp.load_q((const QT*)a.q + qoff, sub);
  // The ballot is wave-uniform; readfirstlane makes that visible to the
  // compiler, so loops over it stay scalar (no exec-masked flow blocks).
  const uint64_t bal = __ballot(myid >= 0);
  const uint64_t mask = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(bal >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)bal);

  // m: running max of the scaled scores (log2 domain), wave-uniform; l and
  // acc: this lane's running sum and output for its tokens, all relative to m.
  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kEmpty;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = 0.f;
  }

  // Pool layout [block][kv head][slot][head]: this wave's (block, kv head)
  // tile is block_size contiguous token entries.
  const unsigned char* kbase = a.k_pool + (int64_t)kvh * BS * KP::kHeadBytes;
  const unsigned char* vbase = a.v_pool + (int64_t)kvh * BS * VP::kHeadBytes;
  const int64_t kbb = a.k_block_bytes, vbb = a.v_block_bytes;

  struct Unit {
    uint32_t k[KW];
    uint32_t v[VW];
  };
  // copy unit (j, u) into ring slot r: K then V, 16 bytes per lane and
  // instruction (the last instruction of each may leave lanes idle)
  auto copy_unit = [&](int r, int j, int u) {
    const int32_t blk = __builtin_amdgcn_readlane(myid, j);
    const unsigned char* kg = kbase + blk * kbb + u * KPB;
    const unsigned char* vg = vbase + blk * vbb + u * VPB;
    const uint32_t lk = (uint32_t)__builtin_amdgcn_readfirstlane((int)lds_addr(&stage[r][0]));
    const uint32_t lv = lk + KPB16;
#pragma unroll
    for (int i = 0; i < NDK; ++i)
      if (i * 1024 + lane * 16 < KPB) copy16_to_lds(kg, (uint32_t)(i * 1024 + lane * 16), lk + i * 1024);
#pragma unroll
    for (int i = 0; i < NDV; ++i)
      if (i * 1024 + lane * 16 < VPB) copy16_to_lds(vg, (uint32_t)(i * 1024 + lane * 16), lv + i * 1024);
  };
  // the lane's elements of the unit in slot r, once its copies have landed
  auto read_unit = [&](Unit& U, int r) {
    kp.load_k(&stage[r][tok * KP::kHeadBytes], sub, U.k);
    VP::load(&stage[r][KPB16 + tok * VP::kHeadBytes], sub, U.v);
  };
  // register ring: the lane's elements of unit (j, u) straight from HBM
  auto load_unit = [&](Unit& U, int j, int u) {
    const int32_t blk = __builtin_amdgcn_readlane(myid, j);
    const int slot = u * TPP + tok;
    kp.load_k(kbase + blk * kbb + slot * KP::kHeadBytes, sub, U.k);
    VP::load(vbase + blk * vbb + slot * VP::kHeadBytes, sub, U.v);
  };
  auto compute = [&](Unit& U, int j, int u) {
    const int32_t pos0 = (jb0 + j) * BS + u * TPP;
    const bool full = pos0 >= lo && pos0 + TPP <= hi;  // wave-uniform
    float sc[G];
    kp.dot(U.k, sc);
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = group_sum<LPT>(sc[h]) * a.score_mul;
    if (!full) {
      // window edge: positions outside [lo, hi) get score -inf and value 0
      // (selected, never multiplied, so NaN in those rows cannot leak in)
      const int32_t t = pos0 + tok;
      const bool ok = t >= lo && t < hi;
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = ok ? sc[h] : -INFINITY;
#pragma unroll
      for (int i = 0; i < VW; ++i) U.v[i] = ok ? U.v[i] : 0u;
    }
    // The max only moves when some score exceeds it; most units skip the
    // cross-lane reduction and the rescale entirely.
    bool above = false;
#pragma unroll
    for (int h = 0; h < G; ++h) above |= sc[h] > m[h];
    if (__builtin_amdgcn_ballot_w64(above)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(m[h], wave_max_tokens<LPT>(sc[h]));
        const float alpha = fast_exp2(m[h] - mn);  // 1 if unchanged, 0 from empty
        l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[h][e] *= alpha;
        m[h] = mn;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = fast_exp2(sc[h] - m[h]);  // -inf -> 0
      l[h] += pr;
      VP::fma_acc(U.v, pr, acc[h]);
    }
  };

  // Units (one pass each) run in order over the non-hole blocks; copies (or
  // loads) run RING-1 units ahead of compute through the ring of RING LDS
  // slots (or register buffers).  The ring is unrolled so every slot keeps
  // a fixed role.  The body has a fixed number of steps with one exit at its
  // top: an exit in the middle would become an exec-masked flow block whose
  // join makes the compiler drain all outstanding loads.  Steps past the
  // last unit copy that unit again (cache hits) and skip the compute, so the
  // number of copies issued after any unit is fixed and each wait leaves the
  // later copies in flight.
  struct Cursor {
    uint64_t rest;  // blocks after j still to visit
    int j, u;
  };
  auto advance = [&](Cursor& c) {
    if (++c.u == NU) {
      c.u = 0;
      c.j = c.rest ? __builtin_ctzll(c.rest) : 64;
      c.rest &= c.rest - 1;
    }
  };
  const int n_units = __builtin_popcountll(mask) * NU;
  if (n_units > 0) {
    Cursor lc;
    lc.j = __builtin_ctzll(mask);
    lc.rest = mask & (mask - 1);
    lc.u = 0;
    Cursor cc = lc;
    int issued = 0;
    const int n_pad = (n_units + RING - 1) / RING * RING;
    if constexpr (kLds) {
      auto copy_next = [&](int r) {
        copy_unit(r, lc.j, lc.u);
        if (++issued < n_units) advance(lc);
      };
#pragma unroll
      for (int r = 0; r < RING - 1; ++r) copy_next(r);
      // The compiler does not count the copies (inline assembly) among the
      // loads in flight.  Waiting here for everything issued so far (q, then
      // the first RING - 1 units) is what tells it that q has arrived;
      // otherwise it would place waits for q at q's first use inside the
      // loop, where in hardware they would also wait for every copy the ring
      // has in flight, on every step.
      wait_vm<0>();
      for (int i = 0; i < n_pad; i += RING) {
#pragma unroll
        for (int r = 0; r < RING; ++r) {
          // slot (r - 1) mod RING was read by the previous step's compute,
          // which waited for those reads before using them
          copy_next((r + RING - 1) % RING);
          // the RING - 1 units copied after unit r may still be in flight
          wait_vm<(RING - 1) * NDMA>();
          asm volatile("" ::: "memory");
          if (cc.j < 64) {
            Unit U;
            read_unit(U, r);
            compute(U, cc.j, cc.u);
          }
          advance(cc);
        }
      }
      // no copy may land in LDS after the wave ends
      wait_vm<0>();
    } else {
      auto load_next = [&](Unit& U) {
        load_unit(U, lc.j, lc.u);
        if (++issued < n_units) advance(lc);
      };
      Unit buf[RING];
#pragma unroll
      for (int r = 0; r < RING - 1; ++r) load_next(buf[r]);
      for (int i = 0; i < n_pad; i += RING) {
#pragma unroll
        for (int r = 0; r < RING; ++r) {
          load_next(buf[(r + RING - 1) % RING]);
          if (cc.j < 64) compute(buf[r], cc.j, cc.u);
          advance(cc);
        }
      }
    }
  }
  // A wave that saw no visible token reports an empty partial.
#pragma unroll
  for (int h = 0; h < G; ++h)
    if (m[h] == kEmpty) m[h] = -INFINITY;

  // Sum lanes that hold the same elements (all share the wave-wide max).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l[h] = strided_sum<LPT>(l[h]);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[h][e] = strided_sum<LPT>(acc[h][e]);
  }
  const int64_t base = prow * a.n_q_heads + (int64_t)kvh * G;
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

// Launch of one split kernel instance: planned, one one-wave workgroup per
// unit the call can have at most (max_units); direct, grid (kv head, slot,
// sequence).
template <int HD, int BS, int G, int COMBO>
hipError_t launch_split_instance(const AttnArgs& a, int64_t max_units, hipStream_t st) {
  const dim3 grid = (a.items || a.self_plan) ? dim3((unsigned)max_units)
                            : dim3((unsigned)a.n_kv_heads, (unsigned)(a.n_runs * a.nspl), (unsigned)a.n_seqs);
  hipLaunchKernelGGL((decode_split_kernel<HD, BS, G, COMBO>), grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

// Merge the partials of each (sequence, q head) by log-sum-exp:
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i, lse = (M + log2 L) ln 2.
// A workgroup takes 256 consecutive (q head, dim) outputs of one sequence,
// each lane four of them (16-byte loads, so a wave loads 1 KiB of a partial
// row at once); its NW waves share the rows (wave w takes rows w, w + NW,
// ..., in order, with a running max, the loads of four rows issued before
// their arithmetic) and wave 0 combines the NW results in wave order
// through LDS.  NW = 8 where the grid is small (fewer than 512
// workgroups: each sequence's rows are walked in fewer dependent rounds),
// else 4 (SmolLM2-like merge 7.7 against 8.3 us per launch, long context
// 13.7 against 15.2; the 7B-class batch, 1,024 workgroups, 11.0 against
// 12.9 with eight).  Fixed order for a given shape, so results are
// deterministic.  A run's non-empty slots and their pieces hold one
// contiguous range of rows, found from the run's bounds exactly as the plan
// places them.
template <int HD, int NW>
__global__ __launch_bounds__(64 * NW) void decode_merge_kernel(AttnArgs a) {
  constexpr int kUnroll = 4, kWaves = NW;
  __shared__ float part[kWaves - 1][6][64];
  const int s = blockIdx.y;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int idx = blockIdx.x * 256 + lane * 4;  // q head * HD + dim of the lane's first output
  const bool live = idx < a.n_q_heads * HD;
  const int h = live ? idx / HD : 0, d = live ? idx - h * HD : 0;
  const int32_t lim = clamp_seq_len(a.seq_lens[s], a.max_blocks, a.block_size);
  int32_t rl, rh;
  int nfull = 0;
  for (int r = 0; r < a.n_runs; ++r) {
    run_range(a, s, r, lim, rl, rh);
    nfull += full_slots(rl, rh, a.split);
  }
  const int first_cut = nfull - (nfull < a.fine_per_seq ? nfull : a.fine_per_seq);
  float m = -INFINITY, l = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  auto add = [&](float m2, float l2, const float (&o2)[4]) {
    if (m2 == -INFINITY) return;
    const float mn = fmaxf(m, m2);
    const float ca = fast_exp2(m - mn), cb = fast_exp2(m2 - mn);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = acc[e] * ca + o2[e] * cb;
    l = l * ca + l2 * cb;
    m = mn;
  };
  int full_before = 0;
  for (int r = 0; r < a.n_runs; ++r) {
    run_range(a, s, r, lim, rl, rh);
    if (rh <= rl) continue;
    const int nf = full_slots(rl, rh, a.split);
    const int k0 = rl / a.split, k1 = (rh - 1) / a.split;
    const int cut0 = full_before > first_cut ? full_before - first_cut : 0;
    const int cut1 = full_before + nf > first_cut ? full_before + nf - first_cut : 0;
    full_before += nf;
    const int64_t row_a = (int64_t)s * a.rows_per_seq + (int64_t)r * a.nspl + k0 + (int64_t)cut0 * (a.nsub - 1);
    const int n_rows = k1 - k0 + 1 + (cut1 - cut0) * (a.nsub - 1);
    for (int i0 = wv; live && i0 < n_rows; i0 += kWaves * kUnroll) {
      float2 ml[kUnroll];
      float4 o[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        ml[u] = make_float2(-INFINITY, 0.f);
        o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        const int i = i0 + kWaves * u;
        if (i < n_rows) {
          const int64_t row = (row_a + i) * a.n_q_heads + h;
          ml[u] = *(const float2*)(a.part_ml + row * 2);
          o[u] = *(const float4*)(a.part_o + row * HD + d);
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const float ov[4] = {o[u].x, o[u].y, o[u].z, o[u].w};
        add(ml[u].x, ml[u].y, ov);
      }
    }
  }
  if (wv > 0) {
    part[wv - 1][0][lane] = m;
    part[wv - 1][1][lane] = l;
#pragma unroll
    for (int e = 0; e < 4; ++e) part[wv - 1][2 + e][lane] = acc[e];
  }
  __syncthreads();
  if (wv > 0 || !live) return;
#pragma unroll
  for (int w2 = 0; w2 < kWaves - 1; ++w2) {
    const float ov[4] = {part[w2][2][lane], part[w2][3][lane], part[w2][4][lane], part[w2][5][lane]};
    add(part[w2][0][lane], part[w2][1][lane], ov);
  }
  float* orow = a.out + ((int64_t)s * a.n_q_heads + h) * HD + d;
  if (m == -INFINITY) {
    *(float4*)orow = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.lse && d == 0) a.lse[(int64_t)s * a.n_q_heads + h] = -INFINITY;
  } else {
    const float inv = 1.f / l;
    *(float4*)orow = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    if (a.lse && d == 0) a.lse[(int64_t)s * a.n_q_heads + h] = (m + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

}  // namespace pkv
