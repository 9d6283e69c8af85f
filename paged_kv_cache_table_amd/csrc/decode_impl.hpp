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
  // Register ring of one-pass units: as many as fit the instance's budget
  // next to q, the running outputs and the temporaries; the loads run
  // RING-1 units ahead of compute.
  constexpr int kBudget = SplitRegs<HD, G, COMBO>::kBudget;
  constexpr int kRingFit = kBudget / (KW + VW);
  constexpr int RING = kRingFit < 2 ? 2 : (kRingFit > 8 ? 8 : kRingFit);
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
  if (a.items) {
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
    split_range(a, s, slot, clamp_seq_len(a.seq_lens[s], a.max_blocks, BS), lo, hi);
    if (lo >= hi) return;  // not a work item
    prow = (int64_t)s * a.rows_per_seq + slot;
  }

  const int32_t jb0 = lo / BS;
  const int32_t nblk = (hi - 1) / BS - jb0 + 1;  // <= 64 by construction
  int32_t myid = -1;
  if (lane < nblk) myid = block_id(a, s, jb0 + lane, kvh == 0);
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

  // Units (one pass each) run in order over the non-hole blocks; loads run
  // RING-1 units ahead of compute through a ring of RING register buffers.
  // The ring is unrolled so every buffer keeps a fixed role.  The body has a
  // fixed number of steps with one exit at its top: an exit in the middle
  // would become an exec-masked flow block whose join makes the compiler
  // drain all outstanding loads.  Steps past the last unit load that unit
  // again (cache hits) and skip the compute, so the number of loads issued
  // after any unit is fixed and each wait leaves the later loads in flight.
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
    auto load_next = [&](Unit& U) {
      load_unit(U, lc.j, lc.u);
      if (++issued < n_units) advance(lc);
    };
    const int n_pad = (n_units + RING - 1) / RING * RING;
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
  const dim3 grid = a.items ? dim3((unsigned)max_units)
                            : dim3((unsigned)a.n_kv_heads, (unsigned)(a.n_runs * a.nspl), (unsigned)a.n_seqs);
  hipLaunchKernelGGL((decode_split_kernel<HD, BS, G, COMBO>), grid, dim3(64), 0, st, a);
  return hipGetLastError();
}

// Merge the partials of each (sequence, q head) by log-sum-exp:
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i, lse = (M + log2 L) ln 2.
// Four waves per workgroup, one lane per (q head, dim) output, so each load
// is 256 contiguous bytes.  merge_split = 1: each wave merges all rows of
// its own 64 outputs (256 outputs per workgroup).  merge_split = 4 (grids
// too small to fill the device that way): the four waves share 64 outputs,
// wave w merging rows w, w + 4, ..., and wave 0 combines the four results
// in wave order through LDS.  Within a wave the rows go in order with a
// running max, the loads of eight rows issued before their arithmetic.
// Fixed order for a given shape, so results are deterministic.
// A run's non-empty slots and their pieces hold one contiguous range of
// rows, found from the run's bounds exactly as the plan pass places them.
template <int HD, int NW>
__global__ __launch_bounds__(256) void decode_merge_kernel(AttnArgs a) {
  constexpr int kUnroll = 8, kWaves = 4;
  __shared__ float part[3][kWaves - 1][64];
  const int s = blockIdx.y;
  constexpr int nw = NW;  // waves per output group (merge_split): 1 or 4
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = wv / nw, phase = wv - grp * nw;
  const int idx = (blockIdx.x * (kWaves / nw) + grp) * 64 + lane;  // q head * HD + dim
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
  float m = -INFINITY, l = 0.f, acc = 0.f;
  // merge (m2, l2, o2) into the running (m, l, acc); a partial that saw
  // nothing (m2 = -inf) carries no weight, and an empty running value (m =
  // -inf, l = acc = 0) is scaled by 2^-inf = 0
  auto add = [&](float m2, float l2, float o2) {
    if (m2 == -INFINITY) return;
    const float mn = fmaxf(m, m2);
    const float ca = fast_exp2(m - mn), cb = fast_exp2(m2 - mn);
    acc = acc * ca + o2 * cb;
    l = l * ca + l2 * cb;
    m = mn;
  };
  // row(slot) = slot + (cut slots before it) * (nsub - 1)
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
    for (int i0 = phase; live && i0 < n_rows; i0 += nw * kUnroll) {
      float2 ml[kUnroll];
      float o[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        ml[u] = make_float2(-INFINITY, 0.f);
        o[u] = 0.f;
        const int i = i0 + nw * u;
        if (i < n_rows) {
          const int64_t row = (row_a + i) * a.n_q_heads + h;
          ml[u] = *(const float2*)(a.part_ml + row * 2);
          o[u] = a.part_o[row * HD + d];
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) add(ml[u].x, ml[u].y, o[u]);
    }
  }
  if constexpr (nw > 1) {
    if (phase > 0) {
      part[0][phase - 1][lane] = m;
      part[1][phase - 1][lane] = l;
      part[2][phase - 1][lane] = acc;
    }
    __syncthreads();
    if (phase > 0) return;
#pragma unroll
    for (int w2 = 0; w2 < kWaves - 1; ++w2) add(part[0][w2][lane], part[1][w2][lane], part[2][w2][lane]);
  }
  if (!live) return;
  const int64_t oi = ((int64_t)s * a.n_q_heads + h) * HD + d;
  if (m == -INFINITY) {
    a.out[oi] = 0.f;
    if (a.lse && d == 0) a.lse[(int64_t)s * a.n_q_heads + h] = -INFINITY;
  } else {
    a.out[oi] = acc / l;
    if (a.lse && d == 0) a.lse[(int64_t)s * a.n_q_heads + h] = (m + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

}  // namespace pkv
