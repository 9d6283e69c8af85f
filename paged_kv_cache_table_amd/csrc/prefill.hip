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
// Work decomposition.  A workgroup (4 waves) takes one kv head, a block of
// consecutive queries of one sequence (128 rows = (query, q head of the
// GQA group) pairs, 32 per wave in two 16-row tiles) and one of nch chunks
// of the window: the window's runs, clipped to [0, min(seq_len, largest
// causal limit of the rows)), are seen as one concatenated index space cut
// into nch equal chunks.  With nch > 1 each workgroup writes (max, sum,
// unnormalised output) per row and a merge kernel combines them with the
// log-sum-exp rule; with nch = 1 the output is written directly.  Workgroups
// that share a chunk's K/V are numbered so that they land on the same XCD
// (consecutive task numbers map to one XCD's share of the grid).
//
// Per tile of T window positions (never crossing a run): K is staged in LDS
// row-major (f16, or q8_0 codes widened to f16 exactly plus one f32 scale per
// (position, 32-wide block)); V row-major.  Tiles are double-buffered: the
// loads of the next tile are in flight while the current one is computed,
// and the block-table entries are fetched two tiles ahead.  Scores are
// computed transposed, S^T = K Q^T, so each lane holds T/4 scores of one row
// (positions g + 4j of the tile for lane group g): the row's running max and
// sum live in the lane and the rounded probabilities are already the B
// operand of O^T = V^T P^T, whose A operand gathers one head_dim column of V
// over positions g + 4j with 16-bit LDS reads (rows g and g + 1 are 8 banks
// apart, so the four lane groups never collide).  For q8_0 K every 32-wide
// head_dim block is one MFMA whose result is scaled by that position's block
// scale before it is added: the dequantised value scale * code is never
// rounded to f16.  Positions outside the run, in a hole or past a row's
// causal limit get probability 0 by selection; a tile with none of these
// skips the masking.  Staged K/V of such positions are zeros.
#include "pkv_internal.hpp"

namespace pkv {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kPWaves = 4;      // waves per workgroup
constexpr int kRowTiles = 2;    // 16-row tiles per wave
constexpr int kRowsWG = kPWaves * kRowTiles * 16;
constexpr float kEmptyMax = -1e30f;
constexpr int kTargetTasks = 1024;  // workgroups the chunking aims for
constexpr int kMaxChunks = 16;
constexpr float kLazyMax = 8.0f;    // log2 growth of a row max that forces a rescale

// V is stored for the PV A operand: word i of (32-position half kh, lane
// group g, column d) holds the f16 pair (V[32 kh + g + 8 i][d],
// V[32 kh + g + 8 i + 4][d]), the four words of a (kh, g, d) are one 16-byte
// read, and every eighth column is followed by a 16-byte gap so that the
// staging writes (16 columns apart) spread over the banks.
template <int HD, int T>
struct __attribute__((aligned(16))) PrefillSmem {
  static constexpr int KLD = HD + 8;         // K row stride (halfs): 16-byte rows, 4 banks apart
  static constexpr int VDP = HD + HD / 8;    // padded columns per (kh, g)
  _Float16 k[2][T][KLD];
  uint32_t v[2][T / 32][4][VDP][4];
  float ks[2][HD / 32][T];  // q8_0 block scales, in the order the score lanes read them
  int32_t id[2][T];         // physical block of each staged position, -1 = not visible
  int32_t lim_max;          // largest causal limit of the workgroup's rows
};

__device__ __forceinline__ float4_t mfma16x16x32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Four int8 codes (one dword) to four exactly equal f16 values: with the sign
// bit flipped a code is u = code + 128 in [0, 255], the f16 with bits
// 0x6400 | u is 1024 + u, and subtracting 1152 is exact.
__device__ __forceinline__ void codes_to_f16(uint32_t x, half2_t& lo, half2_t& hi) {
  const uint32_t y = x ^ 0x80808080u;
  const uint32_t plo = __builtin_amdgcn_perm(0x64646464u, y, 0x04010400u);
  const uint32_t phi = __builtin_amdgcn_perm(0x64646464u, y, 0x04030402u);
  const half2_t bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(half2_t, plo) - bias;
  hi = __builtin_bit_cast(half2_t, phi) - bias;
}

// This workgroup's walk over the window: runs in order, each clipped to
// [0, lim), as one concatenated index space of which [va, vend) is ours.
// All fields are wave-uniform.
struct Walk {
  int32_t r;       // current run (== n_runs: finished)
  int32_t vb;      // index-space offset of run r
  int32_t len;     // clipped length of run r
  int32_t lo, hi;  // our positions of run r
  int32_t t0;      // current tile start
};

__device__ inline void walk_seek(const AttnArgs& a, int s, int32_t lim, int32_t va, int32_t vend,
                                 Walk& w) {
  while (w.r < a.n_runs) {
    int32_t ra, rb;
    run_range(a, s, w.r, lim, ra, rb);
    ra = uni(ra);
    rb = uni(rb);
    w.len = rb - ra;
    const int32_t v0 = va > w.vb ? va : w.vb;
    const int32_t v1 = vend < w.vb + w.len ? vend : w.vb + w.len;
    if (v0 < v1) {
      w.lo = ra + (v0 - w.vb);
      w.hi = ra + (v1 - w.vb);
      w.t0 = w.lo;
      return;
    }
    w.vb += w.len;
    ++w.r;
  }
}

template <int T>
__device__ inline void walk_next(const AttnArgs& a, int s, int32_t lim, int32_t va, int32_t vend,
                                 Walk& w) {
  if (w.r >= a.n_runs) return;
  w.t0 += T;
  if (w.t0 < w.hi) return;
  w.vb += w.len;
  ++w.r;
  walk_seek(a, s, lim, va, vend, w);
}

template <int HD, int BS, int G, bool KQ8, int T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HD <= 128 ? 2 : 1, HD <= 128 ? 2 : 1)))
void prefill_kernel(AttnArgs a, int32_t n_tasks, int32_t nqb) {
  constexpr int KS = HD / 32;                     // MFMA k-steps over head_dim
  constexpr int DT = HD / 16;                     // 16-wide head_dim tiles of the output
  constexpr int CHR = HD / 8;                     // 16-byte chunks per f16 row
  constexpr int QPB = kRowsWG / G;                // queries per workgroup
  constexpr int NKH = T / 32;                     // 32-position halves of a tile
  constexpr int NJ = T / 4;                       // scores per lane per row tile
  constexpr int NCH = (T * CHR + 255) / 256;      // f16 row chunks per thread
  constexpr int UPR = HD / 16;                    // q8_0 half blocks per row
  constexpr int NQ8 = (T * UPR + 255) / 256;      // q8_0 half blocks per thread
  constexpr int NID = (T + BS - 1) / BS + 1;      // table entries one tile can touch
  static_assert(T == 32 || T == 64, "tile");
  __shared__ __attribute__((aligned(16))) PrefillSmem<HD, T> sm;

  // ---- task: ((s * Hkv + kvh) * nch + c) * nqb + qb, XCD-major numbering
  const int32_t n8 = (n_tasks + 7) >> 3;
  const int32_t u = (int32_t)(blockIdx.x & 7) * n8 + (int32_t)(blockIdx.x >> 3);
  if (u >= n_tasks) return;
  const int qb = u % nqb;
  int32_t rest = u / nqb;
  const int c = rest % a.nch;
  rest /= a.nch;
  const int kvh = rest % a.n_kv_heads;
  const int s = rest / a.n_kv_heads;

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
  bool rok[kRowTiles];
  int32_t lim[kRowTiles];
  half8_t qf[kRowTiles][KS];
  if (t == 0) sm.lim_max = 0;
  __syncthreads();
  int32_t lmin = 0x7fffffff;
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    const int rr = w * 32 + rt * 16 + n16;
    jq[rt] = j0 + rr / G;
    hq[rt] = rr % G;
    rok[rt] = rr < QPB * G && jq[rt] < j1;
    int64_t lm = 0;
    if (rok[rt]) {
      lm = (int64_t)a.q_pos[jq[rt]] + 1;
      if (lm > L) lm = L;
      if (lm < 0) lm = 0;
    }
    lim[rt] = (int32_t)lm;
    if (rok[rt] && lim[rt] < lmin) lmin = lim[rt];
    const _Float16* qrow =
        (const _Float16*)a.q + ((int64_t)(rok[rt] ? jq[rt] : 0) * a.n_q_heads + kvh * G + hq[rt]) * HD;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      half8_t v = {};
      if (rok[rt]) v = *(const half8_t*)(qrow + ks * 32 + g * 8);
      qf[rt][ks] = a.score_mul < 0.f ? -v : v;  // a negative scale: negate q (exact), use |scale|
    }
    if (rok[rt]) atomicMax(&sm.lim_max, lim[rt]);
  }
  // smallest causal limit over the wave's rows (wave-uniform)
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int32_t o = __shfl_xor(lmin, m, 64);
    lmin = o < lmin ? o : lmin;
  }
  const int32_t lim_min_w = uni(lmin);
  __syncthreads();
  const int32_t lim_max = uni(sm.lim_max);

  // ---- this workgroup's chunk of the window
  int32_t W = 0;
  for (int r = 0; r < a.n_runs; ++r) {
    int32_t ra, rb;
    run_range(a, s, r, lim_max, ra, rb);
    W += rb - ra;
  }
  W = uni(W);
  const int32_t chl = ((W + a.nch - 1) / a.nch + T - 1) / T * T;
  const int32_t va = c * chl, vend = va + chl < W ? va + chl : W;

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
  const bool count_bad = kvh == 0 && qb == 0 && t == 0;
  // |scale| * log2(e), kept above 0 so that a hidden score (-inf) always
  // gives p = 0 (a zero scale then weighs every visible position equally)
  const float mul = fmaxf(fabsf(a.score_mul), 1e-30f);

  // table entries of the blocks a tile touches, loaded raw (wave-uniform
  // addresses) a tile before they are used, and checked when used
  auto load_ids = [&](const Walk& x, int32_t (&ids)[NID]) {
    const int32_t b0 = x.t0 / BS;
    const int32_t te = x.t0 + T < x.hi ? x.t0 + T : x.hi;
    const int32_t blast = (te - 1) / BS;
    const int32_t* row = a.table + (int64_t)s * a.max_blocks;
#pragma unroll
    for (int i = 0; i < NID; ++i) ids[i] = b0 + i <= blast ? row[b0 + i] : -1;
  };
  const bool checked = (a.flags & PKV_FLAG_CHECKED) && a.err && kvh == 0 && qb == 0;
  auto check_ids = [&](const Walk& x, int32_t (&ids)[NID]) {
    const int32_t b0 = x.t0 / BS;
    int bad = 0;
#pragma unroll
    for (int i = 0; i < NID; ++i) {
      const int32_t id = uni(ids[i]);
      const bool out = id < -1 || id >= a.n_pool_blocks;
      // count a bad entry once: in the tile holding the block's first visible position
      if (out && ((b0 + i) * BS >= x.t0 || x.t0 == x.lo)) ++bad;
      ids[i] = (id < 0 || out) ? -1 : id;
    }
    if (checked && bad) {
      if (t == 0) atomicAdd(a.err, bad);
    }
  };

  // staged data of one tile, in registers between load and LDS store
  constexpr int NVU = (T / 2 * CHR + 255) / 256;  // V units (position pair, 8 columns) per thread
  uint4 vr[NVU][2];
  uint4 kr[KQ8 ? 1 : NCH];
  uint32_t qw[KQ8 ? NQ8 : 1][5];
  int32_t vid[NVU][2], kid[KQ8 ? NQ8 : NCH];

  auto pick = [&](const int32_t (&ids)[NID], int32_t i) {
    int32_t id = ids[0];
#pragma unroll
    for (int k = 1; k < NID; ++k) id = i == k ? ids[k] : id;
    return id;
  };
  // Loads are unconditional (a position that is not visible reads block 0,
  // which always exists, and is zeroed when stored) so that no lane-divergent
  // branch sits between the loads and the compute they overlap.  A lane's
  // address is one of the tile's (at most NID) block bases plus a 32-bit
  // offset inside the block.
  auto stage_issue = [&](const Walk& x, const int32_t (&ids)[NID]) {
    const int32_t te = x.t0 + T < x.hi ? x.t0 + T : x.hi;
    const int32_t b0 = x.t0 / BS;
    // block bases (wave-uniform); a hole reads block 0
    const unsigned char* vb[NID];
    const unsigned char* kb[NID];
#pragma unroll
    for (int i = 0; i < NID; ++i) {
      const int64_t idc = ids[i] >= 0 ? ids[i] : 0;
      vb[i] = vbase + idc * a.v_block_bytes;
      kb[i] = kbase + idc * a.k_block_bytes;
    }
    auto sel = [&](const unsigned char* const (&bases)[NID], int32_t bi) {
      const unsigned char* p = bases[0];
#pragma unroll
      for (int k = 1; k < NID; ++k) p = bi == k ? bases[k] : p;
      return p;
    };
#pragma unroll
    for (int e = 0; e < NVU; ++e) {
      const int uv = t + 256 * e;
      const int pr = uv / CHR, ch = uv - pr * CHR;  // pair pr = (kh, g, i)
      const int p0 = 32 * (pr >> 4) + ((pr >> 2) & 3) + 8 * (pr & 3);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int32_t pos = x.t0 + p0 + 4 * h;
        const int32_t bi = pos / BS - b0;
        vid[e][h] = uv < T / 2 * CHR && pos < te ? pick(ids, bi) : -1;
        const uint32_t off = (uint32_t)(pos % BS) * (uint32_t)a.v_seg_bytes + ch * 16;
        vr[e][h] = *(const uint4*)(sel(vb, bi) + off);
      }
    }
    if constexpr (!KQ8) {
#pragma unroll
      for (int e = 0; e < NCH; ++e) {
        const int cc = t + 256 * e;
        const int p = cc / CHR, ch = cc - p * CHR;
        const int32_t pos = x.t0 + p;
        const int32_t bi = pos / BS - b0;
        kid[e] = cc < T * CHR && pos < te ? pick(ids, bi) : -1;
        const uint32_t off = (uint32_t)(pos % BS) * (uint32_t)a.k_seg_bytes + ch * 16;
        kr[e] = *(const uint4*)(sel(kb, bi) + off);
      }
    } else {
#pragma unroll
      for (int e = 0; e < NQ8; ++e) {
        const int uq = t + 256 * e;
        const int p = uq / UPR, rem = uq - p * UPR;
        const int bq = rem >> 1, h = rem & 1;
        const int32_t pos = x.t0 + p;
        const int32_t bi = pos / BS - b0;
        kid[e] = uq < T * UPR && pos < te ? pick(ids, bi) : -1;
        // bytes [lb, lb + 18) of the segment: f16 scale (used when h == 0)
        // then 16 codes; lb is even, read as five aligned dwords
        const int lb = 34 * bq + 16 * h;
        const uint32_t off = (uint32_t)(pos % BS) * (uint32_t)a.k_seg_bytes + (lb & ~3);
        const uint32_t* src = (const uint32_t*)(sel(kb, bi) + off);
#pragma unroll
        for (int i = 0; i < 5; ++i) qw[e][i] = src[i];
      }
    }
  };

  auto keep = [](bool ok, uint4 x) {
    return make_uint4(ok ? x.x : 0u, ok ? x.y : 0u, ok ? x.z : 0u, ok ? x.w : 0u);
  };
  auto stage_store = [&](int b) {
#pragma unroll
    for (int e = 0; e < NVU; ++e) {
      const int uv = t + 256 * e;
      if (uv < T / 2 * CHR) {
        const int pr = uv / CHR, ch = uv - pr * CHR;
        const int kh = pr >> 4, gg = (pr >> 2) & 3, i = pr & 3;
        const uint4 x0 = keep(vid[e][0] >= 0, vr[e][0]);
        const uint4 x1 = keep(vid[e][1] >= 0, vr[e][1]);
        const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w}, a1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // columns 8 ch + 2 k and 8 ch + 2 k + 1: low halves, then high halves
          const int d = 8 * ch + 2 * k;
          const int dp = d + (d >> 3);
          sm.v[b][kh][gg][dp][i] = __builtin_amdgcn_perm(a1[k], a0[k], 0x05040100u);
          sm.v[b][kh][gg][dp + 1][i] = __builtin_amdgcn_perm(a1[k], a0[k], 0x07060302u);
        }
        if (ch == 0) {
          const int p0 = 32 * kh + gg + 8 * i;
          sm.id[b][p0] = vid[e][0];
          sm.id[b][p0 + 4] = vid[e][1];
        }
      }
    }
    if constexpr (!KQ8) {
#pragma unroll
      for (int e = 0; e < NCH; ++e) {
        const int cc = t + 256 * e;
        if (cc < T * CHR) {
          const int p = cc / CHR, ch = cc - p * CHR;
          *(uint4*)&sm.k[b][p][ch * 8] = keep(kid[e] >= 0, kr[e]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < NQ8; ++e) {
        const int uq = t + 256 * e;
        if (uq < T * UPR) {
          const int p = uq / UPR, rem = uq - p * UPR;
          const int bq = rem >> 1, h = rem & 1;
          const int sh = (34 * bq + 16 * h) & 3;  // 0 or 2
          const bool ok = kid[e] >= 0;
          uint32_t cw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            cw[i] = sh ? qw[e][i + 1] : __builtin_amdgcn_alignbyte(qw[e][i + 1], qw[e][i], 2);
            cw[i] = ok ? cw[i] : 0u;
          }
          half2_t hv[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) codes_to_f16(cw[i], hv[2 * i], hv[2 * i + 1]);
          half8_t lo8 = {hv[0][0], hv[0][1], hv[1][0], hv[1][1], hv[2][0], hv[2][1], hv[3][0], hv[3][1]};
          half8_t hi8 = {hv[4][0], hv[4][1], hv[5][0], hv[5][1], hv[6][0], hv[6][1], hv[7][0], hv[7][1]};
          *(half8_t*)&sm.k[b][p][32 * bq + 16 * h] = lo8;
          *(half8_t*)&sm.k[b][p][32 * bq + 16 * h + 8] = hi8;
          if (h == 0) {
            const uint32_t sw = ok ? (sh ? (qw[e][0] >> 16) : (qw[e][0] & 0xFFFFu)) : 0u;
            const int pidx = (p >> 4) * 16 + (p & 3) * 4 + ((p >> 2) & 3);
            sm.ks[b][bq][pidx] = (float)__builtin_bit_cast(_Float16, (unsigned short)sw);
          }
        }
      }
    }
  };

  auto compute = [&](int b, const Walk& x) {
    // validity of the tile's positions (wave-uniform bit mask)
    const uint64_t vm = __builtin_amdgcn_ballot_w64(sm.id[b][l % T] >= 0);
    const uint64_t all = T == 64 ? ~0ull : 0xffffffffull;
    const bool full = (vm & all) == all && x.t0 + T <= lim_min_w;

    // S^T = K Q^T: for 16-position tile st the lane holds positions
    // 16 st + g + 4 i (i = 0..3) of row n16; sc[rt][4 st + i]
    float sc[kRowTiles][NJ];
#pragma unroll
    for (int st = 0; st < T / 16; ++st) {
      const int krow = 16 * st + (n16 >> 2) + 4 * (n16 & 3);
      float4_t acc[kRowTiles];
#pragma unroll
      for (int rt = 0; rt < kRowTiles; ++rt) acc[rt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const half8_t af = *(const half8_t*)&sm.k[b][krow][ks * 32 + g * 8];
        if constexpr (!KQ8) {
#pragma unroll
          for (int rt = 0; rt < kRowTiles; ++rt) acc[rt] = mfma16x16x32(af, qf[rt][ks], acc[rt]);
        } else {
          const float4_t scl = *(const float4_t*)&sm.ks[b][ks][st * 16 + g * 4];
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
        for (int i = 0; i < 4; ++i) sc[rt][4 * st + i] = acc[rt][i];
      __builtin_amdgcn_sched_barrier(0);  // bounds the fragments in flight (register pressure)
    }

    // ---- online softmax per row (the four lane groups hold the same row).
    // The running max moves lazily: only when a row's max would grow by more
    // than 2^8, so p stays <= 256 (exact enough in f16) and the output is
    // rarely rescaled.  Hidden positions score -inf and so get p = 0.
    half8_t pf[kRowTiles][NKH];
#pragma unroll
    for (int rt = 0; rt < kRowTiles; ++rt) {
      if (!full) {
        // score jj is position p = 16 (jj / 4) + g + 4 (jj % 4) of the tile
        const uint32_t vg = (uint32_t)(vm >> g);
        const int32_t lr = lim[rt] - x.t0 - g;
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
          const int pc = 16 * (jj >> 2) + 4 * (jj & 3);
          const bool ok = ((vg >> pc) & 1u) && pc < lr;
          sc[rt][jj] = ok ? sc[rt][jj] : -INFINITY;
        }
      }
      float mx = sc[rt][0];
#pragma unroll
      for (int jj = 1; jj < NJ; ++jj) mx = fmaxf(mx, sc[rt][jj]);
      mx = fmaxf(mx, shfl_xor(mx, 16));
      mx = fmaxf(mx, shfl_xor(mx, 32));
      const float mc = mx * mul;
      const bool grow = mc > m[rt] + kLazyMax;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float mn = grow ? mc : m[rt];
        const float alpha = fast_exp2(m[rt] - mn);
        lsum[rt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= alpha;
        m[rt] = mn;
      }
#pragma unroll
      for (int jj = 0; jj < NJ; ++jj) {
        const float p = fast_exp2(fmaf(sc[rt][jj], mul, -m[rt]));
        lsum[rt] += p;
        pf[rt][jj >> 3][jj & 7] = (_Float16)p;
      }
    }

    __builtin_amdgcn_sched_barrier(0);
    // ---- O^T += V^T P^T over each 32-position half: A gathers column d of V
    // at positions 32 kh + g + 4 j
#pragma unroll
    for (int kh = 0; kh < NKH; ++kh) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = dt * 16 + n16;
        const half8_t vf = *(const half8_t*)&sm.v[b][kh][g][d + (d >> 3)][0];
#pragma unroll
        for (int rt = 0; rt < kRowTiles; ++rt) o[rt][dt] = mfma16x16x32(vf, pf[rt][kh], o[rt][dt]);
      }
    }
  };

  // ---- pipeline over the chunk's tiles
  Walk wc{0, 0, 0, 0, 0, 0};
  if (va < vend) walk_seek(a, s, lim_max, va, vend, wc);
  else wc.r = a.n_runs;
  if (wc.r < a.n_runs) {
    int32_t ids[NID], idn[NID];
    load_ids(wc, ids);
    check_ids(wc, ids);
    stage_issue(wc, ids);
    stage_store(0);
    Walk wn = wc;
    walk_next<T>(a, s, lim_max, va, vend, wn);
    if (wn.r < a.n_runs) load_ids(wn, idn);
    __syncthreads();
    int b = 0;
    for (;;) {
      const bool more = wn.r < a.n_runs;
      Walk wnn = wn;
      walk_next<T>(a, s, lim_max, va, vend, wnn);
      int32_t idnn[NID];
      if (wnn.r < a.n_runs) load_ids(wnn, idnn);
      if (more) {
        check_ids(wn, idn);
        stage_issue(wn, idn);
      }
      compute(b, wc);
      if (more) stage_store(b ^ 1);
      __syncthreads();
      if (!more) break;
      wc = wn;
      wn = wnn;
#pragma unroll
      for (int i = 0; i < NID; ++i) idn[i] = idnn[i];
      b ^= 1;
    }
  }

  // ---- finish: sum the row's lane groups; write the output or the partial
#pragma unroll
  for (int rt = 0; rt < kRowTiles; ++rt) {
    float ls = lsum[rt];
    ls += shfl_xor(ls, 16);
    ls += shfl_xor(ls, 32);
    if (!rok[rt]) continue;
    const bool empty = m[rt] == kEmptyMax;
    const int64_t row = (int64_t)jq[rt] * a.n_q_heads + kvh * G + hq[rt];
    if (a.nch == 1) {
      const float inv = empty ? 0.f : 1.f / ls;
      float* orow = a.out + row * HD;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const float4_t v = o[rt][dt] * inv;
        *(float4*)(orow + dt * 16 + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (a.lse && g == 0) a.lse[row] = empty ? -INFINITY : (m[rt] + __builtin_amdgcn_logf(ls)) * kLn2;
    } else {
      const int64_t pr = row * a.nch + c;
      if (g == 0) *(float2*)(a.part_ml + pr * 2) = make_float2(m[rt], empty ? 0.f : ls);
      if (!empty) {
        float* orow = a.part_o + pr * HD;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *(float4*)(orow + dt * 16 + 4 * g) = make_float4(o[rt][dt][0], o[rt][dt][1], o[rt][dt][2], o[rt][dt][3]);
      }
    }
  }
}

// Combine the chunk partials of each (query, q head) row:
// M = max_c m_c, L = sum_c l_c 2^(m_c - M), out = sum_c 2^(m_c - M) O_c / L,
// lse = (M + log2 L) ln 2; chunks that saw nothing (m_c empty) carry no
// weight and their output slots are never read.  grid (row blocks, S).
template <int HD>
__global__ __launch_bounds__(256) void prefill_merge_kernel(AttnArgs a) {
  constexpr int TPR = HD / 4;      // threads per row, 4 dims each
  constexpr int RPB = 256 / TPR;   // rows per block
  const int s = blockIdx.y;
  int q0 = a.cu_q[s], q1 = a.cu_q[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > a.n_q_total ? a.n_q_total : q0);
  q1 = q1 < q0 ? q0 : (q1 > a.n_q_total ? a.n_q_total : q1);
  if (q1 > q0 + a.max_q) q1 = q0 + a.max_q;
  const int64_t nrow = (int64_t)(q1 - q0) * a.n_q_heads;
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  if (r >= nrow) return;
  const int d4 = threadIdx.x % TPR;
  const int64_t row = (int64_t)q0 * a.n_q_heads + r;
  const float* ml = a.part_ml + row * a.nch * 2;
  float M = kEmptyMax;
  for (int c = 0; c < a.nch; ++c) M = fmaxf(M, ml[2 * c]);
  float* orow = a.out + row * HD + 4 * d4;
  if (M == kEmptyMax) {
    *(float4*)orow = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.lse && d4 == 0) a.lse[row] = -INFINITY;
    return;
  }
  float Ls = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c = 0; c < a.nch; ++c) {
    const float mc = ml[2 * c];
    if (mc == kEmptyMax) continue;
    const float wgt = fast_exp2(mc - M);
    Ls += ml[2 * c + 1] * wgt;
    const float4 v = *(const float4*)(a.part_o + (row * a.nch + c) * HD + 4 * d4);
    acc.x += wgt * v.x;
    acc.y += wgt * v.y;
    acc.z += wgt * v.z;
    acc.w += wgt * v.w;
  }
  const float inv = 1.f / Ls;
  *(float4*)orow = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (a.lse && d4 == 0) a.lse[row] = (M + __builtin_amdgcn_logf(Ls)) * kLn2;
}

namespace {

constexpr int tile_for(int hd) { return hd <= 128 ? 32 : 32; }

// Chunks per window: enough workgroups to fill the chip twice over, each
// chunk still at least four tiles of the largest possible window.
int plan_chunks(const AttnArgs& a, int hd, int g) {
  const int T = tile_for(hd);
  const int qpb = kRowsWG / g;
  const int64_t nqb = ((int64_t)a.max_q + qpb - 1) / qpb;
  const int64_t base = (int64_t)a.n_seqs * a.n_kv_heads * (nqb > 0 ? nqb : 1);
  int64_t nch = (kTargetTasks + base - 1) / base;
  if (nch > kMaxChunks) nch = kMaxChunks;
  const int64_t wmax = (int64_t)(a.mode == PKV_WIN_KV_MAP ? a.n_runs : 1) * a.max_blocks * a.block_size;
  const int64_t cap = wmax / (4 * T);
  if (nch > cap) nch = cap;
  return nch < 1 ? 1 : (int)nch;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t prefill_workspace(const AttnArgs& a, int combo, int hd, int bs, int g, bool* found) {
  (void)bs;
  *found = combo == kComboF16 || combo == kComboQ8H;
  if (!*found) return 0;
  const int nch = plan_chunks(a, hd, g);
  size_t need = 0;
  if (nch > 1) {
    const size_t rows = (size_t)a.n_q_total * a.n_q_heads * nch;
    need = align256(rows * 2 * sizeof(float)) + align256(rows * hd * sizeof(float));
  }
  if (a.flags & PKV_FLAG_CHECKED) need += 256;
  return need;
}

hipError_t launch_prefill(const AttnArgs& a0, int combo, int hd, int bs, int g, hipStream_t st,
                          bool* found) {
  *found = false;
  if (combo != kComboF16 && combo != kComboQ8H) return hipSuccess;
  const bool q8 = combo == kComboQ8H;
  AttnArgs a = a0;
  a.nch = plan_chunks(a, hd, g);
  if (a.nch > 1) {
    const size_t rows = (size_t)a.n_q_total * a.n_q_heads * a.nch;
    unsigned char* base = (unsigned char*)a0.part_o;
    a.part_ml = (float*)base;
    a.part_o = (float*)(base + align256(rows * 2 * sizeof(float)));
  }
  const int qpb = kRowsWG / g;
  const int32_t nqb = (a.max_q + qpb - 1) / qpb;
  const int64_t n_tasks = (int64_t)a.n_seqs * a.n_kv_heads * a.nch * nqb;
  if (n_tasks > (int64_t)1 << 28) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((n_tasks + 7) / 8 * 8));
#define PKV_PCASE(HD, BS, G)                                                                          \
  if (hd == HD && bs == BS && g == G) {                                                               \
    constexpr int T = tile_for(HD);                                                                   \
    if (q8)                                                                                           \
      hipLaunchKernelGGL((prefill_kernel<HD, BS, G, true, T>), grid, dim3(256), 0, st, a,             \
                         (int32_t)n_tasks, nqb);                                                      \
    else                                                                                              \
      hipLaunchKernelGGL((prefill_kernel<HD, BS, G, false, T>), grid, dim3(256), 0, st, a,            \
                         (int32_t)n_tasks, nqb);                                                      \
    *found = true;                                                                                    \
  }
#define PKV_PCASES_G(HD, BS) PKV_PCASE(HD, BS, 1) PKV_PCASE(HD, BS, 2) PKV_PCASE(HD, BS, 3) PKV_PCASE(HD, BS, 4) PKV_PCASE(HD, BS, 8)
  PKV_PCASES_G(64, 16)
  PKV_PCASES_G(128, 16)
  PKV_PCASES_G(256, 16)
  PKV_PCASES_G(128, 32)
#undef PKV_PCASES_G
#undef PKV_PCASE
  if (!*found) return hipSuccess;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nch == 1) return e;
  const int rpb = 256 / (hd / 4);
  const dim3 mgrid((unsigned)(((int64_t)a.max_q * a.n_q_heads + rpb - 1) / rpb), (unsigned)a.n_seqs);
  if (hd == 64) hipLaunchKernelGGL(prefill_merge_kernel<64>, mgrid, dim3(256), 0, st, a);
  else if (hd == 128) hipLaunchKernelGGL(prefill_merge_kernel<128>, mgrid, dim3(256), 0, st, a);
  else hipLaunchKernelGGL(prefill_merge_kernel<256>, mgrid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pkv
