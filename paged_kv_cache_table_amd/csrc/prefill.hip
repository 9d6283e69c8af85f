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
// Work decomposition.  A workgroup (8 waves, two per SIMD) takes one kv
// head, a block of consecutive queries of one sequence (rows = (query, q head
// of the GQA group) pairs, 16 * RT per wave) and one of nch chunks of the
// window.  Each run of the window, clipped to [0, min(seq_len, largest causal
// limit of the rows)), is covered by the T-aligned tiles that meet it; the
// runs' tiles in order form one list that is cut into nch equal chunks.  With
// nch > 1 each workgroup writes (max, sum, unnormalised output) per row and a
// merge kernel combines them with the log-sum-exp rule; with nch = 1 the
// output is written directly.  A one-workgroup kernel first orders the
// sequences by their number of window tiles; workgroups are numbered longest
// sequence first, so that the longest chunks start first and shorter ones
// fill the machine behind them.
//
// Data movement.  A tile is T/BS whole blocks.  Each wave copies its T/8
// positions of a tile (which lie in one block: one scalar base address per
// tile, fixed per-lane offsets) straight from HBM into LDS
// (global_load_lds: no registers in between), three tiles ahead of the
// compute, into a ring of four tile slots; it then waits for its own copies
// only (vmcnt) and prepares its rows (V rows of positions that are not
// visible zeroed; q8_0 K rows become their int8 codes as f16, which is exact,
// and the block scales are kept apart as f32), so one barrier per tile
// suffices.  f16 rows are stored row-major with their 16-byte chunks
// XOR-permuted by a key of the row (swz_key), which keeps the score-operand
// reads, the transposing V reads and the q8_0 expansion writes free of bank
// conflicts.
//
// Compute.  Scores are computed transposed, S^T = K Q^T, so each lane holds
// T/4 scores of one row (positions 16 st + 4 g + i): the row's running max
// and sum live in the lane and the rounded probabilities are already the B
// operand of O^T = V^T P^T.  Its A operand (a head_dim column of V over those
// positions) comes from ds_read_b64_tr_b16: within each 16-lane group, lane i
// receives element i % 4 of the 4 halves that lane 4 e + i / 4 addressed, as
// element e.  For q8_0 K each 32-wide MFMA k-step covers exactly one q8_0
// block of every position, so it multiplies the codes (exact in f16) by q
// and the block scale of each position is applied to that partial in f32:
// no product of scale and code is ever formed in f16, whatever the scale
// (any f16 value, 65504 included).  The row sums of
// the rounded probabilities come from one more MFMA per PV step whose A
// operand is all ones (the same rounded values as the numerator).  Positions
// outside the run, in a hole or past a row's causal limit score -inf; a tile
// with none of these skips the masking.
#include "pkv_internal.hpp"


namespace pkv {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4_t;

constexpr int kPWaves = 8;          // waves per workgroup (two per SIMD)
constexpr int kRing = 4;            // LDS tile slots: copies run three tiles ahead
constexpr float kEmptyMax = -1e30f;
constexpr float kLazyMax = 8.0f;    // log2 growth of a row max that forces a rescale
constexpr int kTargetTasks = 384;   // workgroups the chunking aims for (1.5 per CU)
constexpr int kMaxChunks = 16;      // unless a chunk would exceed kMaxTiles
constexpr int kMaxTiles = 256;      // tiles of one workgroup's chunk (its list lives in LDS)

// One tile of a workgroup's chunk, described once before the main loop: its
// first position (a multiple of the tile size), the visibility mask of its
// positions (inside the run, not in a hole) and its checked block ids
// (-1: hole or out of range).
struct __attribute__((aligned(16))) TileRec {
  int32_t t0;
  uint32_t vm_lo, vm_hi;
  int32_t pad;
  int32_t blk[4];
};

// Tile shape per head_dim: positions per tile and 16-row tiles per wave.
__host__ __device__ constexpr int tile_of(int hd) { return hd <= 128 ? 64 : 32; }
__host__ __device__ constexpr int row_tiles_of(int hd) { return hd <= 128 ? 2 : 1; }
__host__ __device__ constexpr int rows_per_wg(int hd) { return kPWaves * row_tiles_of(hd) * 16; }

template <int HD>
struct PGeom {
  static constexpr int T = tile_of(HD);                      // window positions per tile
  static constexpr int RT = row_tiles_of(HD);                // 16-row tiles per wave
  static constexpr int PPW = T / kPWaves;                    // positions each wave copies and prepares
  static constexpr int KS = HD / 32;                         // q8_0 blocks / MFMA k-steps
  static constexpr int CHR = HD / 8;                         // 16-byte chunks per f16 row
  static constexpr int ROWB = HD * 2;                        // bytes per f16 row
  static constexpr int TILEB = T * ROWB;                     // bytes per f16 tile
  static constexpr int NV = PPW * CHR / 64;                  // 16-byte copies per wave per f16 tile
  static constexpr int SEG8 = (KS * 34 + 3) / 4 * 4;         // bytes per q8_0 segment
  static constexpr int RAWW = PPW * SEG8;                    // bytes of a wave's q8_0 rows
  static constexpr int CPW = RAWW / 16;                      // their 16-byte chunks
  static constexpr int NRW = (CPW + 63) / 64;                // 16-byte copies per wave per q8_0 tile
  static constexpr int UPR = HD / 16;                        // q8_0 half blocks per position (even)
  static constexpr int NQ8 = (PPW * UPR + 63) / 64;          // half blocks per lane
  static_assert(PPW * CHR % 64 == 0 && RAWW % 16 == 0, "copy shapes");
};

template <int HD, bool KQ8>
struct __attribute__((aligned(16))) PrefillSmem {
  using Gm = PGeom<HD>;
  unsigned char v[kRing][Gm::TILEB];                                  // V tiles
  // K tiles: f16 as copied, or the int8 codes of q8_0 rows as f16 values
  unsigned char k[KQ8 ? 2 : kRing][Gm::TILEB];
  // q8_0: the block scales as f32, [ks][position] (4 consecutive positions
  // of one k-step are one 16-byte read)
  float ksc[KQ8 ? 2 : 1][KQ8 ? Gm::KS : 1][KQ8 ? Gm::T : 4];
  unsigned char raw[KQ8 ? kRing : 1][KQ8 ? kPWaves * Gm::RAWW : 16];  // q8_0 tiles as stored
  TileRec tiles[kMaxTiles];                                           // this workgroup's chunk
  int32_t lim_max[kPWaves];                                           // each wave's largest causal limit
};

// Row r's 16-byte chunks are stored XOR-permuted by a key of the row so that
// the tile's LDS reads are free of bank conflicts.  Measured on gfx950 (LDS
// bank-conflict counters over probe patterns): 16-byte reads serve 16 lanes
// a cycle over 64 banks of 4 bytes, the lane eighths paired as {0,3}, {1,2},
// {4,7}, {5,6}; 8-byte reads, transposing ones included, serve lanes 0-31
// and then 32-63 over 64 banks; 16-byte writes serve 8 consecutive lanes a
// cycle over 32 banks.  K is read one chunk index across 16 consecutive rows
// (the paired eighths: rows 0-7 at chunk c, rows 8-15 at chunk c ^ 1); V is
// read one 32-byte chunk pair across 8 consecutive rows.  With 256-byte rows
// (head_dim 128) the key 2 (r mod 8) puts the 8 rows' chunk pairs apart and
// rows 0-7 on even chunk positions where rows 8-15 sit on odd ones.  With
// 128-byte rows two rows share the 64 banks and the key r mod 8 does both.
template <int HD>
__host__ __device__ __forceinline__ int swz_key(int r) {
  return (r & 7) << (PGeom<HD>::CHR >= 16 ? 1 : 0);
}

// Byte offset of 16-byte chunk c of row r in an f16 tile.
template <int HD>
__device__ __forceinline__ int swz(int r, int c) {
  return r * PGeom<HD>::ROWB + ((c ^ swz_key<HD>(r)) << 4);
}

__device__ __forceinline__ float4_t mfma16x16x32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int32_t uni(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }

// Max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane groups): each
// swap exchanges the odd rows (or the upper half) of one copy of the value
// with the even rows (lower half) of another copy, so the two registers then
// hold the value of the lane and of its partner.  Written as inline assembly
// with both registers as outputs: the compiler's builtin for these swaps
// returns the first register for both results.
__device__ __forceinline__ float max_over_groups(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 0\n\tv_max_f32 %0, %0, %1" : "+v"(a), "+v"(b));
  b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 0\n\tv_max_f32 %0, %0, %1" : "+v"(a), "+v"(b));
  return a;
}

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

// Run r of sequence s as stored, [x0, x1) before clipping (same rule as
// run_range; reads the window through a pointer the compiler may load with
// scalar loads).  Causal mode has one run, [0, any limit).
__device__ inline void raw_run(const AttnArgs& a, const int32_t* __restrict__ window, int s, int r, int64_t& x0,
                               int64_t& x1) {
  x0 = 0;
  x1 = 0;
  if (a.mode == PKV_WIN_CAUSAL) {
    x1 = INT64_MAX;
  } else if (a.mode == PKV_WIN_SPAN) {
    x0 = window[2 * s];
    x1 = window[2 * s + 1];
  } else {
    const int32_t* wr = window + ((int64_t)s * a.n_runs + r) * 2;
    const int64_t c = wr[0], n = wr[1];
    if (n > 0) {
      x0 = c;
      x1 = c + n;
    }
  }
}

// The runs of a sequence's window, clipped to [0, lim), each covered by the
// T-aligned tiles that meet it (its first and last tile may be partial); the
// runs' tiles in order form one list that is cut into the chunks.
constexpr int kPreRuns = 4;  // runs a workgroup keeps in registers

// One staged tile (wave-uniform): it starts at t0 (a multiple of T) and vm
// has bit p set when position t0 + p is visible (inside the run, not in a
// hole).
struct TileD {
  int32_t t0;
  uint64_t vm;
};

template <int HD, int BS, int G, bool KQ8>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(AttnArgs a, const int32_t* __restrict__ table, const int32_t* __restrict__ window,
                    const unsigned char* __restrict__ kpool, const unsigned char* __restrict__ vpool,
                    const int32_t* __restrict__ order, int32_t n_tasks, int32_t nqb) {
  using Gm = PGeom<HD>;
  constexpr int T = Gm::T;
  constexpr int RT = Gm::RT;
  constexpr int PPW = Gm::PPW;
  constexpr int KS = Gm::KS;                      // MFMA k-steps over head_dim
  constexpr int DT = HD / 16;                     // 16-wide head_dim tiles of the output
  constexpr int QPB = rows_per_wg(HD) / G;        // queries per workgroup
  constexpr int NKH = T / 32;                     // 32-position halves (PV k-steps)
  constexpr int NID = T / BS;                     // blocks per tile (tiles are T-aligned)
  constexpr int NDMA = KQ8 ? Gm::NV + Gm::NRW : 2 * Gm::NV;  // copies per wave per tile
  static_assert(BS == 16 || BS == 32, "a tile is whole blocks and a wave's positions one block");
  __shared__ PrefillSmem<HD, KQ8> sm;

  // ---- task u = ((rank * nch + c) * Hkv + kvh) * nqb + qb: the sequences in
  // order of decreasing window size (longest first), so that the longest
  // chunks start first and the short ones fill in behind them
  const int32_t u = (int32_t)blockIdx.x;
  if (u >= n_tasks) return;
  const int qb = u % nqb;
  int32_t rest = u / nqb;
  const int kvh = rest % a.n_kv_heads;
  rest /= a.n_kv_heads;
  const int c = rest % a.nch;
  const int32_t rank = rest / a.nch;
  int s = order[rank];
  s = s < 0 ? 0 : (s >= a.n_seqs ? a.n_seqs - 1 : s);

  const int t = threadIdx.x, w = uni(t >> 6), l = t & 63, g = l >> 4, n16 = l & 15;
  int q0 = a.cu_q[s], q1 = a.cu_q[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > a.n_q_total ? a.n_q_total : q0);
  q1 = q1 < q0 ? q0 : (q1 > a.n_q_total ? a.n_q_total : q1);
  if (q1 > q0 + a.max_q) q1 = q0 + a.max_q;  // queries past max_q_per_seq are not computed
  const int j0 = q0 + qb * QPB;
  if (j0 >= q1) return;  // whole workgroup: no queries here
  const int j1 = j0 + QPB < q1 ? j0 + QPB : q1;
  const int32_t L = clamp_seq_len(a.seq_lens[s], a.max_blocks, BS);
  // the window's first runs, loaded beside cu_q and seq_lens (wave-uniform)
  int64_t px0[kPreRuns], px1[kPreRuns];
#pragma unroll
  for (int r = 0; r < kPreRuns; ++r) {
    px0[r] = 0;
    px1[r] = 0;
    if (r < a.n_runs) raw_run(a, window, s, r, px0[r], px1[r]);
  }
  // run r clipped to [0, limit), and the number of tiles that cover it
  auto run_tiles = [&](int r, int32_t limit, int32_t& lo, int32_t& hi) {
    int64_t x0 = px0[0], x1 = px1[0];
#pragma unroll
    for (int i = 1; i < kPreRuns; ++i)
      if (r == i) {
        x0 = px0[i];
        x1 = px1[i];
      }
    if (r >= kPreRuns) raw_run(a, window, s, r, x0, x1);
    if (x0 < 0) x0 = 0;
    if (x1 > limit) x1 = limit;
    if (x1 < x0) x1 = x0;
    lo = uni((int32_t)x0);
    hi = uni((int32_t)x1);
    return hi > lo ? (hi + T - 1) / T - lo / T : 0;
  };
  // tile idx of the list clipped to [0, limit): its start and its run
  auto tile_at_list = [&](int32_t idx, int32_t limit, int32_t& t0, int32_t& lo, int32_t& hi) {
    lo = 0;
    hi = 0;
    for (int r = 0; r < a.n_runs; ++r) {
      const int32_t n = run_tiles(r, limit, lo, hi);
      if (idx < n) break;
      idx -= n;
    }
    t0 = (lo / T + idx) * T;
  };
  // this chunk of the list clipped to [0, limit): first tile and count
  auto chunk_of = [&](int32_t limit, int32_t& NT, int32_t& ta, int32_t& ntl) {
    NT = 0;
    for (int r = 0; r < a.n_runs; ++r) {
      int32_t lo, hi;
      NT += run_tiles(r, limit, lo, hi);
    }
    const int32_t per = (NT + a.nch - 1) / a.nch;
    ta = c * per;
    ntl = (ta + per < NT ? ta + per : NT) - ta;
    if (ntl > kMaxTiles) ntl = kMaxTiles;  // the host sizes chunks below this
    if (ntl < 0) ntl = 0;
  };
  const int32_t* trow = table + (int64_t)s * a.max_blocks;

  // ---- rows of this lane: row tile rt covers rows (w * RT + rt) * 16 + n16
  int jq[RT], hq[RT];
  bool rok[RT];
  int32_t lim[RT];
  half8_t qf[RT][KS];
  // The table entries of this chunk's tiles, loaded beside the queries'
  // positions: the chunk is cut from the list clipped to the sequence
  // length, and the entries are used if the queries' causal limit leaves
  // that tile where it was (always when the queries end the sequence).
  int32_t NTs, tas, ntls, t0s = -1;
  chunk_of(L, NTs, tas, ntls);
  int32_t spec[4] = {-1, -1, -1, -1};
  if (t < ntls) {
    int32_t lo, hi;
    tile_at_list(tas + t, L, t0s, lo, hi);
#pragma unroll
    for (int j = 0; j < NID; ++j) {
      const int32_t b = t0s / BS + j;
      spec[j] = b < a.max_blocks ? trow[b] : -1;
    }
  }
  int32_t lmin = 0x7fffffff, lmax = 0;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rr = (w * RT + rt) * 16 + n16;
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
    if (rok[rt] && lim[rt] > lmax) lmax = lim[rt];
  }
  // smallest and largest causal limit over the wave's rows (wave-uniform);
  // the largest over the workgroup bounds its tile list
#pragma unroll
  for (int mm = 1; mm < 64; mm <<= 1) {
    const int32_t o = __shfl_xor(lmin, mm, 64);
    lmin = o < lmin ? o : lmin;
    const int32_t x = __shfl_xor(lmax, mm, 64);
    lmax = x > lmax ? x : lmax;
  }
  const int32_t lim_min_w = uni(lmin);
  if (l == 0) sm.lim_max[w] = lmax;
  __syncthreads();
  int32_t lim_max = 0;
#pragma unroll
  for (int i = 0; i < kPWaves; ++i) lim_max = sm.lim_max[i] > lim_max ? sm.lim_max[i] : lim_max;
  lim_max = uni(lim_max);

  // ---- this workgroup's chunk of the window's tile list
  int32_t NT, ta, ntl;
  chunk_of(lim_max, NT, ta, ntl);

  const unsigned char* kbase = kpool + (int64_t)kvh * BS * a.k_seg_bytes;
  const unsigned char* vbase = vpool + (int64_t)kvh * BS * a.v_seg_bytes;
  int32_t bad = 0;  // out-of-range table entries seen (checked mode)

  // thread i describes tile ta + i of the list (ntl <= kMaxTiles < 512)
  static_assert(kMaxTiles <= 64 * kPWaves, "one tile per thread");
  if (t < ntl) {
    int32_t lo, hi;
    TileRec rc;
    tile_at_list(ta + t, lim_max, rc.t0, lo, hi);
    const bool reuse = NT == NTs && ta == tas && rc.t0 == t0s;
    const int32_t vlo = (lo > rc.t0 ? lo : rc.t0) - rc.t0;
    const int32_t vhi = (hi < rc.t0 + T ? hi : rc.t0 + T) - rc.t0;
    uint64_t vm = (vhi >= 64 ? ~0ull : (1ull << vhi) - 1ull) & ~((1ull << vlo) - 1ull);
    rc.pad = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int32_t id = -1;
      if (j < NID) {
        const int32_t b = rc.t0 / BS + j;
        const int32_t raw = reuse ? spec[j] : (b < a.max_blocks ? trow[b] : -1);
        const bool ok = raw >= 0 && raw < a.n_pool_blocks;
        const uint64_t bm = ((1ull << BS) - 1ull) << (j * BS);
        if (!ok && raw != -1 && (vm & bm)) ++bad;
        if (!ok) vm &= ~bm;
        id = ok ? raw : -1;
      }
      rc.blk[j] = id;
    }
    rc.vm_lo = (uint32_t)vm;
    rc.vm_hi = (uint32_t)(vm >> 32);
    sm.tiles[t] = rc;
  }
  __syncthreads();

  float m[RT];
  float4_t o[RT][DT + 1];  // o[rt][DT]: the row's sum of probabilities
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = kEmptyMax;
#pragma unroll
    for (int dt = 0; dt <= DT; ++dt) o[rt][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  // |scale| * log2(e), kept above 0 so that a hidden score (-inf) always
  // gives p = 0 (a zero scale then weighs every visible position equally)
  const float mul = fmaxf(fabsf(a.score_mul), 1e-30f);
  const int pw0 = w * PPW;    // first position this wave copies and prepares
  const int wblk = pw0 / BS;  // the tile block holding this wave's positions

  // per-lane byte offsets inside a (block, kv head) region: tile-invariant
  uint32_t voff[Gm::NV], qoff[KQ8 ? Gm::NRW : 1];
#pragma unroll
  for (int i = 0; i < Gm::NV; ++i) {
    const int uu = i * 64 + l;
    const int r = pw0 + uu / Gm::CHR, pc = uu % Gm::CHR;
    voff[i] = (uint32_t)((r & (BS - 1)) * a.v_seg_bytes + ((pc ^ swz_key<HD>(r)) << 4));
  }
  if constexpr (KQ8) {
#pragma unroll
    for (int i = 0; i < Gm::NRW; ++i) qoff[i] = (uint32_t)((pw0 & (BS - 1)) * Gm::SEG8 + (i * 64 + l) * 16);
  }

  // tile k of the list as the compute needs it (wave-uniform)
  auto tile_at = [&](int k) {
    const TileRec& rc = sm.tiles[k];
    TileD d;
    d.t0 = uni(rc.t0);
    d.vm = ((uint64_t)(uint32_t)uni((int32_t)rc.vm_hi) << 32) | (uint32_t)uni((int32_t)rc.vm_lo);
    return d;
  };

  // copy this wave's positions of tile k into LDS slot sl (no waiting); a
  // block that is a hole copies block 0, which always exists
  auto issue = [&](int sl, int k) {
    const int32_t id = uni(sm.tiles[k].blk[wblk]);
    const int64_t blk = id >= 0 ? id : 0;
    const unsigned char* vb = vbase + blk * a.v_block_bytes;
    const unsigned char* kb = kbase + blk * a.k_block_bytes;
    const uint32_t lv = (uint32_t)uni((int32_t)lds_addr(&sm.v[sl][pw0 * Gm::ROWB]));
#pragma unroll
    for (int i = 0; i < Gm::NV; ++i) {
      copy16_to_lds(vb, voff[i], lv + i * 1024);
      if constexpr (!KQ8) {
        const uint32_t lk = (uint32_t)uni((int32_t)lds_addr(&sm.k[sl][pw0 * Gm::ROWB]));
        copy16_to_lds(kb, voff[i], lk + i * 1024);
      }
    }
    if constexpr (KQ8) {
      const uint32_t lr = (uint32_t)uni((int32_t)lds_addr(&sm.raw[sl][w * Gm::RAWW]));
#pragma unroll
      for (int i = 0; i < Gm::NRW; ++i) {
        // the last copy may be partial: its idle lanes are switched off so
        // that nothing lands past the wave's rows
        if (i * 64 + l < Gm::CPW) copy16_to_lds(kb, qoff[i], lr + i * 1024);
      }
    }
  };

  // after this wave's copies of a tile landed: turn its q8_0 rows into f16
  // codes in K slot kb and f32 scales, and zero the V rows of its positions
  // that are not visible (their codes and scales become 0 as well)
  auto prepare = [&](int sl, int kb, const TileD& d) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    const uint32_t mine = (uint32_t)(d.vm >> pw0) & ((1u << PPW) - 1u);
    if (mine != (1u << PPW) - 1u) {
      // The zero is made here: a zero vector hoisted out of the loop gets
      // spilled, and the wait for its reload would also wait for every copy
      // in flight (the load counter is in order).
      uint32_t z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
#pragma unroll
      for (int i = 0; i < Gm::NV; ++i) {
        const int uu = i * 64 + l;
        const int r = pw0 + uu / Gm::CHR;
        if (!((d.vm >> r) & 1ull)) *(uint4*)&sm.v[sl][r * Gm::ROWB + (uu % Gm::CHR) * 16] = make_uint4(z, z, z, z);
      }
    }
    if constexpr (KQ8) {
#pragma unroll
      for (int e = 0; e < Gm::NQ8; ++e) {
        const int uq = e * 64 + l;
        if (uq < PPW * Gm::UPR) {
          const int p = uq / Gm::UPR, rem = uq - p * Gm::UPR;
          const int bq = rem >> 1, h = rem & 1;
          const int r = pw0 + p;
          const bool ok = (d.vm >> r) & 1ull;
          // bytes [lb, lb + 18) of the segment: the f16 scale (h == 0) or the
          // last two codes of the first half (h == 1), then 16 codes; lb is
          // even, read as five aligned dwords
          const int lb = 34 * bq + 16 * h;
          const uint32_t* src = (const uint32_t*)&sm.raw[sl][w * Gm::RAWW + p * Gm::SEG8 + (lb & ~3)];
          uint32_t qw[5];
#pragma unroll
          for (int i = 0; i < 5; ++i) qw[i] = src[i];
          const int sh = lb & 3;  // 0 or 2
          // 16-byte writes serve 8 consecutive lanes a cycle over 32 banks;
          // with head_dim 128 those lanes hold one position's 16 chunks, and
          // lanes 4-7 take their two chunks in the other order so that each
          // cycle covers 8 distinct chunks modulo 128 bytes
          const int sw2 = (rem >> 2) & 1;
          uint32_t cw[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            cw[i] = sh ? qw[i + 1] : __builtin_amdgcn_alignbyte(qw[i + 1], qw[i], 2);
            cw[i] = ok ? cw[i] : 0u;
          }
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint32_t lo = cw[i], hi = cw[i + 2];
            cw[i] = sw2 ? hi : lo;
            cw[i + 2] = sw2 ? lo : hi;
          }
          if (h == 0) {
            const uint32_t sw = ok ? (sh ? (qw[0] >> 16) : (qw[0] & 0xFFFFu)) : 0u;
            sm.ksc[kb][bq][r] = (float)__builtin_bit_cast(_Float16, (unsigned short)sw);
          }
          half8_t c8[2];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            half2_t c01, c23;
            codes_to_f16(cw[i], c01, c23);
            c8[i >> 1][4 * (i & 1) + 0] = c01[0];
            c8[i >> 1][4 * (i & 1) + 1] = c01[1];
            c8[i >> 1][4 * (i & 1) + 2] = c23[0];
            c8[i >> 1][4 * (i & 1) + 3] = c23[1];
          }
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) *(half8_t*)&sm.k[kb][swz<HD>(r, 4 * bq + 2 * h + (e2 ^ sw2))] = c8[e2];
        }
      }
    }
  };

  // S^T = K Q^T for the 32-position half kh of a tile: for 16-position tile
  // st the lane holds positions 16 st + 4 g + i of the half, for row n16, as
  // sc[rt][4 st + i].  q8_0: the k-step ks is q8_0 block ks of each position;
  // its MFMA partial (codes times q, products exact in f32) is scaled by the
  // four positions' block scales (ksl: [ks][position] of this tile).
  auto scores = [&](const unsigned char* kt, const float* ksl, int kh, float (&sc)[RT][8]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int krow = 32 * kh + 16 * st + n16;
      float4_t acc[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int off = swz<HD>(krow, 4 * ks + g);
        const half8_t af = *(const half8_t*)&kt[off];
        if constexpr (KQ8) {
          const float4_t s4 = *(const float4_t*)&ksl[ks * T + 32 * kh + 16 * st + 4 * g];
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            const float4_t pk = mfma16x16x32(af, qf[rt][ks], float4_t{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[rt][i] = fmaf(pk[i], s4[i], acc[rt][i]);
          }
        } else {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[rt] = mfma16x16x32(af, qf[rt][ks], acc[rt]);
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[rt][4 * st + i] = acc[rt][i];
    }
  };

  // One tile, in 32-position halves: the online softmax is exact in any
  // order, so each half updates the running max/sum and the output in turn.
  // The scores of the next half (matrix cores) are issued after the running
  // max of the current half and interleaved with its exponentials (vector
  // ALU), so the two overlap.
  auto compute = [&](int sl, int kb, const TileD& d) {
    const unsigned char* kt = KQ8 ? sm.k[kb] : sm.k[sl];
    const float* ksl = &sm.ksc[KQ8 ? kb : 0][0][0];
    const unsigned char* vt = sm.v[sl];
    const half8_t ones = {(_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f,
                          (_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f};
    float sc[RT][8], sn[RT][8];
    scores(kt, ksl, 0, sn);
#pragma unroll
    for (int kh = 0; kh < NKH; ++kh) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) sc[rt][jj] = sn[rt][jj];
      const uint32_t vmh = (uint32_t)(d.vm >> (32 * kh));
      const int32_t t0h = d.t0 + 32 * kh;
      const bool full = vmh == 0xffffffffu && t0h + 32 <= lim_min_w;

      // ---- online softmax per row (the four lane groups hold the same row).
      // The running max moves lazily: only when a row's max would grow by
      // more than 2^8, so p stays <= 256 (exact enough in f16) and the output
      // is rarely rescaled.  Hidden positions score -inf and so get p = 0.
      half8_t pf[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        if (!full) {
          // score jj is position p = 16 (jj / 4) + 4 g + jj % 4 of the half
          const uint32_t vg = vmh >> (4 * g);
          const int32_t lr = lim[rt] - t0h - 4 * g;
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int pc = 16 * (jj >> 2) + (jj & 3);
            const bool ok = ((vg >> pc) & 1u) && pc < lr;
            sc[rt][jj] = ok ? sc[rt][jj] : -INFINITY;
          }
        }
        float mx = sc[rt][0];
#pragma unroll
        for (int jj = 1; jj < 8; ++jj) mx = fmaxf(mx, sc[rt][jj]);
        // A row grows iff one of its lanes holds a score above the threshold
        // (scaling by mul > 0 keeps the order), so the row max across the
        // lane groups is only formed when some row of the wave grows.
        if (__builtin_amdgcn_ballot_w64(mx * mul > m[rt] + kLazyMax)) {
          const float mc = max_over_groups(mx) * mul;
          const bool grow = mc > m[rt] + kLazyMax;
          const float mn = grow ? mc : m[rt];
          const float alpha = fast_exp2(m[rt] - mn);
#pragma unroll
          for (int dt = 0; dt <= DT; ++dt) o[rt][dt] *= alpha;
          m[rt] = mn;
        }
      }
      // the next half's scores (matrix cores) next to this half's
      // exponentials (vector ALU): one basic block, so they interleave
      if (kh + 1 < NKH) scores(kt, ksl, kh + 1, sn);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pf[rt][jj] = (_Float16)fast_exp2(fmaf(sc[rt][jj], mul, -m[rt]));

      // ---- O^T += V^T P^T: two transposing reads give lane (g, n16) column
      // dt*16 + n16 of V at positions 16 h + 4 g + e of the half (operand
      // element 4 h + e); lane n16 addresses row 16 h + 4 g + n16 / 4 of the
      // half at columns dt*16 + 4 (n16 % 4) ...  The wave raises its priority
      // for these matrix instructions, so the two waves of a SIMD drift apart
      // and one's vector work overlaps the other's matrix work.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        half8_t vf;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int R = 32 * kh + 16 * h + 4 * g + (n16 >> 2);
          const int cb = 32 * dt + 8 * (n16 & 3);  // byte offset of the 4 columns in the row
          const int off = swz<HD>(R, cb >> 4) + (cb & 15);
          const short4_t x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4_t*)&vt[off]);
          const half2_t* hx = (const half2_t*)&x;
          vf[4 * h + 0] = hx[0][0];
          vf[4 * h + 1] = hx[0][1];
          vf[4 * h + 2] = hx[1][0];
          vf[4 * h + 3] = hx[1][1];
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) o[rt][dt] = mfma16x16x32(vf, pf[rt], o[rt][dt]);
      }
      // row sums of the rounded probabilities (every element of o[rt][DT])
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) o[rt][DT] = mfma16x16x32(ones, pf[rt], o[rt][DT]);
      __builtin_amdgcn_s_setprio(0);
      // Issue order of this block (a scheduling hint; no effect on values):
      // the K fragment reads run four ahead of the matrix instructions that
      // use them, three vector instructions (the exponentials) sit between
      // each pair of score MFMAs, and the V reads of the PV step again run
      // four ahead.  Masks: 0x100 LDS read, 0x008 MFMA, 0x002 vector ALU.
      if (kh + 1 < NKH) {
        constexpr int kSM = 2 * KS * RT;             // score MFMAs of a half
        constexpr int kSR = 2 * KS * (KQ8 ? 2 : 1);  // their K fragment (and q8_0 scale) reads
        constexpr int kPM = (DT + 1) * RT;                // PV and row-sum MFMAs
        constexpr int kPR = 2 * DT;                       // V reads
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < kSM / 2; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          if (i < kSR - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < kPM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < kPR - 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }
  };

  // ---- pipeline: tile k is computed while tile k+1 is being prepared and
  // tiles k+2 .. k+kRing-1 are being copied; tile t lives in slot t % kRing;
  // one barrier per tile
  constexpr int AH = kRing - 1;  // tiles whose copies run ahead of the computed one
  // wait until at most n tiles' copies of this wave are still in flight
  auto wait_tiles = [&](int n) {
    if (n >= 2) wait_vm<2 * NDMA>();
    else if (n == 1) wait_vm<NDMA>();
    else wait_vm<0>();
  };
  static_assert(AH <= 3, "wait_tiles covers at most two tiles in flight");
  if (ntl > 0) {
    // The compiler does not count the copies (inline assembly) among the
    // loads in flight: this wait tells it that the loads above (q, table
    // entries) are done, so it places no wait for their registers after the
    // copies, where in hardware that wait would also cover the copies.
    wait_vm<0>();
    for (int i = 0; i < AH && i < ntl; ++i) issue(i, i);
    wait_tiles((ntl < AH ? ntl : AH) - 1);
    prepare(0, 0, tile_at(0));
    __syncthreads();
    for (int k = 0;; ++k) {
      if (k + AH < ntl) issue((k + AH) % kRing, k + AH);
      compute(k % kRing, k & 1, tile_at(k));
      // prepare tile k+1 once this wave's copies of it have landed
      if (k + 1 < ntl) {
        const int later = ntl - (k + 2);  // tiles issued after k+1 that may still be in flight
        wait_tiles(later < AH - 1 ? later : AH - 1);
        prepare((k + 1) % kRing, (k + 1) & 1, tile_at(k + 1));
      }
      __syncthreads();
      if (k + 1 >= ntl) break;
    }
  }
  if (bad && (a.flags & PKV_FLAG_CHECKED) && a.err && kvh == 0 && qb == 0 && t == 0) atomicAdd(a.err, bad);

  // ---- finish: sum the row's lane groups; write the output or the partial
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float ls = o[rt][DT][0];
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

// Orders the sequences by decreasing number of window tiles (about the
// prefill kernel's work per sequence), ties by index; one workgroup, bitonic
// sort in LDS.  More than kOrderMax sequences keep their own order.
constexpr int kOrderMax = 4096;

template <int T, int BS>
__global__ __launch_bounds__(1024) void prefill_order_kernel(AttnArgs a, int32_t* order) {
  __shared__ uint64_t key[kOrderMax];
  const int n = a.n_seqs, t = threadIdx.x;
  if (n > kOrderMax) {
    for (int i = t; i < n; i += 1024) order[i] = i;
    return;
  }
  int np = 1;
  while (np < n) np <<= 1;
  for (int i = t; i < np; i += 1024) {
    uint64_t kk = ~0ull;  // padding sorts last
    if (i < n) {
      // the window clipped to the sequence length (the order only needs to
      // be roughly right, so the queries' causal limits are not consulted)
      const int32_t L = clamp_seq_len(a.seq_lens[i], a.max_blocks, BS);
      int32_t nt = 0;
      for (int r = 0; r < a.n_runs; ++r) {
        int32_t lo, hi;
        run_range(a, i, r, L, lo, hi);
        nt += hi > lo ? (hi + T - 1) / T - lo / T : 0;
      }
      kk = ((uint64_t)(uint32_t)(0x7fffffff - nt) << 32) | (uint32_t)i;
    }
    key[i] = kk;
  }
  __syncthreads();
  for (int size = 2; size <= np; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = t; i < np; i += 1024) {
        const int j = i ^ stride;
        if (j > i) {
          const bool up = (i & size) == 0;
          const uint64_t x = key[i], y = key[j];
          if ((x > y) == up) {
            key[i] = y;
            key[j] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  for (int i = t; i < n; i += 1024) order[i] = (int32_t)(uint32_t)key[i];
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

// Chunks per window: about one and a half workgroups per CU (one fits a CU at a time;
// the longest chunks go first and the short ones fill in behind them), each
// chunk still at least four tiles of the largest possible window, and never
// more than kMaxTiles tiles (a run of the table's width spans at most
// width / T + 2 tiles).
int plan_chunks(const AttnArgs& a, int hd, int g) {
  const int T = tile_of(hd);
  const int qpb = rows_per_wg(hd) / g;
  const int64_t nqb = ((int64_t)a.max_q + qpb - 1) / qpb;
  const int64_t base = (int64_t)a.n_seqs * a.n_kv_heads * (nqb > 0 ? nqb : 1);
  int64_t nch = (kTargetTasks + base - 1) / base;
  if (nch > kMaxChunks) nch = kMaxChunks;
  const int64_t runs = a.mode == PKV_WIN_KV_MAP ? a.n_runs : 1;
  const int64_t width = (int64_t)a.max_blocks * a.block_size;
  const int64_t cap = runs * width / (4 * T);
  if (nch > cap) nch = cap;
  const int64_t tiles_bound = runs * (width / T + 2);
  const int64_t need = (tiles_bound + kMaxTiles - 1) / kMaxTiles;
  if (nch < need) nch = need;
  return nch < 1 ? 1 : (int)nch;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t prefill_workspace(const AttnArgs& a, int combo, int hd, int bs, int g, bool* found) {
  (void)bs;
  *found = combo == kComboF16 || combo == kComboQ8H;
  if (!*found) return 0;
  const int nch = plan_chunks(a, hd, g);
  // sequence order, then (max, sum) and output partials when nch > 1
  size_t need = align256((size_t)a.n_seqs * sizeof(int32_t));
  if (nch > 1) {
    const size_t rows = (size_t)a.n_q_total * a.n_q_heads * nch;
    need += align256(rows * 2 * sizeof(float)) + align256(rows * hd * sizeof(float));
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
  unsigned char* base = (unsigned char*)a0.part_o;
  int32_t* order = (int32_t*)base;
  base += align256((size_t)a.n_seqs * sizeof(int32_t));
  if (a.nch > 1) {
    const size_t rows = (size_t)a.n_q_total * a.n_q_heads * a.nch;
    a.part_ml = (float*)base;
    a.part_o = (float*)(base + align256(rows * 2 * sizeof(float)));
  }
  const int qpb = rows_per_wg(hd) / g;
  const int32_t nqb = (a.max_q + qpb - 1) / qpb;
  const int64_t n_tasks = (int64_t)a.n_seqs * a.n_kv_heads * a.nch * nqb;
  if (n_tasks > (int64_t)1 << 28) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)n_tasks);
  if (bs == 16) {
    if (hd <= 128) hipLaunchKernelGGL((prefill_order_kernel<tile_of(128), 16>), dim3(1), dim3(1024), 0, st, a, order);
    else hipLaunchKernelGGL((prefill_order_kernel<tile_of(256), 16>), dim3(1), dim3(1024), 0, st, a, order);
  } else {
    hipLaunchKernelGGL((prefill_order_kernel<tile_of(128), 32>), dim3(1), dim3(1024), 0, st, a, order);
  }
  {
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
#define PKV_PCASE(HD, BS, G)                                                                      \
  if (hd == HD && bs == BS && g == G) {                                                           \
    if (q8)                                                                                       \
      hipLaunchKernelGGL((prefill_kernel<HD, BS, G, true>), grid, dim3(512), 0, st, a, a.table,   \
                         a.window, a.k_pool, a.v_pool, order, (int32_t)n_tasks, nqb);             \
    else                                                                                          \
      hipLaunchKernelGGL((prefill_kernel<HD, BS, G, false>), grid, dim3(512), 0, st, a, a.table,  \
                         a.window, a.k_pool, a.v_pool, order, (int32_t)n_tasks, nqb);             \
    *found = true;                                                                                \
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
