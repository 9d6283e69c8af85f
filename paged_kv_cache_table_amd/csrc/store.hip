// Store: write the K and V rows of new tokens into the paged pools through
// the block table, converting to each pool's format on the way.
//
// "KV Cache Design — cells, format, sessions", section 3: the store has a
// single quantizer — per 32-value block the scale is amax/127, kept as an
// f16, and the codes round to nearest with ties to even; a Q8_0 block is
// that scale followed by its 32 int8 codes, a cell whole blocks rounded up to
// whole 4-byte words.  "Tiered KV cache — architecture", section "The
// paged-attention block model": position t of a sequence lives in physical
// block table[t / block_size] at slot t % block_size.
//
// The quantizer works in binary32 exactly as written: d = amax / 127 and
// x / d are IEEE divisions (correctly rounded), the code is x / d rounded to
// nearest-even (v_rndne) and clamped to +-127, the stored scale is d
// converted to binary16 with round-to-nearest-even.  A block with amax = 0
// stores scale 0 and zero codes.
//
// Work split: a unit is one (token, kv head) segment of head_dim values;
// HD/8 lanes share a unit, 8 consecutive values per lane, so a wave reads
// 64 * 8 consecutive source values.  Each thread carries kSteps units of K
// and of V through the loads before it converts any, to keep enough bytes in
// flight (two steps measured best: more steps cost occupancy).  Sources are
// read once, with non-temporal loads that keep them from displacing the
// pool lines being written (plain stores measured faster than non-temporal
// ones).  f16/f32 pools take one 16-byte store per lane and pool; a q8_0
// segment (34-byte blocks, only 2-byte aligned inside) is assembled in LDS
// and written out as whole 4-byte words.
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kStoreThreads = 256;
constexpr int kStoreWaves = kStoreThreads / kWave;
constexpr int kSteps = 2;

template <int HD>
struct StoreGeom {
  static constexpr int G = HD / 8;                       // lanes per unit
  static constexpr int UW = kWave / G;                   // units per wave and step
  static constexpr int UPB = kStoreWaves * UW * kSteps;  // units per workgroup
  static constexpr int NB = HD / 32;                     // q8_0 blocks per segment
  static constexpr int QSEG = (NB * 34 + 3) / 4 * 4;     // q8_0 segment bytes
  static constexpr int QWORDS = QSEG / 4;
  static constexpr int WAVE_UNITS = UW * kSteps;         // units a wave stages
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Eight source values of one lane as floats (16-byte non-temporal loads).
template <typename S>
struct Src8;
template <>
struct Src8<_Float16> {
  u32x4 w;
  __device__ void load(const unsigned char* p) { w = __builtin_nontemporal_load((const u32x4*)p); }
  __device__ void zero() { w = u32x4{0, 0, 0, 0}; }
  __device__ float at(int i) const {
    const uint32_t x = w[i / 2];
    return (i & 1) ? h2f_hi(x) : h2f_lo(x);
  }
};
template <>
struct Src8<float> {
  f32x4 a, b;
  __device__ void load(const unsigned char* p) {
    a = __builtin_nontemporal_load((const f32x4*)p);
    b = __builtin_nontemporal_load((const f32x4*)p + 1);
  }
  __device__ void zero() { a = b = f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ float at(int i) const { return i < 4 ? a[i] : b[i - 4]; }
};

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  const uint32_t l = __builtin_bit_cast(unsigned short, (_Float16)lo);
  const uint32_t h = __builtin_bit_cast(unsigned short, (_Float16)hi);
  return l | (h << 16);
}

// Max over the 4 lanes of an aligned quad (one q8_0 block = 4 lanes x 8).
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  return x;
}

}  // namespace

template <typename S, int HD>
__global__ __launch_bounds__(kStoreThreads) void store_kernel(StoreArgs a) {
  using Geo = StoreGeom<HD>;
  constexpr int G = Geo::G, UW = Geo::UW, QSEG = Geo::QSEG;
  __shared__ __align__(16) unsigned char stage[2][kStoreWaves][Geo::WAVE_UNITS * QSEG];
  __shared__ int64_t seg_of[kStoreWaves][Geo::WAVE_UNITS];

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int ug = lane / G, li = lane % G;
  // The host keeps n_tok * n_kv_heads and every pool segment index below
  // 2^31, so unit arithmetic is 32-bit.
  const uint32_t n_units = (uint32_t)a.n_tok * (uint32_t)a.n_kv_heads;
  const uint32_t unit0 = blockIdx.x * (uint32_t)Geo::UPB;

  Src8<S> xs[2][kSteps];
  int64_t seg[kSteps];
#pragma unroll
  for (int r = 0; r < kSteps; ++r) {
    const uint32_t u = unit0 + (uint32_t)((r * kStoreWaves + wave) * UW + ug);
    seg[r] = -1;
    xs[0][r].zero();
    xs[1][r].zero();
    if (u >= n_units) continue;
    const int64_t src_off = ((int64_t)u * HD + li * 8) * (int64_t)sizeof(S);
    xs[0][r].load(a.src[0] + src_off);
    if (a.pool[1]) xs[1][r].load(a.src[1] + src_off);
    const int32_t t = (int32_t)(u / (uint32_t)a.n_kv_heads);
    const int32_t h = (int32_t)(u - (uint32_t)t * (uint32_t)a.n_kv_heads);
    const int32_t s = a.seq_ids ? a.seq_ids[t] : t;
    const int32_t p = a.pos[t];
    int32_t blk = -1;
    if (s >= 0 && s < a.n_seqs && p >= 0 && p / a.block_size < a.max_blocks) {
      blk = a.table[(int64_t)s * a.max_blocks + p / a.block_size];
      if (blk >= a.n_pool_blocks) blk = -1;
    }
    if (blk >= 0)
      seg[r] = ((int64_t)blk * a.n_kv_heads + h) * a.block_size + (p % a.block_size);
    else if (h == 0 && li == 0 && a.skipped)
      atomicAdd(a.skipped, 1);
  }

#pragma unroll
  for (int pl = 0; pl < 2; ++pl) {
    unsigned char* pool = a.pool[pl];
    if (!pool) continue;
    const int fmt = a.fmt[pl];
    if (fmt == PKV_F16) {
#pragma unroll
      for (int r = 0; r < kSteps; ++r) {
        if (seg[r] < 0) continue;
        const Src8<S>& x = xs[pl][r];
        uint4 o;
        o.x = pack_h2(x.at(0), x.at(1));
        o.y = pack_h2(x.at(2), x.at(3));
        o.z = pack_h2(x.at(4), x.at(5));
        o.w = pack_h2(x.at(6), x.at(7));
        *(uint4*)(pool + seg[r] * (int64_t)(2 * HD) + li * 16) = o;
      }
    } else if (fmt == PKV_F32) {
#pragma unroll
      for (int r = 0; r < kSteps; ++r) {
        if (seg[r] < 0) continue;
        const Src8<S>& x = xs[pl][r];
        float4* d = (float4*)(pool + seg[r] * (int64_t)(4 * HD) + li * 32);
        d[0] = make_float4(x.at(0), x.at(1), x.at(2), x.at(3));
        d[1] = make_float4(x.at(4), x.at(5), x.at(6), x.at(7));
      }
    } else {
      // q8_0: quantize into this wave's stage, then write whole words.
      unsigned char* st = stage[pl][wave];
#pragma unroll
      for (int r = 0; r < kSteps; ++r) {
        const Src8<S>& x = xs[pl][r];
        float m = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x.at(i)));
        const float amax = quad_max(m);
        const float d = amax / 127.0f;
        unsigned short c[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          int q0 = 0, q1 = 0;
          if (d > 0.f) {
            q0 = (int)fminf(fmaxf(rintf(x.at(2 * i) / d), -127.f), 127.f);
            q1 = (int)fminf(fmaxf(rintf(x.at(2 * i + 1) / d), -127.f), 127.f);
          }
          c[i] = (unsigned short)((q0 & 0xFF) | ((q1 & 0xFF) << 8));
        }
        const int j = li / 4, k = li % 4;  // block of the segment, quarter of the block
        unsigned char* base = st + (r * UW + ug) * QSEG + j * 34;
        unsigned short* cw = (unsigned short*)(base + 2 + 8 * k);
#pragma unroll
        for (int i = 0; i < 4; ++i) cw[i] = c[i];
        if (k == 0) *(unsigned short*)base = __builtin_bit_cast(unsigned short, (_Float16)d);
        if (QSEG > Geo::NB * 34 && k == 0 && j == Geo::NB - 1)
          *(unsigned short*)(base + 34) = 0;  // pad to a whole word
        if (li == 0) seg_of[wave][r * UW + ug] = seg[r];
      }
      __syncthreads();
      const uint32_t* sw = (const uint32_t*)st;
      for (int w = lane; w < Geo::WAVE_UNITS * Geo::QWORDS; w += kWave) {
        const int uu = w / Geo::QWORDS, dw = w - uu * Geo::QWORDS;
        const int64_t sg = seg_of[wave][uu];
        if (sg < 0) continue;
        *(uint32_t*)(pool + sg * (int64_t)QSEG + dw * 4) = sw[w];
      }
    }
  }
}

hipError_t launch_store(const StoreArgs& a, int src_fmt, int hd, hipStream_t st, bool* found) {
  *found = true;
  const int64_t units = (int64_t)a.n_tok * a.n_kv_heads;
  if (units <= 0) return hipSuccess;
  auto go = [&](auto kernel, int upb) {
    const int64_t blocks = (units + upb - 1) / upb;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(kStoreThreads), 0, st, a);
    return hipGetLastError();
  };
#define PKV_STORE_CASE(S, HD) \
  if (hd == HD) return go(store_kernel<S, HD>, StoreGeom<HD>::UPB);
  if (src_fmt == PKV_F16) {
    PKV_STORE_CASE(_Float16, 32)
    PKV_STORE_CASE(_Float16, 64)
    PKV_STORE_CASE(_Float16, 128)
    PKV_STORE_CASE(_Float16, 256)
  } else if (src_fmt == PKV_F32) {
    PKV_STORE_CASE(float, 32)
    PKV_STORE_CASE(float, 64)
    PKV_STORE_CASE(float, 128)
    PKV_STORE_CASE(float, 256)
  }
#undef PKV_STORE_CASE
  *found = false;
  return hipSuccess;
}

}  // namespace pkv
