// int4 cold-block codec.
//
// "Tiered KV cache — architecture", section "The three-tier model": a cold
// block is kept as one f32 scale followed by ceil(n / 2) bytes of packed
// int4 nibbles, one scale per block.  The quantizer here works in binary32
// exactly as written: scale = amax / 7 (IEEE division), code = x / scale
// (IEEE division) rounded to nearest-even (v_rndne) and clamped to +-7,
// 4-bit two's complement, value 2j in the low nibble of byte j; amax = 0
// gives scale 0 and zero codes.  Decoding is scale * code in binary32,
// converted to the pool format with round-to-nearest-even.
//
// A block is one pool block taken flat in memory order (n_kv_heads x
// block_size x head_dim values in this library's layout, contiguous).  One
// workgroup of 512 threads codes one block: element groups of 8 are dealt
// out round-robin (group i*512 + t to thread t), so every load instruction
// of a wave reads 1 KiB (f16) of consecutive memory, and each group becomes
// one 4-byte word of nibbles.  Encode keeps the thread's groups in
// registers between the block-wide amax and the coding, so the pool is read
// once.
#include "pkv_internal.hpp"

namespace pkv {

namespace {

constexpr int kI4Threads = 512;
constexpr int kI4Waves = kI4Threads / kWave;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Group8;
template <>
struct Group8<_Float16> {  // 8 halves = one 16-byte load / store
  u32x4 w;
  __device__ void load(const unsigned char* p) { w = *(const u32x4*)p; }
  __device__ float at(int i) const {
    const uint32_t x = w[i / 2];
    return (i & 1) ? h2f_hi(x) : h2f_lo(x);
  }
  __device__ static void store(unsigned char* p, const float (&v)[8]) {
    u32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t lo = __builtin_bit_cast(unsigned short, (_Float16)v[2 * k]);
      const uint32_t hi = __builtin_bit_cast(unsigned short, (_Float16)v[2 * k + 1]);
      o[k] = lo | (hi << 16);
    }
    *(u32x4*)p = o;
  }
};
template <>
struct Group8<float> {  // 8 floats = two 16-byte loads / stores
  u32x4 a, b;
  __device__ void load(const unsigned char* p) {
    a = ((const u32x4*)p)[0];
    b = ((const u32x4*)p)[1];
  }
  __device__ float at(int i) const {
    return __builtin_bit_cast(float, i < 4 ? a[i] : b[i - 4]);
  }
  __device__ static void store(unsigned char* p, const float (&v)[8]) {
    u32x4 x, y;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[k] = __builtin_bit_cast(uint32_t, v[k]);
      y[k] = __builtin_bit_cast(uint32_t, v[4 + k]);
    }
    ((u32x4*)p)[0] = x;
    ((u32x4*)p)[1] = y;
  }
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

}  // namespace

// Grid: one workgroup per listed block.  NCH = groups of 8 per thread.
template <typename T, int NCH>
__global__ __launch_bounds__(kI4Threads) void int4_encode_kernel(Int4Args a) {
  __shared__ float wmax[kI4Waves];
  const int32_t blk = a.blocks[blockIdx.x];
  unsigned char* blob = a.blobs + (int64_t)blockIdx.x * a.blob_stride;
  const int t = threadIdx.x;
  const int64_t groups = a.block_elems / 8;
  const bool ok = blk >= 0 && blk < a.n_pool_blocks;
  const unsigned char* base = a.pool + (ok ? (int64_t)blk : 0) * a.block_elems * (int64_t)sizeof(T);
  Group8<T> g[NCH];
  float m = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int64_t gi = (int64_t)c * kI4Threads + t;
    if (ok && gi < groups) {
      g[c].load(base + gi * 8 * (int64_t)sizeof(T));
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(g[c].at(i)));
    }
  }
  m = wave_max(m);
  if (t % kWave == 0) wmax[t / kWave] = m;
  __syncthreads();
  float amax = wmax[0];
#pragma unroll
  for (int w = 1; w < kI4Waves; ++w) amax = fmaxf(amax, wmax[w]);
  const float scale = amax / 7.0f;
  if (t == 0) *(float*)blob = ok ? scale : 0.f;
  // code = rint(x / scale) with the binary32 division.  Fast form: with
  // r = RN(1 / scale) and |x / scale| <= 7, t = RN(x * r) is within 2^-20 of
  // x / scale, so rint(t) is the code unless t lies within 2^-18 of a
  // half-integer (then RN(x / scale) could sit on the other side of it, or
  // on it); those elements, and blocks whose scale is extreme, take the
  // division.  t - rint(t) is exact in binary32 and at most 1/2 in size, so
  // "within 2^-18 of a half-integer" is |t - rint(t)| >= 1/2 - 2^-18.
  const bool fast = scale >= 0x1p-100f && scale <= 0x1p+100f;
  const float r = 1.0f / scale;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int64_t gi = (int64_t)c * kI4Threads + t;
    if (gi >= groups) continue;
    uint32_t word = 0;
    if (ok && scale > 0.f) {
      float q[8];
      bool slow = !fast;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = g[c].at(i);
        const float tq = x * r;
        q[i] = rintf(tq);
        slow |= fabsf(tq - q[i]) >= 0.5f - 0x1p-18f;  // within 2^-18 of a half-integer
      }
      if (slow) {  // rare: redo the group with the division
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = rintf(g[c].at(i) / scale);
      }
      // code + 8 (1..15) is the low nibble of the binary32 2^23 + 8 + code;
      // xor 8 turns it into the code's 4-bit two's complement
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t bits = __builtin_bit_cast(uint32_t, fminf(fmaxf(q[i], -7.f), 7.f) + 8388616.0f);
        word |= (bits & 0xFu) << (4 * i);
      }
      word ^= 0x88888888u;
    }
    *(uint32_t*)(blob + 4 + gi * 4) = word;
  }
}

template <typename T>
__global__ __launch_bounds__(kI4Threads) void int4_decode_kernel(Int4Args a) {
  const int32_t blk = a.blocks[blockIdx.x];
  if (blk < 0 || blk >= a.n_pool_blocks) return;
  const unsigned char* blob = a.blobs + (int64_t)blockIdx.x * a.blob_stride;
  unsigned char* base = a.pool + (int64_t)blk * a.block_elems * (int64_t)sizeof(T);
  const float scale = *(const float*)blob;
  const int64_t groups = a.block_elems / 8;
  for (int64_t gi = threadIdx.x; gi < groups; gi += kI4Threads) {
    const uint32_t word = *(const uint32_t*)(blob + 4 + gi * 4);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = ((int)(word << (28 - 4 * i))) >> 28;  // sign-extend nibble i
      v[i] = scale * (float)q;
    }
    Group8<T>::store(base + gi * 8 * (int64_t)sizeof(T), v);
  }
}

hipError_t launch_int4(bool encode, const Int4Args& a, int fmt, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  const dim3 grid((unsigned)a.n), block(kI4Threads);
  if (!encode) {
    if (fmt == PKV_F16) hipLaunchKernelGGL(int4_decode_kernel<_Float16>, grid, block, 0, st, a);
    else hipLaunchKernelGGL(int4_decode_kernel<float>, grid, block, 0, st, a);
    return hipGetLastError();
  }
  const int64_t per_thread = (a.block_elems / 8 + kI4Threads - 1) / kI4Threads;
#define PKV_I4_ENC(N)                                                                     \
  if (per_thread <= N) {                                                                  \
    if (fmt == PKV_F16) hipLaunchKernelGGL((int4_encode_kernel<_Float16, N>), grid, block, 0, st, a); \
    else hipLaunchKernelGGL((int4_encode_kernel<float, N>), grid, block, 0, st, a);       \
    return hipGetLastError();                                                             \
  }
  PKV_I4_ENC(1)
  PKV_I4_ENC(2)
  PKV_I4_ENC(4)
  PKV_I4_ENC(8)
  PKV_I4_ENC(16)
#undef PKV_I4_ENC
  return hipErrorInvalidValue;
}

}  // namespace pkv
