// Row copies for copy_cells ("KV Cache Design — cells, format, sessions",
// section 2: a compaction moves rows verbatim).  The host has already
// reduced the ordered moves to one final source per changed row; these
// kernels only move bytes:
//   phase 1 (gather): stage[i]   <- pool[src]   for sources that are
//                                                 themselves overwritten;
//   phase 2 (scatter): pool[dst] <- pool[src] or stage[i].
// Within a phase no row is both read and written, so every thread may run
// in any order and the result is the sequential result, bit for bit.
#include "pkv_internal.hpp"

namespace pkv {

// One work unit = one W-sized word of one row; a row is n_kv_heads segments.
template <typename W>
__global__ __launch_bounds__(256) void copy_rows_kernel(int phase, PoolGeom g, unsigned char* stage,
                                                        const int32_t* pairs, int32_t n_pairs) {
  const int64_t per_seg = g.seg_bytes / (int64_t)sizeof(W);
  const int64_t per_row = per_seg * g.n_kv_heads;
  const int64_t total = per_row * n_pairs;
  const int64_t head_stride = g.block_size * g.seg_bytes;
  const int64_t block_bytes = g.n_kv_heads * head_stride;
  const int64_t row_bytes = g.n_kv_heads * g.seg_bytes;  // a row in the stage is contiguous
  auto pool_word = [&](int64_t row, int64_t h, int64_t c) {
    const int64_t blk = row / g.block_size, slot = row - blk * g.block_size;
    return (W*)(g.base + blk * block_bytes + h * head_stride + slot * g.seg_bytes) + c;
  };
  for (int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; f < total;
       f += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = f / per_row, w = f - p * per_row;
    const int64_t h = w / per_seg, c = w - h * per_seg;
    const int32_t x = pairs[2 * p], y = pairs[2 * p + 1];
    if (phase == 1) {
      // x = pool row, y = stage index
      W* dst = (W*)(stage + (int64_t)y * row_bytes) + w;
      *dst = *pool_word(x, h, c);
    } else {
      // x = pool row; y >= 0 pool row, y < 0 stage index -(y + 1)
      const W* src = y >= 0 ? pool_word(y, h, c) : (const W*)(stage + (int64_t)(-(y + 1)) * row_bytes) + w;
      *pool_word(x, h, c) = *src;
    }
  }
}

hipError_t launch_copy_rows(int phase, const PoolGeom& pool, unsigned char* stage,
                            const int32_t* pairs, int32_t n_pairs, hipStream_t st) {
  if (n_pairs <= 0) return hipSuccess;
  const bool wide = (pool.seg_bytes % 16) == 0;
  const int64_t units = (pool.seg_bytes / (wide ? 16 : 4)) * pool.n_kv_heads * (int64_t)n_pairs;
  int64_t blocks = (units + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (wide)
    hipLaunchKernelGGL(copy_rows_kernel<uint4>, dim3((unsigned)blocks), dim3(256), 0, st, phase,
                       pool, stage, pairs, n_pairs);
  else
    hipLaunchKernelGGL(copy_rows_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, st, phase,
                       pool, stage, pairs, n_pairs);
  return hipGetLastError();
}

}  // namespace pkv
