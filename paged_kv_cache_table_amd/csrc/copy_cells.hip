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

template <typename W>
__global__ __launch_bounds__(256) void copy_rows_kernel(int phase, unsigned char* pool,
                                                        unsigned char* stage, int64_t row_bytes,
                                                        const int32_t* pairs, int32_t n_pairs) {
  const int64_t per_row = row_bytes / (int64_t)sizeof(W);
  const int64_t total = per_row * n_pairs;
  for (int64_t f = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; f < total;
       f += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = f / per_row, c = f - p * per_row;
    const int32_t x = pairs[2 * p], y = pairs[2 * p + 1];
    if (phase == 1) {
      // x = pool row, y = stage index
      const W* src = (const W*)(pool + (int64_t)x * row_bytes);
      W* dst = (W*)(stage + (int64_t)y * row_bytes);
      dst[c] = src[c];
    } else {
      // x = pool row; y >= 0 pool row, y < 0 stage index -(y + 1)
      const W* src = y >= 0 ? (const W*)(pool + (int64_t)y * row_bytes)
                            : (const W*)(stage + (int64_t)(-(y + 1)) * row_bytes);
      W* dst = (W*)(pool + (int64_t)x * row_bytes);
      dst[c] = src[c];
    }
  }
}

hipError_t launch_copy_rows(int phase, unsigned char* pool, unsigned char* stage,
                            int64_t row_bytes, const int32_t* pairs, int32_t n_pairs,
                            int64_t stage_offset_bytes, int64_t stage_row_stride, hipStream_t st) {
  (void)stage_row_stride;
  if (n_pairs <= 0) return hipSuccess;
  unsigned char* stg = stage ? stage + stage_offset_bytes : nullptr;
  const bool wide = (row_bytes % 16) == 0;
  const int64_t units = (row_bytes / (wide ? 16 : 4)) * (int64_t)n_pairs;
  int64_t blocks = (units + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (wide)
    hipLaunchKernelGGL(copy_rows_kernel<uint4>, dim3((unsigned)blocks), dim3(256), 0, st, phase,
                       pool, stg, row_bytes, pairs, n_pairs);
  else
    hipLaunchKernelGGL(copy_rows_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, st, phase,
                       pool, stg, row_bytes, pairs, n_pairs);
  return hipGetLastError();
}

}  // namespace pkv
