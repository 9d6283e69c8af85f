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

// One wave per (row, source) pair; a row is n_kv_heads segments of
// seg_bytes, block-strided in the pool and contiguous in the stage.  The
// lanes take the row's W-sized words in order; each lane splits its first
// word into (segment, word) once and then steps by 64 words with a carry,
// so no division runs per word.
template <typename W>
__global__ __launch_bounds__(256) void copy_rows_kernel(int phase, PoolGeom g, unsigned char* stage,
                                                        int32_t n_stage, const int32_t* pairs, int32_t n_pairs) {
  const int lane = threadIdx.x & 63;
  const int32_t p = (int32_t)blockIdx.x * 4 + (int32_t)(threadIdx.x >> 6);  // wave-uniform
  if (p >= n_pairs) return;
  const int32_t per_seg = (int32_t)(g.seg_bytes / (int64_t)sizeof(W));
  const int32_t per_row = per_seg * g.n_kv_heads;
  const int64_t head_stride = (int64_t)g.block_size * g.seg_bytes;
  const int64_t block_bytes = g.n_kv_heads * head_stride;
  const int64_t row_bytes = (int64_t)g.n_kv_heads * g.seg_bytes;  // a row in the stage
  auto pool_row = [&](int32_t row) {  // first byte of the row's segment 0 in the pool
    const int32_t blk = row / g.block_size, slot = row - blk * g.block_size;
    return g.base + (int64_t)blk * block_bytes + (int64_t)slot * g.seg_bytes;
  };
  const int32_t x = pairs[2 * p], y = pairs[2 * p + 1];
  // the plan is device data: a pair naming a row outside the pool or a slot
  // outside the stage is skipped
  if (x < 0 || x >= g.n_rows) return;
  if (phase == 1 ? (y < 0 || y >= n_stage) : (y >= g.n_rows || (y < 0 && -(int64_t)y - 1 >= n_stage))) return;
  int32_t h = lane / per_seg, c = lane - h * per_seg;
  const int32_t dh = 64 / per_seg, dc = 64 - dh * per_seg;
  if (phase == 1) {
    // x = pool row, y = stage index
    const unsigned char* src = pool_row(x);
    W* dst = (W*)(stage + (int64_t)y * row_bytes);
    for (int32_t w = lane; w < per_row; w += 64) {
      dst[w] = ((const W*)(src + h * head_stride))[c];
      c += dc;
      h += dh;
      if (c >= per_seg) {
        c -= per_seg;
        ++h;
      }
    }
  } else {
    // x = pool row; y >= 0 pool row, y < 0 stage index -(y + 1)
    unsigned char* dst = pool_row(x);
    if (y >= 0) {
      const unsigned char* src = pool_row(y);
      for (int32_t w = lane; w < per_row; w += 64) {
        ((W*)(dst + h * head_stride))[c] = ((const W*)(src + h * head_stride))[c];
        c += dc;
        h += dh;
        if (c >= per_seg) {
          c -= per_seg;
          ++h;
        }
      }
    } else {
      const W* src = (const W*)(stage + (int64_t)(-(y + 1)) * row_bytes);
      for (int32_t w = lane; w < per_row; w += 64) {
        ((W*)(dst + h * head_stride))[c] = src[w];
        c += dc;
        h += dh;
        if (c >= per_seg) {
          c -= per_seg;
          ++h;
        }
      }
    }
  }
}

// Disjoint runs: when no move's destination touches any move's source and
// destinations do not overlap, every order gives the same bytes, so all rows
// copy at once straight from the moves.  Workgroup b takes global rows
// [16b, 16b + 16) of the concatenated moves (cum = prefix sums of the move
// lengths) and copies each row's n_kv_heads segments.
template <typename W>
__global__ __launch_bounds__(256) void copy_runs_kernel(PoolGeom g, const int32_t* moves,
                                                        const int32_t* cum, int32_t n_moves,
                                                        int32_t total_rows) {
  constexpr int kRows = 16;
  __shared__ int64_t src_off[kRows], dst_off[kRows];  // byte offset of the row's first segment
  const int64_t head_stride = g.block_size * g.seg_bytes;
  const int64_t block_bytes = g.n_kv_heads * head_stride;
  const int32_t r0 = (int32_t)blockIdx.x * kRows;
  if (threadIdx.x < kRows) {
    const int32_t r = r0 + (int32_t)threadIdx.x;
    int64_t so = -1, dof = -1;
    if (r < total_rows) {
      int32_t lo = 0, hi = n_moves - 1;  // last move with cum[m] <= r
      while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (cum[mid] <= r) lo = mid;
        else hi = mid - 1;
      }
      const int64_t o = r - cum[lo];
      const int64_t sr = moves[3 * lo] + o, dr = moves[3 * lo + 1] + o;
      // the plan is device data: rows outside the pool are skipped
      if (sr >= 0 && sr < g.n_rows && dr >= 0 && dr < g.n_rows) {
        so = (sr / g.block_size) * block_bytes + (sr % g.block_size) * g.seg_bytes;
        dof = (dr / g.block_size) * block_bytes + (dr % g.block_size) * g.seg_bytes;
      }
    }
    src_off[threadIdx.x] = so;
    dst_off[threadIdx.x] = dof;
  }
  __syncthreads();
  // wave v copies rows v, v + 4, ...; its lanes walk a row's words by an
  // incremental (segment, word) pair, so no division runs per word
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int32_t per_seg = (int32_t)(g.seg_bytes / (int64_t)sizeof(W));
  const int32_t per_row = per_seg * g.n_kv_heads;
  const int32_t h0 = lane / per_seg, c0 = lane - h0 * per_seg;
  const int32_t dh = 64 / per_seg, dc = 64 - dh * per_seg;
  for (int i = wv; i < kRows; i += 4) {
    const int64_t so = src_off[i], dof = dst_off[i];
    if (so < 0) continue;  // past the last row (wave-uniform)
    int32_t h = h0, c = c0;
    for (int32_t w = lane; w < per_row; w += 64) {
      const int64_t off = h * head_stride + (int64_t)c * (int64_t)sizeof(W);
      *(W*)(g.base + dof + off) = *(const W*)(g.base + so + off);
      c += dc;
      h += dh;
      if (c >= per_seg) {
        c -= per_seg;
        ++h;
      }
    }
  }
}

hipError_t launch_copy_runs(const PoolGeom& pool, const int32_t* moves, const int32_t* cum,
                            int32_t n_moves, int32_t total_rows, hipStream_t st) {
  if (n_moves <= 0 || total_rows <= 0) return hipSuccess;
  const bool wide = (pool.seg_bytes % 16) == 0;
  const unsigned blocks = (unsigned)((total_rows + 15) / 16);
  if (wide)
    hipLaunchKernelGGL(copy_runs_kernel<uint4>, dim3(blocks), dim3(256), 0, st, pool, moves, cum, n_moves,
                       total_rows);
  else
    hipLaunchKernelGGL(copy_runs_kernel<uint32_t>, dim3(blocks), dim3(256), 0, st, pool, moves, cum,
                       n_moves, total_rows);
  return hipGetLastError();
}

hipError_t launch_copy_rows(int phase, const PoolGeom& pool, unsigned char* stage, int32_t n_stage,
                            const int32_t* pairs, int32_t n_pairs, hipStream_t st) {
  if (n_pairs <= 0) return hipSuccess;
  const bool wide = (pool.seg_bytes % 16) == 0;
  const int64_t blocks = ((int64_t)n_pairs + 3) / 4;  // one wave per pair
  if (wide)
    hipLaunchKernelGGL(copy_rows_kernel<uint4>, dim3((unsigned)blocks), dim3(256), 0, st, phase,
                       pool, stage, n_stage, pairs, n_pairs);
  else
    hipLaunchKernelGGL(copy_rows_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, st, phase,
                       pool, stage, n_stage, pairs, n_pairs);
  return hipGetLastError();
}

// Copy-on-write ops: grid (op, pool, chunk); workgroup (i, k, c) copies
// chunk c (kCowChunk bytes) of op i's source block in pool k (a block is
// contiguous in the pool layout), and workgroup (i, 0, 0) also patches the
// device table entry of op i.  Chunks spread one block over several
// workgroups: a batch of a few hundred copies then still fills the chip.
// An op whose source or destination lies outside [0, n_blocks), or whose
// source equals its destination, copies nothing; an entry outside the
// table is not patched.  Sources and destinations of one launch are
// disjoint (the pool hands out fresh destinations), so workgroups never
// race.
constexpr int64_t kCowChunk = 8192;

template <typename W>
__global__ __launch_bounds__(256) void cow_apply_kernel(CowArgs a) {
  constexpr int kUnroll = 2;
  const int32_t src = a.ops[3 * blockIdx.x], dst = a.ops[3 * blockIdx.x + 1];
  const int32_t entry = a.ops[3 * blockIdx.x + 2];
  if (blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0 && a.table && entry >= 0 &&
      entry < a.table_entries)
    a.table[entry] = dst;
  if (src < 0 || dst < 0 || src >= a.n_blocks || dst >= a.n_blocks || src == dst) return;
  unsigned char* base = a.pool[blockIdx.y];
  if (!base) return;
  const int64_t bytes = a.block_bytes[blockIdx.y];
  const int64_t lo = (int64_t)blockIdx.z * kCowChunk;
  if (lo >= bytes) return;
  const int64_t words = (bytes < lo + kCowChunk ? bytes - lo : kCowChunk) / (int64_t)sizeof(W);
  const W* from = (const W*)(base + (int64_t)src * bytes + lo);
  W* to = (W*)(base + (int64_t)dst * bytes + lo);
  for (int64_t w0 = threadIdx.x; w0 < words; w0 += (int64_t)kUnroll * blockDim.x) {
    W v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t w = w0 + (int64_t)u * blockDim.x;
      if (w < words) v[u] = from[w];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t w = w0 + (int64_t)u * blockDim.x;
      if (w < words) to[w] = v[u];
    }
  }
}

hipError_t launch_cow_apply(const CowArgs& a, hipStream_t st) {
  if (a.n_ops <= 0) return hipSuccess;
  const bool wide = (a.block_bytes[0] % 16) == 0 && (!a.pool[1] || (a.block_bytes[1] % 16) == 0);
  const int64_t most = a.block_bytes[0] > a.block_bytes[1] ? a.block_bytes[0] : a.block_bytes[1];
  const int64_t chunks = (most + kCowChunk - 1) / kCowChunk;
  if (chunks > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)a.n_ops, 2, (unsigned)chunks);
  if (wide)
    hipLaunchKernelGGL(cow_apply_kernel<uint4>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(cow_apply_kernel<uint32_t>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace pkv
