// Internal declarations shared by the host layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Format combinations (q, K, V) the kernels are built for.
enum Combo : int { kComboF32 = 0, kComboF16 = 1, kComboQ8H = 2, kComboQ8F = 3, kNumCombos = 4 };

// Everything an attention kernel reads, flattened into one by-value struct.
struct AttnArgs {
  const void* q;
  const unsigned char* k_pool;
  const unsigned char* v_pool;
  const int32_t* table;     // [n_seqs][max_blocks]
  const int32_t* seq_lens;  // [n_seqs]
  const int32_t* window;    // span [S][2] | kv_map [S][n_runs][2] | null
  const int32_t* cu_q;      // prefill [S+1]
  const int32_t* q_pos;     // prefill [n_q_total]
  float* out;
  float* lse;
  float* part_o;   // decode partials [S][rows_per_seq][Hq][HD]; prefill [Nq][Hq][nch][HD]
  float* part_ml;  // decode partials [S][rows_per_seq][Hq][2] = (max, sum); prefill [Nq][Hq][nch][2]
  int32_t* err;    // checked mode: count of bad block ids
  int32_t n_seqs, n_q_heads, n_kv_heads, n_pool_blocks, max_blocks, block_size;
  int32_t mode, n_runs;  // n_runs = runs per sequence (1 unless kv_map)
  int32_t split, nspl;   // decode: tokens per split, split slots per run
  // Decode work list (written by the plan pass): items [n][4] = (sequence,
  // lo, hi, partial row); hdr[0] = units (items x kv heads); seqinfo [S][4]
  // = the sequence's first place in each group of the list and its number
  // of whole full slots.  A sequence's last fine_per_seq full slots are cut
  // into nsub pieces of fine_tokens positions.  A sequence's partial rows
  // follow its slots in order, a cut slot's pieces right after it, so the
  // row of (slot, piece p) is slot + (cut slots before it) * (nsub - 1) + p.
  const uint4* items;
  uint32_t* hdr;
  uint4* seqinfo;
  int32_t nsub, fine_tokens, fine_per_seq;
  // Planned calls with at most kSelfPlanMaxSeqs sequences skip the plan
  // pass: each wave derives its own item of the same list (self_plan = 1).
  int32_t self_plan;
  int64_t rows_per_seq;
  int32_t n_q_total, max_q;
  int32_t nch;           // prefill: chunks each workgroup's window is split into
  // Pool layout [n_blocks][n_kv_heads][block_size][seg]: seg = bytes of one
  // token of one kv head; a block is n_kv_heads * block_size * seg bytes.
  int64_t k_seg_bytes, v_seg_bytes, k_block_bytes, v_block_bytes;
  float score_mul;  // scale * log2(e): scores are kept in the log2 domain
  uint32_t flags;
};

// ---------------------------------------------------------------------------
// Window geometry, shared by the split kernel, the merge and the resolver so
// that all of them agree on which work items exist.

__host__ __device__ inline int32_t clamp_seq_len(int32_t L, int32_t max_blocks, int32_t bs) {
  int64_t cap = (int64_t)max_blocks * bs;
  if (L < 0) return 0;
  return (int64_t)L > cap ? (int32_t)cap : L;
}

// Run r of sequence s as a half-open range of positions, clipped to
// [0, limit).  Causal is one run [0, limit); a span is one run [lo, hi); a
// kv_map run (cell, len) is [cell, cell + len), unused when len <= 0.
__device__ inline void run_range(const AttnArgs& a, int s, int r, int32_t limit, int32_t& lo,
                                 int32_t& hi) {
  int64_t x0 = 0, x1 = 0;
  if (a.mode == PKV_WIN_CAUSAL) {
    x0 = 0;
    x1 = limit;
  } else if (a.mode == PKV_WIN_SPAN) {
    x0 = a.window[2 * s];
    x1 = a.window[2 * s + 1];
  } else {
    const int32_t* w = a.window + ((int64_t)s * a.n_runs + r) * 2;
    int64_t c = w[0], n = w[1];
    if (n > 0) {
      x0 = c;
      x1 = c + n;
    }
  }
  if (x0 < 0) x0 = 0;
  if (x1 > limit) x1 = limit;
  if (x1 < x0) x1 = x0;
  lo = (int32_t)x0;
  hi = (int32_t)x1;
}

// Positions a decode split slot covers: [lo, hi) of run r intersected with
// the aligned split window [k*split, (k+1)*split).  Empty => no work item.
__device__ inline void split_range(const AttnArgs& a, int s, int slot, int32_t limit, int32_t& lo,
                                   int32_t& hi) {
  int r = slot / a.nspl;
  int k = slot - r * a.nspl;
  int32_t rl, rh;
  run_range(a, s, r, limit, rl, rh);
  int64_t w0 = (int64_t)k * a.split, w1 = w0 + a.split;
  int64_t x0 = rl > w0 ? rl : w0;
  int64_t x1 = rh < w1 ? rh : w1;
  if (x1 < x0) x1 = x0;
  lo = (int32_t)x0;
  hi = (int32_t)x1;
}

constexpr int kSelfPlanMaxSeqs = 256;  // 4 sequences per lane of one wave

// Number of split slots of a run [rl, rh) that it covers completely.
__host__ __device__ inline int32_t full_slots(int32_t rl, int32_t rh, int32_t split) {
  if (rh <= rl) return 0;
  const int32_t k0 = (int32_t)(((int64_t)rl + split - 1) / split), k1 = rh / split;
  return k1 > k0 ? k1 - k0 : 0;
}

// Physical block of logical block b, or -1 for a hole; ids outside
// [0, n_pool_blocks) count as holes (and, in checked mode, are counted by
// the one reader that passes count = true).
__device__ inline int32_t block_id(const AttnArgs& a, int s, int32_t b, bool count = false) {
  int32_t id = a.table[(int64_t)s * a.max_blocks + b];
  if (id < 0 || id >= a.n_pool_blocks) {
    if (count && id != PKV_INVALID_BLOCK_ID && (a.flags & PKV_FLAG_CHECKED) && a.err)
      atomicAdd(a.err, 1);
    return -1;
  }
  return id;
}

// ---------------------------------------------------------------------------
// Cross-lane helpers.  DPP controls (GFX9 encoding): quad_perm selectors,
// row_ror:n = 0x120 + n, row_half_mirror = 0x141.

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                               0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppRor4 = 0x124;
constexpr int kDppRor8 = 0x128;

__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

// Sum over the aligned group of N consecutive lanes; every lane of the group
// ends with the same bits (each step pairs lanes symmetrically).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group width");
  if constexpr (N >= 2) x += dpp<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRor8>(x);
  return x;
}

// Reduce over lanes with equal (lane % N), N = lanes per token.
template <int N>
__device__ __forceinline__ float strided_sum(float x) {
  if constexpr (N == 4) {
    x += dpp<kDppRor4>(x);
    x += dpp<kDppRor8>(x);
  } else if constexpr (N == 8) {
    x += dpp<kDppRor8>(x);
  }
  if constexpr (N <= 16) x += shfl_xor(x, 16);
  x += shfl_xor(x, 32);
  return x;
}

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// Max over the wave of a value that is equal on the N lanes of each token
// group (N = lanes per token).  Within a 16-lane row the token groups are
// combined with DPP rotations; the four rows are then read into scalar
// registers, so the result is wave-uniform and no LDS round trip is needed.
template <int N>
__device__ __forceinline__ float wave_max_tokens(float x) {
  if constexpr (N == 4) {
    x = fmaxf(x, dpp<kDppRor4>(x));
    x = fmaxf(x, dpp<kDppRor8>(x));
  } else if constexpr (N == 8) {
    x = fmaxf(x, dpp<kDppRor8>(x));
  }
  return fmaxf(fmaxf(lane_value(x, 0), lane_value(x, 16)), fmaxf(lane_value(x, 32), lane_value(x, 48)));
}

__device__ __forceinline__ float uniform(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float h2f_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float h2f_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

// ---------------------------------------------------------------------------
// Launchers (defined in the .hip files).

// Decode plan pass (one workgroup): the work list and the unit count.
hipError_t launch_decode_plan(const AttnArgs& a, hipStream_t st);
// Decode split pass: grid max_units (the host's bound on units) x 64 threads.
hipError_t launch_decode_split(const AttnArgs& a, int combo, int hd, int bs, int g,
                               int64_t max_units, hipStream_t st, bool* found);
// Decode merge pass: grid (ceil(n_q_heads * head_dim / 256), n_seqs), 256 threads.
hipError_t launch_decode_merge(const AttnArgs& a, int hd, hipStream_t st);
// Prefill: workspace bytes a call needs (a multiple of 256, the last 256
// bytes hold the checked-mode error word; 0 if none) and whether a kernel
// exists for the tuple; then the launch (a.part_o = the workspace base).
size_t prefill_workspace(const AttnArgs& a, int combo, int hd, int bs, int g, bool* found);
hipError_t launch_prefill(const AttnArgs& a, int combo, int hd, int bs, int g, hipStream_t st,
                          bool* found);
// f32 prefill through the decode kernels (prefill_f32.hip): per query its
// virtual table row, length and window, whether prefill computes it; then
// the computed rows of the decode output copied out.
hipError_t launch_prefill_expand(const AttnArgs& a, int32_t* vtable, int32_t* vlens, int32_t* vwin,
                                 int32_t win_ints, uint8_t* computed, hipStream_t st);
hipError_t launch_prefill_copy_rows(const float* tmp_out, const float* tmp_lse, const uint8_t* computed,
                                    float* out, float* lse, int64_t n_rows, int32_t hq, int32_t hd,
                                    hipStream_t st);
// Resolver export.
hipError_t launch_resolve(const AttnArgs& a, int bs, int n_cand, int32_t* rows_out, hipStream_t st);
// Row copies for copy_cells: a row (token cell) is n_kv_heads segments of
// seg_bytes, one per kv head, block_size * seg_bytes apart.  Rows outside
// [0, n_rows) (and stage slots outside [0, n_stage)) in a device plan are
// skipped.
struct PoolGeom {
  unsigned char* base;
  int64_t seg_bytes, n_kv_heads, block_size, n_rows;
};
// Phase 1: stage[slot] <- pool[row] for pairs (row, slot); phase 2:
// pool[row] <- pool[src] (src >= 0) or stage[-(src + 1)] for pairs (row,
// src).  Grid ceil(n_pairs / 4) x 256 threads (one wave per pair).
hipError_t launch_copy_rows(int phase, const PoolGeom& pool, unsigned char* stage, int32_t n_stage,
                            const int32_t* pairs, int32_t n_pairs, hipStream_t st);
// Disjoint row moves (no destination touches a source): moves [n][3] and
// cum [n + 1] (prefix sums of the lengths) on the device; grid
// ceil(total_rows / 16) x 256 threads.
hipError_t launch_copy_runs(const PoolGeom& pool, const int32_t* moves, const int32_t* cum,
                            int32_t n_moves, int32_t total_rows, hipStream_t st);
hipError_t launch_zero_words(int32_t* p, int n, hipStream_t st);

// int4 cold-block codec: n listed blocks of the pool <-> n blobs.
struct Int4Args {
  unsigned char* pool;   // [n_pool_blocks][block_elems] of f16 or f32 (read by encode)
  unsigned char* blobs;  // [n][blob_stride]: f32 scale, then block_elems / 2 bytes
  const int32_t* blocks; // [n] pool block ids
  int64_t blob_stride, block_elems;
  int32_t n, n_pool_blocks;
};
// Grid n x 512 threads.  block_elems % 8 == 0 and <= 65536.
hipError_t launch_int4(bool encode, const Int4Args& a, int fmt, hipStream_t st);

// Store of new K/V rows through the block table (pool[1] may be null).
struct StoreArgs {
  const unsigned char* src[2];  // [n_tok][n_kv_heads][head_dim] of the source type
  unsigned char* pool[2];       // [n_pool_blocks][n_kv_heads][block_size][seg]
  int32_t fmt[2];               // pool formats
  const int32_t* seq_ids;       // [n_tok] or null: token t belongs to sequence t
  const int32_t* pos;           // [n_tok]
  const int32_t* table;         // [n_seqs][max_blocks]
  int32_t* skipped;             // tokens not stored are added here, or null
  int32_t n_tok, n_seqs, n_kv_heads, block_size, n_pool_blocks, max_blocks;
};
// Grid: ceil(n_tok * n_kv_heads / units per workgroup) x 256 threads.
hipError_t launch_store(const StoreArgs& a, int src_fmt, int hd, hipStream_t st, bool* found);

// Copy-on-write ops: copy block src (if >= 0) to dst in both pools and set
// table[entry] = dst (pool[1] and table may be null).
struct CowArgs {
  unsigned char* pool[2];
  int64_t block_bytes[2];  // bytes of one block of each pool (a multiple of 4)
  const int32_t* ops;      // [n_ops][3] = (src or -1, dst, table entry)
  int32_t* table;          // device block tables, table_entries int32
  int64_t table_entries;
  int32_t n_ops, n_blocks;
};
// Grid (n_ops, 2, ceil(largest block bytes / 8 KiB)) x 256 threads.
hipError_t launch_cow_apply(const CowArgs& a, hipStream_t st);

// HBM -> LDS copies (global_load_lds): each lane's bytes land at lds + lane *
// size.  Issued as inline assembly so that the compiler, which cannot tell
// which LDS reads they may alias, adds no waits of its own; kernels wait for
// them explicitly (wait_vm) before reading the copied bytes.  M0 is named
// as clobbered (the generated code writes it right before these copies).
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// 16 bytes from base + off (base wave-uniform, off per lane) to lds + 16 * lane.
// Callers derive base and lds from readfirstlane results only, so both are
// scalar registers.
__device__ __forceinline__ void copy16_to_lds(const unsigned char* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds)
               : "memory", "m0");
}

// s_waitcnt vmcnt(n) with the other counters left alone (GFX9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace pkv
