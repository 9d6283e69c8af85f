// C ABI of the paged-attention library: argument validation, dispatch over
// (head_dim, block_size, group, formats) and split planning (order_moves and
// the copy_cells plan live in copy_plan.cpp).  Every host-checkable condition is checked before
// the first launch, so a refused call leaves outputs and pools untouched.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pkv_internal.hpp"

namespace {

thread_local std::string g_err;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

pkv_status ok() {
  g_err.clear();
  return PKV_OK;
}

const char* fmt_name(int f) {
  switch (f) {
    case PKV_F32: return "f32";
    case PKV_F16: return "f16";
    case PKV_Q8_0: return "q8_0";
    default: return "?";
  }
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Bytes of one token of one kv head: head_dim values, or for q8_0 head_dim/32
// blocks of (f16 scale, 32 int8) rounded up to whole 4-byte words.
int64_t seg_bytes_of(int fmt, int hd) {
  if (hd <= 0) return 0;
  switch (fmt) {
    case PKV_F32: return 4ll * hd;
    case PKV_F16: return 2ll * hd;
    case PKV_Q8_0: {
      if (hd % 32) return 0;
      const int64_t raw = (int64_t)(hd / 32) * 34;
      return (raw + 3) / 4 * 4;
    }
    default: return 0;
  }
}

int64_t row_bytes_of(int fmt, int hkv, int hd) {
  if (hkv <= 0) return 0;
  return (int64_t)hkv * seg_bytes_of(fmt, hd);
}

bool supported_head_block(int hd, int bs) {
  return (hd == 64 && bs == 16) || (hd == 128 && bs == 16) || (hd == 256 && bs == 16) ||
         (hd == 128 && bs == 32);
}

bool supported_group(int g) { return g == 1 || g == 2 || g == 3 || g == 4 || g == 8; }

// Format combination index, or -1.
int combo_of(int qf, int kf, int vf) {
  if (qf == PKV_F32 && kf == PKV_F32 && vf == PKV_F32) return pkv::kComboF32;
  if (qf == PKV_F16 && kf == PKV_F16 && vf == PKV_F16) return pkv::kComboF16;
  if (qf == PKV_F16 && kf == PKV_Q8_0 && vf == PKV_F16) return pkv::kComboQ8H;
  if (qf == PKV_F32 && kf == PKV_Q8_0 && vf == PKV_F32) return pkv::kComboQ8F;
  return -1;
}

struct Plan {
  int combo = -1, g = 0, runs = 1, split = 0, nspl = 0;
  // decode: whether the call runs the plan pass, pieces per cut slot, their
  // size, cut slots per sequence, partial rows per sequence and the most
  // items a call can have
  bool planned = false;
  int nsub = 1, fine = 0, fine_per_seq = 0;
  int64_t rows_per_seq = 0, max_items = 0;
  size_t off_o = 0, off_ml = 0, off_err = 0, off_items = 0, off_seq = 0, off_hdr = 0, total = 0;
};

// Validation shared by every attention call.
pkv_status check_attn(const pkv_shape* sh, int mode, int n_runs, const void* window, Plan* P) {
  if (!sh) return fail(PKV_E_ARG, "shape is NULL");
  if (sh->n_seqs < 0 || sh->n_seqs > 65535)
    return fail(PKV_E_ARG, "n_seqs %d outside [0, 65535]", sh->n_seqs);
  if (sh->n_q_heads <= 0 || sh->n_kv_heads <= 0 || sh->n_kv_heads > 65535)
    return fail(PKV_E_ARG, "head counts must be positive (n_q_heads %d, n_kv_heads %d)",
                sh->n_q_heads, sh->n_kv_heads);
  if (sh->n_q_heads % sh->n_kv_heads)
    return fail(PKV_E_ARG, "n_q_heads %d is not a multiple of n_kv_heads %d", sh->n_q_heads,
                sh->n_kv_heads);
  if (sh->head_dim <= 0 || sh->block_size <= 0)
    return fail(PKV_E_ARG, "head_dim %d and block_size %d must be positive", sh->head_dim,
                sh->block_size);
  if (sh->n_pool_blocks <= 0 || sh->max_blocks_per_seq <= 0)
    return fail(PKV_E_ARG, "n_pool_blocks %d and max_blocks_per_seq %d must be positive",
                sh->n_pool_blocks, sh->max_blocks_per_seq);
  if ((int64_t)sh->max_blocks_per_seq * sh->block_size > INT32_MAX)
    return fail(PKV_E_ARG, "max_blocks_per_seq * block_size overflows int32");
  for (int f : {sh->q_fmt, sh->k_fmt, sh->v_fmt})
    if (f != PKV_F32 && f != PKV_F16 && f != PKV_Q8_0)
      return fail(PKV_E_ARG, "unknown KV format value %d", f);
  if (!std::isfinite(sh->scale)) return fail(PKV_E_ARG, "scale is not finite");
  if (mode != PKV_WIN_CAUSAL && mode != PKV_WIN_SPAN && mode != PKV_WIN_KV_MAP)
    return fail(PKV_E_ARG, "unknown window mode %d", mode);
  if (mode == PKV_WIN_KV_MAP && (n_runs < 1 || n_runs > PKV_KV_MAP_MAX_SPANS))
    return fail(PKV_E_ARG, "kv_map needs 1..%d runs per sequence, got %d", PKV_KV_MAP_MAX_SPANS,
                n_runs);
  if (mode != PKV_WIN_CAUSAL && !window && sh->n_seqs > 0)
    return fail(PKV_E_ARG, "window mode %d needs a window input", mode);
  const int g = sh->n_q_heads / sh->n_kv_heads;
  if (!supported_head_block(sh->head_dim, sh->block_size))
    return fail(PKV_E_UNSUPPORTED,
                "unsupported (head_dim, block_size) = (%d, %d): supported are (64,16), (128,16), "
                "(256,16), (128,32)",
                sh->head_dim, sh->block_size);
  if (!supported_group(g))
    return fail(PKV_E_UNSUPPORTED, "unsupported GQA group %d (n_q_heads %d / n_kv_heads %d)", g,
                sh->n_q_heads, sh->n_kv_heads);
  const int combo = combo_of(sh->q_fmt, sh->k_fmt, sh->v_fmt);
  if (combo < 0)
    return fail(PKV_E_UNSUPPORTED,
                "unsupported (q, K, V) formats (%s, %s, %s): supported are (f32,f32,f32), "
                "(f16,f16,f16), (f16,q8_0,f16), (f32,q8_0,f32)",
                fmt_name(sh->q_fmt), fmt_name(sh->k_fmt), fmt_name(sh->v_fmt));
  P->combo = combo;
  P->g = g;
  P->runs = mode == PKV_WIN_KV_MAP ? n_runs : 1;
  return PKV_OK;
}

// Decode split size: the largest of 64, 32, 16, 8, 4 blocks that still gives
// enough work items (an upper bound from the table width) to keep every CU
// busy: long splits write fewer partials for the merge, short ones shorten
// the tail.  Depends on the shape only.
int auto_split(const pkv_shape* sh, int runs) {
  const int64_t ctx = (int64_t)sh->max_blocks_per_seq * sh->block_size;
  const int64_t target = 6144;
  for (int nb : {64, 32, 16, 8}) {
    const int64_t sp = (int64_t)nb * sh->block_size;
    const int64_t items = (int64_t)sh->n_seqs * sh->n_kv_heads * runs * ((ctx + sp - 1) / sp);
    if (items >= target) return (int)sp;
  }
  return 4 * sh->block_size;
}

pkv_status plan_decode(const pkv_shape* sh, int mode, int n_runs, const void* window, Plan* P) {
  pkv_status st = check_attn(sh, mode, n_runs, window, P);
  if (st) return st;
  int split = sh->split_tokens;
  if (split == 0) {
    split = auto_split(sh, P->runs);
  } else if (split < 0 || split % sh->block_size || split > 64 * sh->block_size) {
    return fail(PKV_E_ARG, "split_tokens %d must be a positive multiple of block_size %d, at most 64 blocks",
                split, sh->block_size);
  }
  const int64_t ctx = (int64_t)sh->max_blocks_per_seq * sh->block_size;
  const int64_t nspl = (ctx + split - 1) / split;
  if (nspl * P->runs > 65535)
    return fail(PKV_E_UNSUPPORTED,
                "%lld split slots per sequence (max_blocks_per_seq %d x block %d / split %d x %d runs) "
                "exceed 65535; use a larger split_tokens",
                (long long)(nspl * P->runs), sh->max_blocks_per_seq, sh->block_size, split, P->runs);
  P->split = split;
  P->nspl = (int)nspl;
  // Calls that can have more than kPlanMinUnits units run the plan pass:
  // the items without gaps, ending on short units, for which each sequence
  // cuts its last few full slots into pieces of >= 256 positions, about
  // kCutWaves units of pieces over the whole batch (at most kMaxCutPerSeq
  // slots per sequence).  Smaller calls launch one workgroup per possible
  // slot: there the plan pass costs more than it saves (measured on a
  // long-context batch of exactly 8192 possible units, all non-empty).
  constexpr int64_t kPlanMinUnits = 4 * 2048, kCutWaves = 4096, kMaxCutPerSeq = 2;
  const int64_t slots_per_seq = nspl * P->runs;
  P->planned = (int64_t)sh->n_seqs * slots_per_seq * sh->n_kv_heads > kPlanMinUnits;
  P->nsub = split / 256 < 1 ? 1 : (split / 256 > 4 ? 4 : split / 256);
  P->fine = (int)(((split + P->nsub - 1) / P->nsub + sh->block_size - 1) / sh->block_size * sh->block_size);
  while (P->nsub > 1 && (int64_t)(P->nsub - 1) * P->fine >= split) --P->nsub;
  P->fine_per_seq = 0;
  if (P->planned && P->nsub > 1) {
    const int64_t per = (int64_t)P->nsub * sh->n_kv_heads * sh->n_seqs;
    int64_t m = (kCutWaves + per - 1) / per;
    if (m > kMaxCutPerSeq) m = kMaxCutPerSeq;
    P->fine_per_seq = (int)(m < slots_per_seq ? m : slots_per_seq);
  }
  P->rows_per_seq = slots_per_seq + (int64_t)P->fine_per_seq * (P->nsub - 1);
  const int64_t rows = (int64_t)sh->n_seqs * P->rows_per_seq;
  P->max_items = rows;
  if (rows >= ((int64_t)1 << 32) || P->max_items * sh->n_kv_heads >= ((int64_t)1 << 31))
    return fail(PKV_E_UNSUPPORTED,
                "%lld decode work items x %d kv heads exceed the 32-bit counters; use a larger split_tokens",
                (long long)P->max_items, sh->n_kv_heads);
  const size_t slots = (size_t)rows * sh->n_q_heads;
  P->off_o = 0;
  P->off_ml = align_up(slots * sh->head_dim * sizeof(float), 256);
  P->off_items = P->off_ml + align_up(slots * 2 * sizeof(float), 256);
  P->off_seq = P->off_items + align_up((size_t)P->max_items * 16, 256);
  P->off_hdr = P->off_seq + align_up((size_t)sh->n_seqs * 16, 256);
  P->off_err = P->off_hdr + 256;
  P->total = P->off_err + 256;
  return PKV_OK;
}

pkv::AttnArgs base_args(const pkv_shape* sh, const Plan& P) {
  pkv::AttnArgs a{};
  a.n_seqs = sh->n_seqs;
  a.n_q_heads = sh->n_q_heads;
  a.n_kv_heads = sh->n_kv_heads;
  a.n_pool_blocks = sh->n_pool_blocks;
  a.max_blocks = sh->max_blocks_per_seq;
  a.block_size = sh->block_size;
  a.k_seg_bytes = seg_bytes_of(sh->k_fmt, sh->head_dim);
  a.v_seg_bytes = seg_bytes_of(sh->v_fmt, sh->head_dim);
  a.k_block_bytes = a.k_seg_bytes * sh->n_kv_heads * sh->block_size;
  a.v_block_bytes = a.v_seg_bytes * sh->n_kv_heads * sh->block_size;
  a.score_mul = (float)((double)sh->scale * 1.4426950408889634);
  a.flags = sh->flags;
  a.n_runs = P.runs;
  a.split = P.split;
  a.nspl = P.nspl;
  return a;
}

pkv_status device_fail(hipError_t e, const char* what) {
  return fail(PKV_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

pkv_status finish_checked(const pkv::AttnArgs& a, hipStream_t st) {
  if (!(a.flags & PKV_FLAG_CHECKED)) return ok();
  int32_t bad = 0;
  hipError_t e = hipMemcpyAsync(&bad, a.err, sizeof bad, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return device_fail(e, "reading the checked-mode error word");
  if (bad)
    return fail(PKV_E_ARG,
                "%d block-table entries are outside [-1, n_pool_blocks); they were read as holes",
                bad);
  return ok();
}

enum DecodePart { kBoth, kPartials, kMerge };

pkv_status decode_impl(DecodePart part, const pkv_shape* sh, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table, const int32_t* seq_lens,
                       int32_t mode, int32_t n_runs, const int32_t* window, float* out, float* lse,
                       void* ws, size_t ws_bytes, void* stream) {
  Plan P;
  pkv_status st = plan_decode(sh, mode, n_runs, window, &P);
  if (st) return st;
  if (sh->n_seqs == 0) return ok();
  if (!seq_lens) return fail(PKV_E_ARG, "seq_lens is NULL");
  if (part != kMerge && (!q || !k_pool || !v_pool || !block_table))
    return fail(PKV_E_ARG, "q, k_pool, v_pool and block_table must be non-NULL");
  if (part != kPartials && !out) return fail(PKV_E_ARG, "out is NULL");
  if (!ws || ws_bytes < P.total)
    return fail(PKV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws ? ws_bytes : (size_t)0, P.total);
  if (((uintptr_t)ws) % 256) return fail(PKV_E_WORKSPACE, "workspace must be 256-byte aligned");
  pkv::AttnArgs a = base_args(sh, P);
  a.q = q;
  a.k_pool = (const unsigned char*)k_pool;
  a.v_pool = (const unsigned char*)v_pool;
  a.table = block_table;
  a.seq_lens = seq_lens;
  a.window = window;
  a.mode = mode;
  a.out = out;
  a.lse = lse;
  a.part_o = (float*)((char*)ws + P.off_o);
  a.part_ml = (float*)((char*)ws + P.off_ml);
  a.err = (int32_t*)((char*)ws + P.off_err);
  // planned calls over few sequences derive the list in the split kernel
  a.self_plan = P.planned && sh->n_seqs <= pkv::kSelfPlanMaxSeqs ? 1 : 0;
  a.items = P.planned && !a.self_plan ? (const uint4*)((char*)ws + P.off_items) : nullptr;
  a.hdr = (uint32_t*)((char*)ws + P.off_hdr);
  a.nsub = P.nsub;
  a.fine_tokens = P.fine;
  a.fine_per_seq = P.fine_per_seq;
  a.rows_per_seq = P.rows_per_seq;
  a.seqinfo = (uint4*)((char*)ws + P.off_seq);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (part != kMerge) {
    if (a.flags & PKV_FLAG_CHECKED) {
      e = pkv::launch_zero_words(a.err, 1, s);
      if (e != hipSuccess) return device_fail(e, "clearing the error word");
    }
    if (a.items) {
      e = pkv::launch_decode_plan(a, s);
      if (e != hipSuccess) return device_fail(e, "decode plan launch");
    }
    bool found = false;
    e = pkv::launch_decode_split(a, P.combo, sh->head_dim, sh->block_size, P.g,
                                 P.max_items * sh->n_kv_heads, s, &found);
    if (!found)
      return fail(PKV_E_UNSUPPORTED, "no decode kernel for head_dim %d block %d group %d",
                  sh->head_dim, sh->block_size, P.g);
    if (e != hipSuccess) return device_fail(e, "decode split launch");
  }
  if (part != kPartials) {
    e = pkv::launch_decode_merge(a, sh->head_dim, s);
    if (e != hipSuccess) return device_fail(e, "decode merge launch");
  }
  if (part != kMerge) return finish_checked(a, s);
  return ok();
}

// f32 prefill (q f32; K f32 or q8_0; V f32) runs through the decode
// kernels, one virtual decode sequence per query (prefill_f32.hip): the
// workspace holds the virtual tables, lengths and windows, a flag per query,
// the decode output and the decode workspace.
struct F32Prefill {
  pkv_shape vsh;
  Plan VP;
  int win_ints = 0;
  size_t off_vtable = 0, off_vlens = 0, off_vwin = 0, off_comp = 0, off_out = 0, off_lse = 0, off_dec = 0,
         total = 0;
};

pkv_status plan_f32_prefill(const pkv_shape* sh, int32_t n_q_total, int32_t mode, int32_t n_runs,
                            F32Prefill* F) {
  if (n_q_total > 65535)
    return fail(PKV_E_UNSUPPORTED,
                "f32 prefill computes each query as a decode sequence: n_q_total %d is above 65535", n_q_total);
  F->vsh = *sh;
  F->vsh.n_seqs = n_q_total;
  F->vsh.split_tokens = 0;
  static const int32_t dummy[2] = {0, 0};
  pkv_status st = plan_decode(&F->vsh, mode, n_runs, mode == PKV_WIN_CAUSAL ? nullptr : dummy, &F->VP);
  if (st) return st;
  F->win_ints = mode == PKV_WIN_SPAN ? 2 : (mode == PKV_WIN_KV_MAP ? 2 * n_runs : 0);
  const size_t nq = (size_t)n_q_total;
  F->off_vtable = 0;
  F->off_vlens = F->off_vtable + align_up(nq * sh->max_blocks_per_seq * sizeof(int32_t), 256);
  F->off_vwin = F->off_vlens + align_up(nq * sizeof(int32_t), 256);
  F->off_comp = F->off_vwin + align_up(nq * F->win_ints * sizeof(int32_t), 256);
  F->off_out = F->off_comp + align_up(nq, 256);
  F->off_lse = F->off_out + align_up(nq * sh->n_q_heads * sh->head_dim * sizeof(float), 256);
  F->off_dec = F->off_lse + align_up(nq * sh->n_q_heads * sizeof(float), 256);
  F->total = F->off_dec + F->VP.total;
  return PKV_OK;
}

}  // namespace

namespace pkv_host {
// Error message shared with the pool calls (pool.cpp).
void set_error(const char* msg) { g_err = msg; }
}  // namespace pkv_host

extern "C" {

int64_t pkv_row_bytes(int32_t fmt, int32_t n_kv_heads, int32_t head_dim) {
  return row_bytes_of(fmt, n_kv_heads, head_dim);
}

const char* pkv_last_error(void) { return g_err.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 gfx950"; }

size_t pkv_decode_workspace_bytes(const pkv_shape* shape, int32_t mode, int32_t n_runs) {
  Plan P;
  static const int32_t dummy[2] = {0, 0};
  if (plan_decode(shape, mode, n_runs, mode == PKV_WIN_CAUSAL ? nullptr : dummy, &P)) return 0;
  return P.total;
}

int32_t pkv_decode_split_tokens(const pkv_shape* shape, int32_t mode, int32_t n_runs) {
  Plan P;
  static const int32_t dummy[2] = {0, 0};
  if (plan_decode(shape, mode, n_runs, mode == PKV_WIN_CAUSAL ? nullptr : dummy, &P)) return 0;
  return P.split;
}

pkv_status pkv_paged_attn_decode(const pkv_shape* shape, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t mode, int32_t n_runs,
                                 const int32_t* window, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return decode_impl(kBoth, shape, q, k_pool, v_pool, block_table, seq_lens, mode, n_runs, window,
                     out, lse, workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_attn_decode_partials(const pkv_shape* shape, const void* q,
                                          const void* k_pool, const void* v_pool,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          int32_t mode, int32_t n_runs, const int32_t* window,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(kPartials, shape, q, k_pool, v_pool, block_table, seq_lens, mode, n_runs,
                     window, nullptr, nullptr, workspace, workspace_bytes, stream);
}

pkv_status pkv_paged_attn_decode_merge(const pkv_shape* shape, const int32_t* seq_lens,
                                       int32_t mode, int32_t n_runs, const int32_t* window,
                                       float* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  return decode_impl(kMerge, shape, nullptr, nullptr, nullptr, nullptr, seq_lens, mode, n_runs,
                     window, out, lse, workspace, workspace_bytes, stream);
}

size_t pkv_prefill_workspace_bytes(const pkv_shape* shape, int32_t n_q_total,
                                   int32_t max_q_per_seq, int32_t mode, int32_t n_runs) {
  Plan P;
  static const int32_t dummy[2] = {0, 0};
  if (check_attn(shape, mode, n_runs, mode == PKV_WIN_CAUSAL ? nullptr : dummy, &P)) return 0;
  if (n_q_total < 0 || max_q_per_seq < 0) return 0;
  if (P.combo == pkv::kComboF32 || P.combo == pkv::kComboQ8F) {
    F32Prefill F;
    if (plan_f32_prefill(shape, n_q_total, mode, n_runs, &F)) return 0;
    return F.total;
  }
  pkv::AttnArgs a = base_args(shape, P);
  a.mode = mode;
  a.n_q_total = n_q_total;
  a.max_q = max_q_per_seq;
  bool found = false;
  const size_t need = pkv::prefill_workspace(a, P.combo, shape->head_dim, shape->block_size, P.g, &found);
  return found ? need : 0;
}

pkv_status pkv_paged_attn_prefill_window(const pkv_shape* sh, int32_t n_q_total,
                                         int32_t max_q_per_seq, const void* q,
                                         const int32_t* cu_q, const int32_t* q_pos,
                                         const void* k_pool, const void* v_pool,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         int32_t mode, int32_t n_runs, const int32_t* window,
                                         float* out, float* lse, void* ws, size_t ws_bytes,
                                         void* stream) {
  Plan P;
  pkv_status st = check_attn(sh, mode, n_runs, window, &P);
  if (st) return st;
  if (n_q_total < 0 || max_q_per_seq < 0)
    return fail(PKV_E_ARG, "n_q_total %d and max_q_per_seq %d must be >= 0", n_q_total,
                max_q_per_seq);
  if (sh->n_seqs == 0 || n_q_total == 0 || max_q_per_seq == 0) return ok();
  if (!q || !cu_q || !q_pos || !k_pool || !v_pool || !block_table || !seq_lens || !out)
    return fail(PKV_E_ARG, "prefill inputs and out must be non-NULL");
  pkv::AttnArgs a = base_args(sh, P);
  a.q = q;
  a.cu_q = cu_q;
  a.q_pos = q_pos;
  a.k_pool = (const unsigned char*)k_pool;
  a.v_pool = (const unsigned char*)v_pool;
  a.table = block_table;
  a.seq_lens = seq_lens;
  a.window = window;
  a.mode = mode;
  a.out = out;
  a.lse = lse;
  a.n_q_total = n_q_total;
  a.max_q = max_q_per_seq;
  if (P.combo == pkv::kComboF32 || P.combo == pkv::kComboQ8F) {
    F32Prefill F;
    st = plan_f32_prefill(sh, n_q_total, mode, n_runs, &F);
    if (st) return st;
    if (!ws || ws_bytes < F.total)
      return fail(PKV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  ws ? ws_bytes : (size_t)0, F.total);
    if (((uintptr_t)ws) % 256) return fail(PKV_E_WORKSPACE, "workspace must be 256-byte aligned");
    char* w = (char*)ws;
    int32_t* vtable = (int32_t*)(w + F.off_vtable);
    int32_t* vlens = (int32_t*)(w + F.off_vlens);
    int32_t* vwin = F.win_ints ? (int32_t*)(w + F.off_vwin) : nullptr;
    uint8_t* comp = (uint8_t*)(w + F.off_comp);
    float* tmp_out = (float*)(w + F.off_out);
    float* tmp_lse = (float*)(w + F.off_lse);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = pkv::launch_prefill_expand(a, vtable, vlens, vwin, F.win_ints, comp, s);
    if (e != hipSuccess) return device_fail(e, "prefill expand launch");
    st = decode_impl(kBoth, &F.vsh, q, k_pool, v_pool, vtable, vlens, mode, n_runs, vwin, tmp_out, tmp_lse,
                     w + F.off_dec, F.VP.total, stream);
    if (st) return st;
    e = pkv::launch_prefill_copy_rows(tmp_out, tmp_lse, comp, out, lse, n_q_total, sh->n_q_heads, sh->head_dim, s);
    if (e != hipSuccess) return device_fail(e, "prefill copy launch");
    return ok();
  }
  bool found = false;
  const size_t need = pkv::prefill_workspace(a, P.combo, sh->head_dim, sh->block_size, P.g, &found);
  if (!found)
    return fail(PKV_E_UNSUPPORTED, "no prefill kernel for head_dim %d block %d group %d formats (%s, %s, %s)",
                sh->head_dim, sh->block_size, P.g, fmt_name(sh->q_fmt), fmt_name(sh->k_fmt),
                fmt_name(sh->v_fmt));
  if (need && (!ws || ws_bytes < need))
    return fail(PKV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws ? ws_bytes : (size_t)0, need);
  if (need && ((uintptr_t)ws) % 256) return fail(PKV_E_WORKSPACE, "workspace must be 256-byte aligned");
  a.part_o = (float*)ws;
  a.err = need ? (int32_t*)((char*)ws + need - 256) : nullptr;
  hipStream_t s = (hipStream_t)stream;
  if ((a.flags & PKV_FLAG_CHECKED) && a.err) {
    hipError_t e = pkv::launch_zero_words(a.err, 1, s);
    if (e != hipSuccess) return device_fail(e, "clearing the error word");
  } else {
    a.flags &= ~PKV_FLAG_CHECKED;
  }
  hipError_t e = pkv::launch_prefill(a, P.combo, sh->head_dim, sh->block_size, P.g, s, &found);
  if (e != hipSuccess) return device_fail(e, "prefill launch");
  return finish_checked(a, s);
}

pkv_status pkv_resolve_rows(const pkv_shape* sh, int32_t n_q_total, const int32_t* cu_q,
                            const int32_t* q_pos, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t mode, int32_t n_runs,
                            const int32_t* window, int32_t n_cand, int32_t* rows_out,
                            void* stream) {
  Plan P;
  pkv_status st = check_attn(sh, mode, n_runs, window, &P);
  if (st) return st;
  if (n_q_total < 0 || n_cand < 0) return fail(PKV_E_ARG, "negative n_q_total or n_cand");
  if ((cu_q == nullptr) != (q_pos == nullptr))
    return fail(PKV_E_ARG, "cu_q and q_pos must both be given (prefill) or both be NULL (decode)");
  if (!cu_q && n_q_total != sh->n_seqs)
    return fail(PKV_E_ARG, "decode resolve needs n_q_total == n_seqs (%d != %d)", n_q_total,
                sh->n_seqs);
  if (n_q_total == 0 || n_cand == 0) return ok();
  if (n_q_total > 65535) return fail(PKV_E_ARG, "n_q_total %d above 65535", n_q_total);
  if (!block_table || !seq_lens || !rows_out) return fail(PKV_E_ARG, "NULL input");
  pkv::AttnArgs a = base_args(sh, P);
  a.table = block_table;
  a.seq_lens = seq_lens;
  a.window = window;
  a.mode = mode;
  a.cu_q = cu_q;
  a.q_pos = q_pos;
  a.n_q_total = n_q_total;
  a.flags &= ~PKV_FLAG_CHECKED;
  hipError_t e = pkv::launch_resolve(a, sh->block_size, n_cand, rows_out, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "resolve launch");
  return ok();
}

pkv_status pkv_kv_store(const pkv_shape* sh, int32_t n_tok, int32_t src_fmt, const void* k_new,
                        const void* v_new, const int32_t* seq_ids, const int32_t* positions,
                        const int32_t* block_table, void* k_pool, void* v_pool, int32_t* skipped,
                        void* stream) {
  if (!sh) return fail(PKV_E_ARG, "shape is NULL");
  if (n_tok < 0) return fail(PKV_E_ARG, "negative token count %d", n_tok);
  if (sh->n_seqs < 0 || sh->n_kv_heads <= 0 || sh->block_size <= 0 || sh->n_pool_blocks <= 0 ||
      sh->max_blocks_per_seq <= 0)
    return fail(PKV_E_ARG,
                "n_seqs %d must be >= 0 and n_kv_heads %d, block_size %d, n_pool_blocks %d, "
                "max_blocks_per_seq %d positive",
                sh->n_seqs, sh->n_kv_heads, sh->block_size, sh->n_pool_blocks,
                sh->max_blocks_per_seq);
  if (src_fmt != PKV_F32 && src_fmt != PKV_F16)
    return fail(PKV_E_ARG, "source format must be f32 or f16, got %s", fmt_name(src_fmt));
  for (int f : {sh->k_fmt, sh->v_fmt})
    if (f != PKV_F32 && f != PKV_F16 && f != PKV_Q8_0)
      return fail(PKV_E_ARG, "unknown KV format value %d", f);
  const int hd = sh->head_dim;
  if (hd != 32 && hd != 64 && hd != 128 && hd != 256)
    return fail(PKV_E_UNSUPPORTED, "store supports head_dim 32, 64, 128 and 256, not %d", hd);
  if ((int64_t)n_tok * sh->n_kv_heads > INT32_MAX)
    return fail(PKV_E_ARG, "n_tok * n_kv_heads exceeds 2^31 - 1");
  if ((int64_t)sh->n_pool_blocks * sh->n_kv_heads * sh->block_size > INT32_MAX)
    return fail(PKV_E_ARG, "n_pool_blocks * n_kv_heads * block_size exceeds 2^31 - 1");
  if ((int64_t)sh->max_blocks_per_seq * sh->block_size > INT32_MAX)
    return fail(PKV_E_ARG, "max_blocks_per_seq * block_size overflows int32");
  if (!seq_ids && n_tok > sh->n_seqs)
    return fail(PKV_E_ARG, "without seq_ids token t belongs to sequence t: n_tok %d > n_seqs %d",
                n_tok, sh->n_seqs);
  if (n_tok == 0) return ok();  // nothing is read, so no pointer is checked
  if (!k_new || !k_pool || !positions || !block_table)
    return fail(PKV_E_ARG, "k_new, k_pool, positions and block_table must be non-NULL");
  if ((v_new == nullptr) != (v_pool == nullptr))
    return fail(PKV_E_ARG, "v_new and v_pool must both be given or both be NULL");
  for (const void* p : {k_new, v_new, (const void*)k_pool, (const void*)v_pool})
    if (((uintptr_t)p) % 16) return fail(PKV_E_ARG, "sources and pools must be 16-byte aligned");
  pkv::StoreArgs a{};
  a.src[0] = (const unsigned char*)k_new;
  a.src[1] = (const unsigned char*)v_new;
  a.pool[0] = (unsigned char*)k_pool;
  a.pool[1] = (unsigned char*)v_pool;
  a.fmt[0] = sh->k_fmt;
  a.fmt[1] = sh->v_fmt;
  a.seq_ids = seq_ids;
  a.pos = positions;
  a.table = block_table;
  a.skipped = skipped;
  a.n_tok = n_tok;
  a.n_seqs = sh->n_seqs;
  a.n_kv_heads = sh->n_kv_heads;
  a.block_size = sh->block_size;
  a.n_pool_blocks = sh->n_pool_blocks;
  a.max_blocks = sh->max_blocks_per_seq;
  bool found = false;
  hipError_t e = pkv::launch_store(a, src_fmt, hd, (hipStream_t)stream, &found);
  if (!found) return fail(PKV_E_UNSUPPORTED, "no store kernel for head_dim %d", hd);
  if (e != hipSuccess) return device_fail(e, "store launch");
  return ok();
}

pkv_status pkv_cow_apply(void* k_pool, void* v_pool, int32_t n_pool_blocks, int64_t k_block_bytes,
                         int64_t v_block_bytes, const int32_t* ops, int32_t n, int32_t* table,
                         int64_t table_entries, void* stream) {
  if (n < 0) return fail(PKV_E_ARG, "negative op count %d", n);
  if (n == 0) return ok();
  if (!k_pool || !ops) return fail(PKV_E_ARG, "k_pool and ops must be non-NULL");
  if (n_pool_blocks <= 0) return fail(PKV_E_ARG, "n_pool_blocks %d must be positive", n_pool_blocks);
  if (k_block_bytes <= 0 || k_block_bytes % 4 || (v_pool && (v_block_bytes <= 0 || v_block_bytes % 4)))
    return fail(PKV_E_ARG, "block bytes must be positive multiples of 4");
  if (table && table_entries < 0) return fail(PKV_E_ARG, "negative table size");
  if (k_block_bytes > ((int64_t)65535 << 13) || v_block_bytes > ((int64_t)65535 << 13))
    return fail(PKV_E_ARG, "blocks larger than 512 MiB are not supported");
  for (const void* p : {(const void*)k_pool, (const void*)v_pool})
    if (((uintptr_t)p) % 16) return fail(PKV_E_ARG, "pools must be 16-byte aligned");
  pkv::CowArgs a{};
  a.pool[0] = (unsigned char*)k_pool;
  a.pool[1] = (unsigned char*)v_pool;
  a.block_bytes[0] = k_block_bytes;
  a.block_bytes[1] = v_pool ? v_block_bytes : 0;
  a.ops = ops;
  a.table = table;
  a.table_entries = table ? table_entries : 0;
  a.n_ops = n;
  a.n_blocks = n_pool_blocks;
  hipError_t e = pkv::launch_cow_apply(a, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "cow_apply launch");
  return ok();
}

int64_t pkv_int4_blob_bytes(int64_t n_elts) { return n_elts < 0 ? 0 : 4 + (n_elts + 1) / 2; }

namespace {
pkv_status int4_call(bool encode, void* pool, int32_t fmt, int32_t n_pool_blocks, int64_t block_elems,
                     const int32_t* blocks, int32_t n, void* blobs, int64_t blob_stride, void* stream) {
  if (n < 0) return fail(PKV_E_ARG, "negative block count %d", n);
  if (fmt != PKV_F16 && fmt != PKV_F32)
    return fail(PKV_E_UNSUPPORTED, "the int4 codec reads and writes f16 or f32 pools, not %s", fmt_name(fmt));
  if (n_pool_blocks <= 0) return fail(PKV_E_ARG, "n_pool_blocks %d must be positive", n_pool_blocks);
  if (block_elems <= 0 || block_elems % 8 || block_elems > 65536)
    return fail(PKV_E_UNSUPPORTED, "block_elems %lld must be a positive multiple of 8 up to 65536",
                (long long)block_elems);
  if (blob_stride < pkv_int4_blob_bytes(block_elems) || blob_stride % 4)
    return fail(PKV_E_ARG, "blob_stride %lld must be a multiple of 4 of at least %lld bytes",
                (long long)blob_stride, (long long)pkv_int4_blob_bytes(block_elems));
  if (n == 0) return ok();
  if (!pool || !blocks || !blobs) return fail(PKV_E_ARG, "pool, blocks and blobs must be non-NULL");
  if (((uintptr_t)pool) % 16 || ((uintptr_t)blobs) % 4)
    return fail(PKV_E_ARG, "the pool must be 16-byte and the blobs 4-byte aligned");
  pkv::Int4Args a{};
  a.pool = (unsigned char*)pool;
  a.blobs = (unsigned char*)blobs;
  a.blocks = blocks;
  a.blob_stride = blob_stride;
  a.block_elems = block_elems;
  a.n = n;
  a.n_pool_blocks = n_pool_blocks;
  hipError_t e = pkv::launch_int4(encode, a, fmt, (hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, encode ? "int4 encode launch" : "int4 decode launch");
  return ok();
}
}  // namespace

pkv_status pkv_int4_encode(const void* pool, int32_t fmt, int32_t n_pool_blocks, int64_t block_elems,
                           const int32_t* blocks, int32_t n, void* blobs, int64_t blob_stride,
                           void* stream) {
  return int4_call(true, (void*)pool, fmt, n_pool_blocks, block_elems, blocks, n, blobs, blob_stride,
                   stream);
}

pkv_status pkv_int4_decode(const void* blobs, int64_t blob_stride, int32_t n, void* pool, int32_t fmt,
                           int32_t n_pool_blocks, int64_t block_elems, const int32_t* blocks,
                           void* stream) {
  return int4_call(false, pool, fmt, n_pool_blocks, block_elems, blocks, n, (void*)blobs, blob_stride,
                   stream);
}

}  // extern "C"
