// C ABI of the paged-attention library: argument validation, dispatch over
// (head_dim, block_size, group, formats), split planning, order_moves and
// the copy_cells plan.  Every host-checkable condition is checked before
// the first launch, so a refused call leaves outputs and pools untouched.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
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
  const int64_t target = 3072;
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

// order_moves: indices of the effective moves, upward moves (dst > src) by
// descending src then descending dst, then downward moves by ascending src
// then ascending dst; ties by input index.
// Stable LSD radix sort of (key, index) pairs by key, 8 bits per pass;
// passes whose digit is the same for every key are skipped.
void radix_sort_pairs(std::vector<std::pair<uint64_t, int32_t>>* v) {
  // host buffers keep their capacity between calls (no page faults in
  // steady state); thread-local, so concurrent callers do not share them
  static thread_local std::vector<std::pair<uint64_t, int32_t>> tmp;
  tmp.resize(v->size());
  uint64_t all_or = 0, all_and = ~0ull;
  for (const auto& x : *v) {
    all_or |= x.first;
    all_and &= x.first;
  }
  for (int shift = 0; shift < 64; shift += 8) {
    if ((((all_or ^ all_and) >> shift) & 0xFF) == 0) continue;  // constant digit
    size_t count[257] = {0};
    for (const auto& x : *v) ++count[((x.first >> shift) & 0xFF) + 1];
    for (int b = 0; b < 256; ++b) count[b + 1] += count[b];
    for (const auto& x : *v) tmp[count[(x.first >> shift) & 0xFF]++] = x;
    v->swap(tmp);
  }
}

// order_moves: moves with dst > src first, by src then dst descending; then
// moves with dst < src, by src then dst ascending; ties keep input order.
// Moves with len <= 0 or src == dst are dropped.  (Keys are built so that an
// ascending stable sort gives that order: flipping the sign bit maps int32
// onto uint32 in order, and 2^32 - 1 - x reverses it.)
// The result lives in a thread-local buffer, valid until the next call.
const std::vector<int32_t>& order_moves_impl(const int32_t* mv, int32_t n) {
  static thread_local std::vector<std::pair<uint64_t, int32_t>> up, down;
  static thread_local std::vector<int32_t> o;
  up.clear();
  down.clear();
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = mv[3 * i], d = mv[3 * i + 1], len = mv[3 * i + 2];
    if (len <= 0 || d == s) continue;
    const uint64_t us = (uint32_t)s ^ 0x80000000u, ud = (uint32_t)d ^ 0x80000000u;
    if (d > s) up.push_back({((0xFFFFFFFFull - us) << 32) | (0xFFFFFFFFull - ud), i});
    else down.push_back({(us << 32) | ud, i});
  }
  radix_sort_pairs(&up);
  radix_sort_pairs(&down);
  o.clear();
  for (const auto& x : up) o.push_back(x.second);
  for (const auto& x : down) o.push_back(x.second);
  return o;
}

// The effective moves (len > 0, src != dst) as (src, dst, len), and whether
// they are disjoint: destinations do not overlap each other and no
// destination overlaps any source.  Then every application order gives the
// same bytes and all rows can be copied at once.
bool disjoint_moves(const int32_t* mv, int32_t n, std::vector<int32_t>* eff) {
  eff->clear();
  for (int32_t i = 0; i < n; ++i) {
    const int64_t s = mv[3 * i], d = mv[3 * i + 1], len = mv[3 * i + 2];
    if (len <= 0 || s == d) continue;
    if (s < d + len && d < s + len) return false;  // a move overlapping itself (a slide)
    eff->insert(eff->end(), {(int32_t)s, (int32_t)d, (int32_t)len});
  }
  const size_t m = eff->size() / 3;
  static thread_local std::vector<std::pair<int64_t, int64_t>> src, dst;
  src.clear();
  dst.clear();
  for (size_t i = 0; i < m; ++i) {
    const int64_t s = (*eff)[3 * i], d = (*eff)[3 * i + 1], len = (*eff)[3 * i + 2];
    src.push_back({s, s + len});
    dst.push_back({d, d + len});
  }
  std::sort(dst.begin(), dst.end());
  for (size_t i = 1; i < dst.size(); ++i)
    if (dst[i].first < dst[i - 1].second) return false;  // two destinations overlap
  std::sort(src.begin(), src.end());
  // destinations are disjoint and sorted; a source overlaps one iff the
  // first destination ending after the source's start begins before its end
  size_t j = 0;
  for (const auto& sr : src) {
    while (j < dst.size() && dst[j].second <= sr.first) ++j;
    if (j < dst.size() && dst[j].first < sr.second) return false;
  }
  return true;
}

// Pinned host staging for plan uploads: grown to the largest plan so far and
// kept until the process ends; one upload at a time.
// Pinned staging for host -> device plan uploads: two buffers per device,
// used in turn, each with an event recorded after its copy, so a call waits
// only for the previous upload out of the same buffer (never for the rest of
// the stream) before refilling it.  Allocated on first use, grown to the
// largest plan seen, kept until the process ends; the mutex makes
// concurrent callers take turns.
struct StageSet {
  void* buf[2] = {nullptr, nullptr};
  size_t bytes[2] = {0, 0};
  hipEvent_t ev[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  int next = 0;
};
std::mutex g_stage_mu;
std::map<int, StageSet> g_stages;

// A pinned host buffer of at least `bytes`, held (with the mutex) until
// commit() sends it to the device.
class StagedUpload {
 public:
  hipError_t begin(size_t bytes) {
    lock_ = std::unique_lock<std::mutex>(g_stage_mu);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    set_ = &g_stages[dev];
    i_ = set_->next;
    set_->next ^= 1;
    if (set_->pending[i_]) {
      e = hipEventSynchronize(set_->ev[i_]);
      if (e != hipSuccess) return e;
      set_->pending[i_] = false;
    }
    if (!set_->ev[i_]) {
      e = hipEventCreateWithFlags(&set_->ev[i_], hipEventDisableTiming);
      if (e != hipSuccess) {
        set_->ev[i_] = nullptr;
        return e;
      }
    }
    if (set_->bytes[i_] < bytes) {
      if (set_->buf[i_]) (void)hipHostFree(set_->buf[i_]);
      set_->buf[i_] = nullptr;
      set_->bytes[i_] = 0;
      const size_t want = std::max(bytes, (size_t)1 << 20);
      e = hipHostMalloc(&set_->buf[i_], want, hipHostMallocDefault);
      if (e != hipSuccess) {
        set_->buf[i_] = nullptr;
        return e;
      }
      set_->bytes[i_] = want;
    }
    return hipSuccess;
  }
  void* host() const { return set_->buf[i_]; }
  // Copies the first `bytes` of the buffer to `dst` on `st` (asynchronous).
  hipError_t commit(void* dst, size_t bytes, hipStream_t st) {
    hipError_t e = hipSuccess;
    if (bytes) {
      e = hipMemcpyAsync(dst, set_->buf[i_], bytes, hipMemcpyHostToDevice, st);
      if (e == hipSuccess) e = hipEventRecord(set_->ev[i_], st);
      if (e == hipSuccess) set_->pending[i_] = true;
    }
    lock_.unlock();
    return e;
  }

 private:
  std::unique_lock<std::mutex> lock_;
  StageSet* set_ = nullptr;
  int i_ = 0;
};

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

pkv_status pkv_order_moves(const int32_t* moves, int32_t n, int32_t* order_out, int32_t* n_out) {
  if (n < 0) return fail(PKV_E_ARG, "negative move count %d", n);
  if (n > 0 && (!moves || !order_out)) return fail(PKV_E_ARG, "moves and order_out must be non-NULL");
  if (!n_out) return fail(PKV_E_ARG, "n_out is NULL");
  const std::vector<int32_t>& o = order_moves_impl(moves, n);
  std::copy(o.begin(), o.end(), order_out);
  *n_out = (int32_t)o.size();
  return ok();
}

size_t pkv_copy_cells_workspace_bytes(const int32_t* moves, int32_t n, int64_t row_bytes_k,
                                      int64_t row_bytes_v) {
  if (n < 0 || (n > 0 && !moves) || row_bytes_k <= 0 || row_bytes_v < 0) return 0;
  static thread_local std::vector<int32_t> eff;
  if (disjoint_moves(moves, n, &eff))  // moves and their prefix sums only
    return align_up((eff.size() + eff.size() / 3 + 1) * sizeof(int32_t), 256) + 256;
  int64_t rows = 0;
  for (int32_t i = 0; i < n; ++i)
    if (moves[3 * i + 2] > 0 && moves[3 * i] != moves[3 * i + 1]) rows += moves[3 * i + 2];
  return align_up((size_t)rows * 2 * sizeof(int32_t) * 2, 256) +
         align_up((size_t)rows * (size_t)row_bytes_k, 256) +
         align_up((size_t)rows * (size_t)row_bytes_v, 256) + 256;
}

pkv_status pkv_kv_copy_cells(void* k_pool, void* v_pool, int32_t n_pool_blocks, int32_t block_size,
                             int32_t n_kv_heads, int64_t seg_bytes_k, int64_t seg_bytes_v,
                             const int32_t* moves, int32_t n, void* ws, size_t ws_bytes,
                             void* stream) {
  if (!k_pool) return fail(PKV_E_ARG, "k_pool is NULL");
  if (n < 0) return fail(PKV_E_ARG, "negative move count %d", n);
  if (n > 0 && !moves) return fail(PKV_E_ARG, "moves is NULL");
  if (n_pool_blocks <= 0 || block_size <= 0 || n_kv_heads <= 0)
    return fail(PKV_E_ARG, "n_pool_blocks %d, block_size %d and n_kv_heads %d must be positive",
                n_pool_blocks, block_size, n_kv_heads);
  const int64_t n_pool_rows = (int64_t)n_pool_blocks * block_size;
  if (n_pool_rows > INT32_MAX)
    return fail(PKV_E_ARG, "%lld pool rows exceed 2^31 - 1", (long long)n_pool_rows);
  if (seg_bytes_k <= 0 || seg_bytes_k % 4)
    return fail(PKV_E_ARG, "seg_bytes_k %lld must be a positive multiple of 4", (long long)seg_bytes_k);
  if (v_pool && (seg_bytes_v <= 0 || seg_bytes_v % 4))
    return fail(PKV_E_ARG, "seg_bytes_v %lld must be a positive multiple of 4", (long long)seg_bytes_v);
  int64_t lo = INT64_MAX, hi = -1;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t s = moves[3 * i], d = moves[3 * i + 1], len = moves[3 * i + 2];
    if (len <= 0 || s == d) continue;
    if (s < 0 || d < 0 || s + len > n_pool_rows || d + len > n_pool_rows)
      return fail(PKV_E_ARG, "move %d (src %lld, dst %lld, len %lld) leaves [0, %lld)", i,
                  (long long)s, (long long)d, (long long)len, (long long)n_pool_rows);
    lo = std::min(lo, std::min(s, d));
    hi = std::max(hi, std::max(s, d) + len);
  }
  const std::vector<int32_t>& order = order_moves_impl(moves, n);
  if (order.empty()) return ok();
  hipStream_t st = (hipStream_t)stream;
  static thread_local std::vector<int32_t> eff;
  if (disjoint_moves(moves, n, &eff)) {
    // No destination touches a source: copy every run at once.  Upload:
    // the moves, then the prefix sums of their lengths.
    const int32_t m = (int32_t)(eff.size() / 3);
    const size_t n_words = eff.size() + (size_t)m + 1;
    const size_t need = align_up(n_words * sizeof(int32_t), 256) + 256;
    if (!ws || ws_bytes < need)
      return fail(PKV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                  ws ? ws_bytes : (size_t)0, need);
    StagedUpload stage;
    hipError_t e = stage.begin(n_words * sizeof(int32_t));
    if (e != hipSuccess) return device_fail(e, "pinned staging buffer");
    int32_t* h = (int32_t*)stage.host();
    std::memcpy(h, eff.data(), eff.size() * sizeof(int32_t));
    int32_t* cum = h + eff.size();
    int64_t total = 0;
    cum[0] = 0;
    for (int32_t i = 0; i < m; ++i) {
      total += eff[3 * i + 2];
      cum[i + 1] = (int32_t)total;  // total <= pool rows < 2^31
    }
    e = stage.commit(ws, n_words * sizeof(int32_t), st);
    if (e != hipSuccess) return device_fail(e, "uploading the moves");
    const int32_t* d_moves = (const int32_t*)ws;
    const int32_t* d_cum = d_moves + eff.size();
    for (const pkv::PoolGeom g : {pkv::PoolGeom{(unsigned char*)k_pool, seg_bytes_k, n_kv_heads, block_size},
                                  pkv::PoolGeom{(unsigned char*)v_pool, seg_bytes_v, n_kv_heads, block_size}}) {
      if (!g.base) continue;
      e = pkv::launch_copy_runs(g, d_moves, d_cum, m, (int32_t)total, st);
      if (e != hipSuccess) return device_fail(e, "copy_cells run launch");
    }
    return ok();
  }
  // Final source of every row of [lo, hi) after the ordered memmoves.
  static thread_local std::vector<int32_t> prov, stage_of;
  static thread_local std::vector<char> changed;
  prov.resize(hi - lo);
  for (int64_t r = lo; r < hi; ++r) prov[r - lo] = (int32_t)r;
  for (int32_t i : order) {
    const int64_t s = moves[3 * i], d = moves[3 * i + 1], len = moves[3 * i + 2];
    std::memmove(&prov[d - lo], &prov[s - lo], (size_t)len * sizeof(int32_t));
  }
  changed.assign(hi - lo, 0);
  int64_t n_changed = 0;
  for (int64_t r = lo; r < hi; ++r)
    if (prov[r - lo] != r) {
      changed[r - lo] = 1;
      ++n_changed;
    }
  // Rows read from a row that is also written go through the stage.  The
  // plan goes straight into the pinned upload buffer: gather pairs (source
  // row, stage slot) from the start, scatter pairs (row, source row or
  // -(stage slot + 1)) from word 2 * n_changed on (gather pairs never
  // outnumber changed rows).
  const int64_t row_k = seg_bytes_k * n_kv_heads, row_v = v_pool ? seg_bytes_v * n_kv_heads : 0;
  const size_t n_words = 4 * (size_t)n_changed;
  const size_t idx_bytes = align_up(n_words * sizeof(int32_t), 256);
  if (!ws || ws_bytes < idx_bytes)
    return fail(PKV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws ? ws_bytes : (size_t)0, idx_bytes);
  StagedUpload upl;
  hipError_t e = upl.begin(n_words * sizeof(int32_t));
  if (e != hipSuccess) return device_fail(e, "pinned staging buffer");
  int32_t* gather = (int32_t*)upl.host();
  int32_t* scatter = gather + 2 * n_changed;
  stage_of.assign(hi - lo, -1);
  int32_t n_stage = 0, n_scatter = 0;
  for (int64_t r = lo; r < hi; ++r) {
    if (!changed[r - lo]) continue;
    const int32_t src = prov[r - lo];
    int32_t y = src;
    if (changed[src - lo]) {
      if (stage_of[src - lo] < 0) {
        gather[2 * n_stage] = src;
        gather[2 * n_stage + 1] = n_stage;
        stage_of[src - lo] = n_stage++;
      }
      y = -(stage_of[src - lo] + 1);
    }
    scatter[2 * n_scatter] = (int32_t)r;
    scatter[2 * n_scatter + 1] = y;
    ++n_scatter;
  }
  const size_t stage_k = align_up((size_t)n_stage * (size_t)row_k, 256);
  const size_t stage_v = align_up((size_t)n_stage * (size_t)row_v, 256);
  const size_t need = idx_bytes + stage_k + stage_v;
  if (ws_bytes < need) {
    (void)upl.commit(nullptr, 0, st);
    return fail(PKV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws_bytes, need);
  }
  int32_t* d_idx = (int32_t*)ws;
  unsigned char* stage = (unsigned char*)ws + idx_bytes;
  e = upl.commit(d_idx, n_words * sizeof(int32_t), st);
  if (e != hipSuccess) return device_fail(e, "uploading the move plan");
  const int32_t n_gather = n_stage;
  const int32_t* d_gather = d_idx;
  const int32_t* d_scatter = d_idx + 2 * n_changed;
  struct Pool { pkv::PoolGeom g; unsigned char* stage; } pools[2] = {
      {{(unsigned char*)k_pool, seg_bytes_k, n_kv_heads, block_size}, stage},
      {{(unsigned char*)v_pool, seg_bytes_v, n_kv_heads, block_size}, stage + stage_k}};
  for (const Pool& pl : pools) {
    if (!pl.g.base) continue;
    e = pkv::launch_copy_rows(1, pl.g, pl.stage, d_gather, n_gather, st);
    if (e != hipSuccess) return device_fail(e, "copy_cells gather launch");
  }
  for (const Pool& pl : pools) {
    if (!pl.g.base) continue;
    e = pkv::launch_copy_rows(2, pl.g, pl.stage, d_scatter, n_scatter, st);
    if (e != hipSuccess) return device_fail(e, "copy_cells scatter launch");
  }
  return ok();
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
