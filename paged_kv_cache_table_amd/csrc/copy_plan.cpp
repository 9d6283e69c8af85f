// order_moves and the copy_cells plan on the host, and the device apply
// ("KV Cache Design — cells, format, sessions", section 2: a compaction
// changes only cells; rows move verbatim through copy_cells in order_moves
// order — upward moves top-down, downward moves bottom-up, upward first —
// so that no destination lands on a row that is not yet copied).
//
// The host functions are pure: every buffer they use is local to the call
// or the caller's, so they hold no state between calls and any thread may
// call them.  The device half only launches kernels.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "pkv_internal.hpp"

namespace pkv_host {
void set_error(const char* msg);
}

namespace {

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  pkv_host::set_error(buf);
  return st;
}

pkv_status ok() {
  pkv_host::set_error("");
  return PKV_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int bits_for(uint64_t range) {  // bits that hold every value in [0, range)
  int b = 0;
  while (b < 63 && ((uint64_t)1 << b) < range) ++b;
  return b;
}

// The moves that do something (len > 0 and src != dst), in input order:
// int32 (src, dst, len, input index).
struct Move {
  int32_t s, d, len, idx;
};

// What one plan needs, from a pass over the moves.
struct Shape {
  int64_t m = 0;       // effective moves
  int64_t rows = 0;    // sum of their lengths
  int64_t lo = 0, hi = 0;  // span of all their source and destination rows
};

Shape shape_of(const int32_t* mv, int32_t n) {
  Shape sh;
  sh.lo = INT64_MAX;
  sh.hi = INT64_MIN;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t s = mv[3 * i], d = mv[3 * i + 1], len = mv[3 * i + 2];
    if (len <= 0 || s == d) continue;
    ++sh.m;
    sh.rows += len;
    sh.lo = std::min(sh.lo, std::min(s, d));
    sh.hi = std::max(sh.hi, std::max(s, d) + len);
  }
  if (!sh.m) sh.lo = sh.hi = 0;
  return sh;
}

// The caller's plan buffer, carved into the plan itself (at the front) and
// the planner's working arrays, so that a call allocates nothing.  Words:
//   plan      max(4m + 1, 4 rows)            the result
//   eff       4m                             Move records
//   order     m                              application order (eff positions)
//   ivl       8m (int64 pairs)               union intervals (start, offset)
//   work      max(8m, bitmap, 2 span + 2 rows + span / 32 + 2), 8-byte aligned
// where span = rows of the index array (the touched span when it is at
// most 2 rows long, else the union of the ranges, at most 2 rows) and
// bitmap = words of a bitmap over the touched span (disjointness test,
// only when that span is at most 2^28 rows).
struct Layout {
  int64_t plan, eff, order, ivl, work, total;
};

int64_t span_rows(const Shape& sh) {
  const int64_t span = sh.hi - sh.lo;
  return span <= 2 * sh.rows ? span : 2 * sh.rows;
}

Layout layout_of(const Shape& sh) {
  Layout L{};
  if (!sh.m) return L;
  const int64_t m = sh.m;
  const int64_t plan = std::max(4 * m + 1, 4 * sh.rows);
  const int64_t span = sh.hi - sh.lo;
  const int64_t bitmap = span <= ((int64_t)1 << 28) ? 2 * ((span + 63) / 64) : 0;
  const int64_t sr = span_rows(sh);
  const int64_t work = std::max(8 * m, std::max(bitmap, 2 * sr + 2 * sh.rows + 2 * ((sr + 63) / 64) + 2));
  L.plan = 0;
  L.eff = plan;
  L.order = L.eff + 4 * m;
  L.ivl = (L.order + m + 1) / 2 * 2;  // 8-byte aligned
  L.work = L.ivl + 8 * m;
  L.total = L.work + work;
  return L;
}

// Stable LSD radix sort of v[0, n) on bits [lo_bit, hi_bit), 8 bits per
// pass, through tmp; passes whose digit is the same for every item are
// skipped.  Returns the array holding the result (v or tmp).
uint64_t* radix_sort(uint64_t* v, uint64_t* tmp, int64_t n, int lo_bit, int hi_bit) {
  if (n < 2) return v;
  uint64_t all_or = 0, all_and = ~0ull;
  for (int64_t i = 0; i < n; ++i) {
    all_or |= v[i];
    all_and &= v[i];
  }
  for (int sh = lo_bit; sh < hi_bit; sh += 8) {
    const int w = hi_bit - sh < 8 ? hi_bit - sh : 8;
    const uint64_t mask = ((uint64_t)1 << w) - 1;
    if ((((all_or ^ all_and) >> sh) & mask) == 0) continue;  // constant digit
    uint32_t count[257] = {0};
    for (int64_t i = 0; i < n; ++i) ++count[((v[i] >> sh) & mask) + 1];
    for (int b = 0; b < 256; ++b) count[b + 1] += count[b];
    for (int64_t i = 0; i < n; ++i) tmp[count[(v[i] >> sh) & mask]++] = v[i];
    std::swap(v, tmp);
  }
  return v;
}

// order_moves into order[0, m) (positions in eff): upward moves (dst > src)
// by descending src, then descending dst; then downward moves by ascending
// src, then ascending dst; ties by input index.  Each item packs the src
// key above the dst key and the position; the items are radix-sorted on
// the src key alone (stable, so positions stay in order), then runs of
// equal src are sorted on the whole item.  When an item does not fit 64
// bits, a comparison sort does the same.  work: 4m words, 8-byte aligned.
void order_moves(const Move* eff, int64_t m, int32_t* order, uint64_t* work) {
  if (!m) return;
  int64_t lo = INT64_MAX, hi = INT64_MIN;
  for (int64_t k = 0; k < m; ++k) {
    lo = std::min<int64_t>(lo, std::min(eff[k].s, eff[k].d));
    hi = std::max<int64_t>(hi, std::max(eff[k].s, eff[k].d));
  }
  const uint64_t range = (uint64_t)(hi - lo) + 1;
  const int br = bits_for(range), bi = bits_for((uint64_t)m);
  if (2 * br + bi <= 64) {
    // one pass builds both key lists without branching: every move's keys
    // are written, and only its own list's count advances
    uint64_t* vu = work;          // upward moves: descending keys, as ascending complements
    uint64_t* vd = work + m;      // downward moves
    uint64_t* tmp = work + 2 * m;
    int64_t nu = 0, nd = 0;
    for (int64_t k = 0; k < m; ++k) {
      const Move& x = eff[k];
      const uint64_t a = (uint64_t)(x.s - lo), b = (uint64_t)(x.d - lo);
      const int up = x.d > x.s;
      vu[nu] = ((range - 1 - a) << (br + bi)) | ((range - 1 - b) << bi) | (uint64_t)k;
      vd[nd] = (a << (br + bi)) | (b << bi) | (uint64_t)k;
      nu += up;
      nd += 1 - up;
    }
    int64_t placed = 0;
    const uint64_t pmask = ((uint64_t)1 << bi) - 1;
    for (int up = 1; up >= 0; --up) {
      const int64_t n = up ? nu : nd;
      // radix sort on the src key alone (stable: positions stay in order),
      // then runs of equal src keys on (dst key, position)
      uint64_t* v = radix_sort(up ? vu : vd, tmp, n, br + bi, 2 * br + bi);
      for (int64_t i = 0; i < n;) {
        int64_t j = i + 1;
        while (j < n && (v[j] >> (br + bi)) == (v[i] >> (br + bi))) ++j;
        if (j - i > 1) std::sort(v + i, v + j);
        i = j;
      }
      for (int64_t i = 0; i < n; ++i) order[placed++] = (int32_t)(v[i] & pmask);
      if (up) tmp = vu;  // vu's storage is free once its order is out
    }
    return;
  }
  int64_t placed = 0;
  for (int up = 1; up >= 0; --up) {
    const int64_t n0 = placed;
    for (int64_t k = 0; k < m; ++k)
      if ((eff[k].d > eff[k].s) == (up == 1)) order[placed++] = (int32_t)k;
    std::stable_sort(order + n0, order + placed, [&](int32_t x, int32_t y) {
      const Move &a = eff[x], &b = eff[y];
      if (a.s != b.s) return up ? a.s > b.s : a.s < b.s;
      if (a.d != b.d) return up ? a.d > b.d : a.d < b.d;
      return false;
    });
  }
}

// Whether no destination overlaps another destination or any source (then
// every application order gives the same bytes): a bitmap of destination
// rows over the touched span (bits: the work array) when that span is at
// most 2^28 rows, else sorted intervals.
bool disjoint(const Move* eff, int64_t m, const Shape& sh, uint64_t* bits) {
  for (int64_t k = 0; k < m; ++k) {
    const Move& x = eff[k];
    if (x.s < x.d + x.len && x.d < x.s + x.len) return false;  // a move overlapping itself
  }
  const int64_t span = sh.hi - sh.lo;
  if (span <= ((int64_t)1 << 28)) {
    const int64_t nw = (span + 63) / 64;
    std::fill(bits, bits + nw, 0ull);
    // visit the rows [a, b) of the bitmap word by word; f(word, mask)
    auto words = [&](int64_t a, int64_t b, auto f) {
      a -= sh.lo;
      b -= sh.lo;
      while (a < b) {
        const int64_t w = a >> 6, o = a & 63;
        const int64_t n = std::min<int64_t>(64 - o, b - a);
        const uint64_t mask = (n == 64 ? ~0ull : (((uint64_t)1 << n) - 1)) << o;
        if (!f(bits[w], mask)) return false;
        a += n;
      }
      return true;
    };
    for (int64_t k = 0; k < m; ++k) {
      const bool fresh = words(eff[k].d, (int64_t)eff[k].d + eff[k].len, [](uint64_t& word, uint64_t mask) {
        if (word & mask) return false;
        word |= mask;
        return true;
      });
      if (!fresh) return false;  // two destinations overlap
    }
    for (int64_t k = 0; k < m; ++k) {
      const bool clear = words(eff[k].s, (int64_t)eff[k].s + eff[k].len,
                               [](uint64_t& word, uint64_t mask) { return (word & mask) == 0; });
      if (!clear) return false;  // a source is some move's destination
    }
    return true;
  }
  std::vector<std::pair<int64_t, int64_t>> src, dst;  // rare: spans above 2^28 rows
  for (int64_t k = 0; k < m; ++k) {
    src.push_back({eff[k].s, (int64_t)eff[k].s + eff[k].len});
    dst.push_back({eff[k].d, (int64_t)eff[k].d + eff[k].len});
  }
  std::sort(dst.begin(), dst.end());
  for (size_t i = 1; i < dst.size(); ++i)
    if (dst[i].first < dst[i - 1].second) return false;
  std::sort(src.begin(), src.end());
  size_t j = 0;
  for (const auto& sr : src) {
    while (j < dst.size() && dst[j].second <= sr.first) ++j;
    if (j < dst.size() && dst[j].first < sr.second) return false;
  }
  return true;
}

// The final source of every row the ordered moves touch, replayed on an
// index array, then the gather/scatter lists.  The rows that matter are the
// union U of the moves' source and destination ranges.  When the touched
// span is at most twice the rows the moves name, the index array covers
// the span directly; otherwise U is laid out compactly (its intervals in
// order, one after another) and, since each range lies inside one interval
// of U, each move is still one contiguous copy there.
void stage_plan(const Move* eff, int64_t m, const Shape& sh, const int32_t* order, int64_t* ivl, int32_t* work,
                int32_t* plan, pkv_copy_plan* info) {
  const bool dense = sh.hi - sh.lo <= 2 * sh.rows;
  int64_t n_iv = 0, n_rows = 0;
  int64_t* ustart = ivl;        // [n_iv <= 2m] first row of each union interval
  int64_t* uoff = ivl + 2 * m;  // [n_iv] its offset in the compact array
  if (dense) {
    n_rows = sh.hi - sh.lo;
  } else {
    // sort the 2m ranges by start in the work array, then merge
    int64_t* iv = (int64_t*)work;  // [2m][2]
    for (int64_t k = 0; k < m; ++k) {
      iv[4 * k] = eff[k].s;
      iv[4 * k + 1] = (int64_t)eff[k].s + eff[k].len;
      iv[4 * k + 2] = eff[k].d;
      iv[4 * k + 3] = (int64_t)eff[k].d + eff[k].len;
    }
    auto* pr = (std::pair<int64_t, int64_t>*)iv;
    std::sort(pr, pr + 2 * m);
    int64_t cur_s = pr[0].first, cur_e = pr[0].second;
    for (int64_t i = 1; i <= 2 * m; ++i) {
      if (i < 2 * m && pr[i].first <= cur_e) {
        cur_e = std::max(cur_e, pr[i].second);
        continue;
      }
      ustart[n_iv] = cur_s;
      uoff[n_iv] = n_rows;
      ++n_iv;
      n_rows += cur_e - cur_s;
      if (i < 2 * m) {
        cur_s = pr[i].first;
        cur_e = pr[i].second;
      }
    }
  }
  auto compact = [&](int64_t row) -> int64_t {  // row lies in U
    if (dense) return row - sh.lo;
    const int64_t k = (std::upper_bound(ustart, ustart + n_iv, row) - ustart) - 1;
    return uoff[k] + (row - ustart[k]);
  };
  auto row_of = [&](int64_t c) -> int32_t {  // compact index -> pool row
    if (dense) return (int32_t)(sh.lo + c);
    const int64_t k = (std::upper_bound(uoff, uoff + n_iv, c) - uoff) - 1;
    return (int32_t)(ustart[k] + (c - uoff[k]));
  };
  // replay: prov[c] = compact index of the row whose bytes row c holds
  int32_t* prov = work;                 // [n_rows]
  int32_t* stage_of = work + n_rows;    // [n_rows]
  int32_t* gather = stage_of + n_rows;  // [2 rows]
  uint64_t* changed = (uint64_t*)(work + ((2 * n_rows + 2 * sh.rows + 1) / 2 * 2));  // [n_rows / 64]
  for (int64_t c = 0; c < n_rows; ++c) prov[c] = (int32_t)c;
  for (int64_t i = 0; i < m; ++i) {
    const Move& x = eff[order[i]];
    std::memmove(prov + compact(x.d), prov + compact(x.s), (size_t)x.len * sizeof(int32_t));
  }
  // rows read from a row that is also written go through the stage; the
  // scatter pairs go to the plan right after room for the most gather pairs
  // (2 per changed row) and the gather pairs, built apart, go in front
  const int64_t nw = (n_rows + 63) / 64;
  int64_t n_changed = 0;
  for (int64_t w = 0; w < nw; ++w) {
    uint64_t bits = 0;
    const int64_t c0 = 64 * w, c1 = std::min<int64_t>(c0 + 64, n_rows);
    for (int64_t c = c0; c < c1; ++c) bits |= (uint64_t)(prov[c] != (int32_t)c) << (c - c0);
    changed[w] = bits;
    n_changed += __builtin_popcountll(bits);
  }
  std::fill(stage_of, stage_of + n_rows, -1);
  int32_t* scatter = plan + 2 * n_changed;
  int32_t n_stage = 0, n_scatter = 0;
  // the changed rows in order, through their bits; the first read of a
  // changed source takes the next stage slot (written unconditionally, kept
  // only then, so the loop does not branch on it)
  for (int64_t w = 0; w < nw; ++w) {
    for (uint64_t bits = changed[w]; bits; bits &= bits - 1) {
      const int64_t c = 64 * w + __builtin_ctzll(bits);
      const int32_t src = prov[c];
      const int32_t ysrc = row_of(src);
      const bool staged = (changed[src >> 6] >> (src & 63)) & 1;  // the source row is overwritten too
      const int32_t slot0 = stage_of[src];
      const bool fresh = staged && slot0 < 0;
      gather[2 * n_stage] = ysrc;
      gather[2 * n_stage + 1] = n_stage;
      const int32_t slot = fresh ? n_stage : slot0;
      stage_of[src] = slot;
      n_stage += fresh ? 1 : 0;
      scatter[2 * n_scatter] = row_of(c);
      scatter[2 * n_scatter + 1] = staged ? -(slot + 1) : ysrc;
      ++n_scatter;
    }
  }
  std::memmove(plan + 2 * n_stage, scatter, (size_t)n_scatter * 2 * sizeof(int32_t));
  std::memcpy(plan, gather, (size_t)n_stage * 2 * sizeof(int32_t));
  info->kind = n_scatter ? 2 : 0;
  info->n_gather = n_stage;
  info->n_scatter = n_scatter;
  info->n_words = 2 * ((int64_t)n_stage + n_scatter);
}

pkv_status check_pools(void* k_pool, void* v_pool, int32_t n_pool_blocks, int32_t block_size,
                       int32_t n_kv_heads, int64_t seg_bytes_k, int64_t seg_bytes_v) {
  if (!k_pool) return fail(PKV_E_ARG, "k_pool is NULL");
  if (n_pool_blocks <= 0 || block_size <= 0 || n_kv_heads <= 0)
    return fail(PKV_E_ARG, "n_pool_blocks %d, block_size %d and n_kv_heads %d must be positive",
                n_pool_blocks, block_size, n_kv_heads);
  if ((int64_t)n_pool_blocks * block_size > INT32_MAX)
    return fail(PKV_E_ARG, "%lld pool rows exceed 2^31 - 1", (long long)n_pool_blocks * block_size);
  if (seg_bytes_k <= 0 || seg_bytes_k % 4)
    return fail(PKV_E_ARG, "seg_bytes_k %lld must be a positive multiple of 4", (long long)seg_bytes_k);
  if (v_pool && (seg_bytes_v <= 0 || seg_bytes_v % 4))
    return fail(PKV_E_ARG, "seg_bytes_v %lld must be a positive multiple of 4", (long long)seg_bytes_v);
  return PKV_OK;
}

pkv_status device_fail(hipError_t e, const char* what) {
  return fail(PKV_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

pkv_status pkv_order_moves(const int32_t* moves, int32_t n, int32_t* order_out, int32_t* n_out) {
  if (n < 0) return fail(PKV_E_ARG, "negative move count %d", n);
  if (n > 0 && (!moves || !order_out)) return fail(PKV_E_ARG, "moves and order_out must be non-NULL");
  if (!n_out) return fail(PKV_E_ARG, "n_out is NULL");
  std::vector<Move> eff;
  for (int32_t i = 0; i < n; ++i)
    if (moves[3 * i + 2] > 0 && moves[3 * i] != moves[3 * i + 1])
      eff.push_back({moves[3 * i], moves[3 * i + 1], moves[3 * i + 2], i});
  std::vector<int32_t> order(eff.size());
  std::vector<uint64_t> work(4 * eff.size());
  order_moves(eff.data(), (int64_t)eff.size(), order.data(), work.data());
  for (size_t i = 0; i < order.size(); ++i) order_out[i] = eff[(size_t)order[i]].idx;
  *n_out = (int32_t)order.size();
  return ok();
}

int64_t pkv_copy_cells_plan_words(const int32_t* moves, int32_t n) {
  if (n < 0 || (n > 0 && !moves)) return 0;
  return layout_of(shape_of(moves, n)).total;
}

pkv_status pkv_copy_cells_plan(const int32_t* moves, int32_t n, int64_t n_pool_rows, int32_t* plan,
                               int64_t plan_words, pkv_copy_plan* info) {
  if (!info) return fail(PKV_E_ARG, "info is NULL");
  std::memset(info, 0, sizeof *info);
  if (n < 0) return fail(PKV_E_ARG, "negative move count %d", n);
  if (n > 0 && !moves) return fail(PKV_E_ARG, "moves is NULL");
  if (n_pool_rows <= 0 || n_pool_rows > INT32_MAX)
    return fail(PKV_E_ARG, "n_pool_rows %lld outside [1, 2^31 - 1]", (long long)n_pool_rows);
  for (int32_t i = 0; i < n; ++i) {
    const int64_t s = moves[3 * i], d = moves[3 * i + 1], len = moves[3 * i + 2];
    if (len <= 0 || s == d) continue;
    if (s < 0 || d < 0 || s + len > n_pool_rows || d + len > n_pool_rows)
      return fail(PKV_E_ARG, "move %d (src %lld, dst %lld, len %lld) leaves [0, %lld)", i, (long long)s,
                  (long long)d, (long long)len, (long long)n_pool_rows);
  }
  const Shape sh = shape_of(moves, n);
  if (!sh.m) return ok();
  const Layout L = layout_of(sh);
  if (!plan) return fail(PKV_E_ARG, "plan is NULL");
  if (plan_words < L.total)
    return fail(PKV_E_WORKSPACE, "plan buffer of %lld words is smaller than the %lld needed (pkv_copy_cells_plan_words)",
                (long long)plan_words, (long long)L.total);
  Move* eff = (Move*)(plan + L.eff);
  int64_t m = 0;
  for (int32_t i = 0; i < n; ++i)
    if (moves[3 * i + 2] > 0 && moves[3 * i] != moves[3 * i + 1])
      eff[m++] = {moves[3 * i], moves[3 * i + 1], moves[3 * i + 2], i};
  int32_t* order = plan + L.order;
  int64_t* ivl = (int64_t*)(plan + L.ivl);
  uint64_t* work64 = (uint64_t*)(plan + L.work);
  if (disjoint(eff, m, sh, work64)) {
    // the moves, then the prefix sums of their lengths (the records start
    // past the plan's 4m + 1 words)
    int32_t* cum = plan + 3 * m;
    int64_t total = 0;
    cum[0] = 0;
    for (int64_t i = 0; i < m; ++i) {
      plan[3 * i] = eff[i].s;
      plan[3 * i + 1] = eff[i].d;
      plan[3 * i + 2] = eff[i].len;
      total += eff[i].len;
      cum[i + 1] = (int32_t)total;  // distinct destination rows: total <= pool rows < 2^31
    }
    info->kind = 1;
    info->n_moves = (int32_t)m;
    info->total_rows = (int32_t)total;
    info->n_words = 4 * m + 1;
    return ok();
  }
  order_moves(eff, m, order, work64);
  stage_plan(eff, m, sh, order, ivl, plan + L.work, plan, info);
  return ok();
}

size_t pkv_copy_cells_stage_bytes(const pkv_copy_plan* info, int64_t row_bytes_k, int64_t row_bytes_v) {
  if (!info || info->kind != 2 || row_bytes_k <= 0 || row_bytes_v < 0) return 0;
  return align_up((size_t)info->n_gather * (size_t)row_bytes_k, 256) +
         align_up((size_t)info->n_gather * (size_t)row_bytes_v, 256);
}

pkv_status pkv_copy_cells_apply(void* k_pool, void* v_pool, int32_t n_pool_blocks, int32_t block_size,
                                int32_t n_kv_heads, int64_t seg_bytes_k, int64_t seg_bytes_v,
                                const pkv_copy_plan* info, const int32_t* plan, void* stage,
                                size_t stage_bytes, void* stream) {
  pkv_status st = check_pools(k_pool, v_pool, n_pool_blocks, block_size, n_kv_heads, seg_bytes_k, seg_bytes_v);
  if (st) return st;
  if (!info) return fail(PKV_E_ARG, "info is NULL");
  if (info->kind == 0) return ok();
  if (info->kind != 1 && info->kind != 2) return fail(PKV_E_ARG, "unknown plan kind %d", info->kind);
  if (!plan) return fail(PKV_E_ARG, "plan is NULL");
  const int64_t n_rows = (int64_t)n_pool_blocks * block_size;
  const pkv::PoolGeom pools[2] = {
      {(unsigned char*)k_pool, seg_bytes_k, n_kv_heads, block_size, n_rows},
      {(unsigned char*)v_pool, seg_bytes_v, n_kv_heads, block_size, n_rows}};
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (info->kind == 1) {
    if (info->n_moves < 0 || info->total_rows < 0 || info->n_words < 4 * (int64_t)info->n_moves + 1)
      return fail(PKV_E_ARG, "inconsistent run plan (%d moves, %lld words)", info->n_moves,
                  (long long)info->n_words);
    for (const pkv::PoolGeom& g : pools) {
      if (!g.base) continue;
      e = pkv::launch_copy_runs(g, plan, plan + 3 * (int64_t)info->n_moves, info->n_moves, info->total_rows, s);
      if (e != hipSuccess) return device_fail(e, "copy_cells run launch");
    }
    return ok();
  }
  if (info->n_gather < 0 || info->n_scatter < 0 ||
      info->n_words < 2 * ((int64_t)info->n_gather + info->n_scatter))
    return fail(PKV_E_ARG, "inconsistent row plan (%d gathered, %d written, %lld words)", info->n_gather,
                info->n_scatter, (long long)info->n_words);
  const size_t need = pkv_copy_cells_stage_bytes(info, seg_bytes_k * n_kv_heads, v_pool ? seg_bytes_v * n_kv_heads : 0);
  if (need && (!stage || stage_bytes < need))
    return fail(PKV_E_WORKSPACE, "stage of %zu bytes is smaller than the %zu needed", stage ? stage_bytes : (size_t)0,
                need);
  if (need && ((uintptr_t)stage) % 16) return fail(PKV_E_WORKSPACE, "stage must be 16-byte aligned");
  const size_t stage_k = align_up((size_t)info->n_gather * (size_t)(seg_bytes_k * n_kv_heads), 256);
  unsigned char* stages[2] = {(unsigned char*)stage, (unsigned char*)stage + stage_k};
  const int32_t* gather = plan;
  const int32_t* scatter = plan + 2 * (int64_t)info->n_gather;
  for (int i = 0; i < 2; ++i) {
    if (!pools[i].base) continue;
    e = pkv::launch_copy_rows(1, pools[i], stages[i], info->n_gather, gather, info->n_gather, s);
    if (e != hipSuccess) return device_fail(e, "copy_cells gather launch");
  }
  for (int i = 0; i < 2; ++i) {
    if (!pools[i].base) continue;
    e = pkv::launch_copy_rows(2, pools[i], stages[i], info->n_gather, scatter, info->n_scatter, s);
    if (e != hipSuccess) return device_fail(e, "copy_cells scatter launch");
  }
  return ok();
}

size_t pkv_copy_cells_workspace_bytes(const int32_t* moves, int32_t n, int64_t row_bytes_k,
                                      int64_t row_bytes_v) {
  if (n < 0 || (n > 0 && !moves) || row_bytes_k <= 0 || row_bytes_v < 0) return 0;
  const Shape sh = shape_of(moves, n);
  if (!sh.m) return 256;
  // the uploaded plan, then (unless the moves are disjoint) a stage for at
  // most every moved row
  std::vector<Move> eff;
  for (int32_t i = 0; i < n; ++i)
    if (moves[3 * i + 2] > 0 && moves[3 * i] != moves[3 * i + 1])
      eff.push_back({moves[3 * i], moves[3 * i + 1], moves[3 * i + 2], i});
  const int64_t span = sh.hi - sh.lo;
  std::vector<uint64_t> bits(span <= ((int64_t)1 << 28) ? (size_t)((span + 63) / 64) : 0);
  if (disjoint(eff.data(), sh.m, sh, bits.data())) return align_up((size_t)(4 * sh.m + 1) * sizeof(int32_t), 256) + 256;
  const size_t plan = align_up((size_t)std::max(4 * sh.m + 1, 4 * sh.rows) * sizeof(int32_t), 256);
  return plan + align_up((size_t)sh.rows * (size_t)row_bytes_k, 256) +
         align_up((size_t)sh.rows * (size_t)row_bytes_v, 256) + 256;
}

pkv_status pkv_kv_copy_cells(void* k_pool, void* v_pool, int32_t n_pool_blocks, int32_t block_size,
                             int32_t n_kv_heads, int64_t seg_bytes_k, int64_t seg_bytes_v,
                             const int32_t* moves, int32_t n, void* ws, size_t ws_bytes, void* stream) {
  pkv_status st = check_pools(k_pool, v_pool, n_pool_blocks, block_size, n_kv_heads, seg_bytes_k, seg_bytes_v);
  if (st) return st;
  if (n < 0) return fail(PKV_E_ARG, "negative move count %d", n);
  if (n > 0 && !moves) return fail(PKV_E_ARG, "moves is NULL");
  const int64_t words = pkv_copy_cells_plan_words(moves, n);
  std::vector<int32_t> plan((size_t)std::max<int64_t>(words, 1));
  pkv_copy_plan info;
  st = pkv_copy_cells_plan(moves, n, (int64_t)n_pool_blocks * block_size, plan.data(), words, &info);
  if (st) return st;
  if (info.kind == 0) return ok();
  const size_t plan_bytes = align_up((size_t)info.n_words * sizeof(int32_t), 256);
  const size_t stage = pkv_copy_cells_stage_bytes(&info, seg_bytes_k * n_kv_heads, v_pool ? seg_bytes_v * n_kv_heads : 0);
  if (!ws || ws_bytes < plan_bytes + stage)
    return fail(PKV_E_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed", ws ? ws_bytes : (size_t)0,
                plan_bytes + stage);
  if (((uintptr_t)ws) % 256) return fail(PKV_E_WORKSPACE, "workspace must be 256-byte aligned");
  // the plan lives in this call's memory: wait until it has been copied
  hipError_t e = hipMemcpyAsync(ws, plan.data(), (size_t)info.n_words * sizeof(int32_t), hipMemcpyHostToDevice,
                                (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return device_fail(e, "uploading the copy_cells plan");
  return pkv_copy_cells_apply(k_pool, v_pool, n_pool_blocks, block_size, n_kv_heads, seg_bytes_k, seg_bytes_v, &info,
                              (const int32_t*)ws, (char*)ws + plan_bytes, ws_bytes - plan_bytes, stream);
}

}  // extern "C"
