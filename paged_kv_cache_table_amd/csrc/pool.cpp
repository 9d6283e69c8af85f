// Copy-on-write block pool: host-side bookkeeping of physical blocks shared
// by forked sequences.
//
// "Tiered KV cache — architecture", section "The paged-attention block
// model": forking only raises per-block reference counts and copies the
// table (no K/V bytes move until a fork writes); a partial removal wipes
// whole logical blocks by setting their entries to the sentinel.  Its file
// list names the physical allocator with reference counts and a watermark.
// "KV Cache Design — cells, format, sessions", sections 1 and 2: a store may
// never land in a prefix another sequence reads in place, so the shared
// block is copied before the first write resolves its row.
//
// Semantics (the same readings as the oracle model):
//  - allocation takes the free block with the smallest id; a block is free
//    exactly when its reference count is 0;
//  - fork(src, dst, n): dst empty; takes src's first ceil(n / bs) entries,
//    each named block gains a reference;
//  - remove(s, p0, p1): clipped to [0, len); reaching the end truncates to
//    p0 and releases every block starting at or after p0; otherwise blocks
//    wholly inside become holes;
//  - prepare_writes: for each write [p0, p0 + n) (p0 <= len) and each
//    logical block it touches, in order: a block the sequence owns alone is
//    written in place, a shared block is copied into a fresh one (returned
//    as a (src, dst) pair for the device), an empty entry gets a fresh
//    block; the length becomes max(len, p0 + n).  Checked in full before
//    any change.  Every table entry it changes is reported as an op
//    (source block or -1, fresh block, entry index) for the device, which
//    copies the source block (if any) and patches its copy of the table;
//  - defrag(need): the live blocks in the top `need` ids, ascending, move
//    into the lowest free blocks, ascending (need < 0: every free block);
//    tables and counts follow; the row moves (consecutive blocks landing on
//    consecutive blocks merged) go to copy_cells.  Every move goes down
//    onto a free row, so no destination is ever a source.
//
// The free set is a two-level bitmap (one bit per block, one bit per 64-bit
// word), so the smallest free id is found in a few word scans.
#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "pkv.h"

namespace pkv_host {
void set_error(const char* msg);  // host.cpp: the message pkv_last_error returns
}

struct pkv_block_pool {
  int32_t n_blocks = 0, n_seqs = 0, max_blocks = 0, bs = 0, watermark = 0;
  int32_t n_free = 0;
  std::vector<int32_t> ref;     // [n_blocks]
  std::vector<int32_t> table;   // [n_seqs][max_blocks], PKV_INVALID_BLOCK_ID when empty
  std::vector<int32_t> length;  // [n_seqs]
  std::vector<uint64_t> l0;     // bit b: block b is free
  std::vector<uint64_t> l1;     // bit w: l0[w] != 0
  size_t l1_lo = 0;             // no l1 word below this index has a bit set
  // Scratch of prepare_writes' checking pass, valid where the stamp equals
  // the call's generation (so nothing is cleared between calls).
  uint32_t gen = 0;
  std::vector<uint32_t> seq_stamp, blk_stamp;
  std::vector<int32_t> seq_len, blk_refs, seq_priv;  // length / live refs / head of private list
  std::vector<int32_t> priv_lb, priv_next;          // private (seq, lb) marks, per-sequence lists

  int32_t* row(int32_t s) { return table.data() + (size_t)s * max_blocks; }

  void mark_free(int32_t b) {
    l0[b >> 6] |= 1ull << (b & 63);
    l1[b >> 12] |= 1ull << ((b >> 6) & 63);
    l1_lo = std::min(l1_lo, (size_t)(b >> 12));
    ++n_free;
  }
  int32_t take_smallest() {
    for (size_t w1 = l1_lo; w1 < l1.size(); ++w1) {
      if (!l1[w1]) {
        l1_lo = w1 + 1;
        continue;
      }
      const size_t w0 = w1 * 64 + __builtin_ctzll(l1[w1]);
      const int32_t b = (int32_t)(w0 * 64 + __builtin_ctzll(l0[w0]));
      l0[w0] &= l0[w0] - 1;
      if (!l0[w0]) l1[w1] &= ~(1ull << (w0 & 63));
      --n_free;
      ref[b] = 1;
      return b;
    }
    return -1;
  }
  void release(int32_t b) {
    if (--ref[b] == 0) mark_free(b);
  }
  bool is_free(int32_t b) const { return (l0[b >> 6] >> (b & 63)) & 1; }
  void take(int32_t b) {  // a specific free block
    l0[b >> 6] &= ~(1ull << (b & 63));
    if (!l0[b >> 6]) l1[b >> 12] &= ~(1ull << ((b >> 6) & 63));
    --n_free;
  }
  int32_t nblk(int64_t n_tokens) const { return (int32_t)((n_tokens + bs - 1) / bs); }
  void next_gen() {
    if (++gen == 0) {  // wrapped: reset every stamp once
      std::fill(seq_stamp.begin(), seq_stamp.end(), 0);
      std::fill(blk_stamp.begin(), blk_stamp.end(), 0);
      gen = 1;
    }
    priv_lb.clear();
    priv_next.clear();
  }
  // Checking-pass views of a sequence's length, a block's references and
  // whether (seq, lb) was already made private earlier in the batch.
  int32_t len_of(int32_t s) const { return seq_stamp[s] == gen ? seq_len[s] : length[s]; }
  int32_t refs_of(int32_t b) const { return blk_stamp[b] == gen ? blk_refs[b] : ref[b]; }
  void touch_seq(int32_t s) {
    if (seq_stamp[s] != gen) {
      seq_stamp[s] = gen;
      seq_len[s] = length[s];
      seq_priv[s] = -1;
    }
  }
  bool is_private(int32_t s, int32_t lb) const {
    if (seq_stamp[s] != gen) return false;
    for (int32_t i = seq_priv[s]; i >= 0; i = priv_next[i])
      if (priv_lb[i] == lb) return true;
    return false;
  }
  void mark_private(int32_t s, int32_t lb) {
    priv_lb.push_back(lb);
    priv_next.push_back(seq_priv[s]);
    seq_priv[s] = (int32_t)priv_lb.size() - 1;
  }
  void drop_ref(int32_t b) {
    if (blk_stamp[b] != gen) {
      blk_stamp[b] = gen;
      blk_refs[b] = ref[b];
    }
    --blk_refs[b];
  }
};

namespace {

pkv_status perr(pkv_status st, const char* msg) {
  pkv_host::set_error(msg);
  return st;
}

pkv_status pok() {
  pkv_host::set_error("");
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_pool_create(int32_t n_blocks, int32_t n_seqs, int32_t max_blocks_per_seq,
                           int32_t block_size, int32_t watermark, pkv_block_pool** out) {
  if (!out) return perr(PKV_E_ARG, "out is NULL");
  *out = nullptr;
  if (n_blocks <= 0 || n_seqs <= 0 || max_blocks_per_seq <= 0 || block_size <= 0 || watermark < 0)
    return perr(PKV_E_ARG, "pool sizes must be positive and the watermark non-negative");
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX ||
      (int64_t)n_seqs * max_blocks_per_seq > INT32_MAX || (int64_t)n_blocks * block_size > INT32_MAX)
    return perr(PKV_E_ARG, "pool geometry too large");
  pkv_block_pool* p = new (std::nothrow) pkv_block_pool;
  if (!p) return perr(PKV_E_ARG, "out of host memory");
  try {
    p->n_blocks = n_blocks;
    p->n_seqs = n_seqs;
    p->max_blocks = max_blocks_per_seq;
    p->bs = block_size;
    p->watermark = watermark;
    p->ref.assign(n_blocks, 0);
    p->table.assign((size_t)n_seqs * max_blocks_per_seq, PKV_INVALID_BLOCK_ID);
    p->length.assign(n_seqs, 0);
    p->l0.assign(((size_t)n_blocks + 63) / 64, 0);
    p->l1.assign((p->l0.size() + 63) / 64, 0);
    p->seq_stamp.assign(n_seqs, 0);
    p->seq_len.assign(n_seqs, 0);
    p->seq_priv.assign(n_seqs, -1);
    p->blk_stamp.assign(n_blocks, 0);
    p->blk_refs.assign(n_blocks, 0);
  } catch (...) {
    delete p;
    return perr(PKV_E_ARG, "out of host memory");
  }
  for (int32_t b = 0; b < n_blocks; ++b) p->mark_free(b);
  *out = p;
  return pok();
}

void pkv_pool_destroy(pkv_block_pool* pool) { delete pool; }

int32_t pkv_pool_free_blocks(const pkv_block_pool* p) { return p ? p->n_free : -1; }

int32_t pkv_pool_can_allocate(const pkv_block_pool* p, int32_t n) {
  return p && n >= 0 && (int64_t)p->n_free - n >= p->watermark ? 1 : 0;
}

int32_t pkv_pool_refcount(const pkv_block_pool* p, int32_t block) {
  return p && block >= 0 && block < p->n_blocks ? p->ref[block] : -1;
}

int32_t pkv_pool_seq_len(const pkv_block_pool* p, int32_t seq) {
  return p && seq >= 0 && seq < p->n_seqs ? p->length[seq] : -1;
}

pkv_status pkv_pool_fork(pkv_block_pool* p, int32_t src, int32_t dst, int32_t n_tokens) {
  if (!p) return perr(PKV_E_ARG, "pool is NULL");
  if (src < 0 || src >= p->n_seqs || dst < 0 || dst >= p->n_seqs || src == dst)
    return perr(PKV_E_ARG, "fork needs two distinct sequences of the pool");
  const int32_t n = n_tokens < 0 ? p->length[src] : n_tokens;
  if (n > p->length[src]) return perr(PKV_E_ARG, "fork length exceeds the source sequence");
  int32_t* d = p->row(dst);
  if (p->length[dst] != 0 ||
      std::any_of(d, d + p->max_blocks, [](int32_t b) { return b != PKV_INVALID_BLOCK_ID; }))
    return perr(PKV_E_ARG, "fork destination is not empty");
  const int32_t* s = p->row(src);
  for (int32_t lb = 0, nb = p->nblk(n); lb < nb; ++lb) {
    d[lb] = s[lb];
    if (s[lb] != PKV_INVALID_BLOCK_ID) ++p->ref[s[lb]];
  }
  p->length[dst] = n;
  return pok();
}

pkv_status pkv_pool_remove(pkv_block_pool* p, int32_t seq, int32_t p0, int32_t p1) {
  if (!p) return perr(PKV_E_ARG, "pool is NULL");
  if (seq < 0 || seq >= p->n_seqs) return perr(PKV_E_ARG, "sequence outside the pool");
  const int32_t L = p->length[seq];
  p0 = std::max(p0, 0);
  p1 = std::min(p1, L);
  if (p0 >= p1) return pok();
  const int32_t first = p->nblk(p0);  // first logical block starting at or after p0
  int32_t last;                       // blocks [first, last) are released
  if (p1 == L) {
    last = p->max_blocks;
    p->length[seq] = p0;
  } else {
    last = p1 / p->bs;
  }
  int32_t* r = p->row(seq);
  for (int32_t lb = first; lb < last; ++lb) {
    if (r[lb] == PKV_INVALID_BLOCK_ID) continue;
    p->release(r[lb]);
    r[lb] = PKV_INVALID_BLOCK_ID;
  }
  return pok();
}

pkv_status pkv_pool_prepare_writes(pkv_block_pool* p, int32_t n, const int32_t* seqs,
                                   const int32_t* p0s, const int32_t* counts, int32_t* ops_out,
                                   int32_t max_ops, int32_t* n_ops) {
  if (!p || n < 0 || (n > 0 && (!seqs || !p0s || !counts)) || !n_ops)
    return perr(PKV_E_ARG, "NULL pool, array or n_ops, or a negative count");
  *n_ops = 0;
  // Pass 1: check every write against the state the earlier writes of the
  // batch leave, and count the fresh blocks and copies needed.
  p->next_gen();
  int64_t fresh = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seqs[i], a = p0s[i], c = counts[i];
    if (c <= 0) continue;
    if (s < 0 || s >= p->n_seqs) return perr(PKV_E_ARG, "write to a sequence outside the pool");
    if (a < 0 || a > p->len_of(s)) return perr(PKV_E_ARG, "write leaves a gap before its first position");
    if ((int64_t)a + c > (int64_t)p->max_blocks * p->bs)
      return perr(PKV_E_ARG, "write runs past the sequence's table");
    p->touch_seq(s);
    const int32_t* r = p->row(s);
    for (int32_t lb = a / p->bs, le = (a + c - 1) / p->bs; lb <= le; ++lb) {
      if (p->is_private(s, lb)) continue;
      const int32_t b = r[lb];
      if (b == PKV_INVALID_BLOCK_ID) {
        ++fresh;
      } else if (p->refs_of(b) > 1) {
        ++fresh;
        p->drop_ref(b);
      } else {
        continue;
      }
      p->mark_private(s, lb);
    }
    p->seq_len[s] = std::max(p->seq_len[s], a + c);
  }
  if (fresh > p->n_free) return perr(PKV_E_CAPACITY, "pool has too few free blocks for these writes");
  if (fresh > 0 && (!ops_out || fresh > max_ops))
    return perr(PKV_E_WORKSPACE, "ops_out is too small for the table changes these writes make");
  // Pass 2: apply, in the same order with the same decisions.
  int32_t k = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t s = seqs[i], a = p0s[i], c = counts[i];
    if (c <= 0) continue;
    int32_t* r = p->row(s);
    for (int32_t lb = a / p->bs, le = (a + c - 1) / p->bs; lb <= le; ++lb) {
      const int32_t b = r[lb];
      int32_t src;
      if (b == PKV_INVALID_BLOCK_ID) {
        src = -1;
      } else if (p->ref[b] > 1) {
        src = b;
        --p->ref[b];
      } else {
        continue;
      }
      r[lb] = p->take_smallest();
      ops_out[3 * k] = src;
      ops_out[3 * k + 1] = r[lb];
      ops_out[3 * k + 2] = s * p->max_blocks + lb;
      ++k;
    }
    p->length[s] = std::max(p->length[s], a + c);
  }
  *n_ops = k;
  return pok();
}

pkv_status pkv_pool_defrag(pkv_block_pool* p, int32_t need, int32_t* moves_out, int32_t max_moves,
                           int32_t* n_moves) {
  if (!p || !n_moves) return perr(PKV_E_ARG, "pool or n_moves is NULL");
  *n_moves = 0;
  if (need < 0) need = p->n_free;
  if (need > p->n_free) return perr(PKV_E_CAPACITY, "fewer free blocks than the defrag needs");
  const int32_t top = p->n_blocks - need;
  std::vector<int32_t> srcs, holes;
  for (int32_t b = top; b < p->n_blocks; ++b)
    if (p->ref[b] > 0) srcs.push_back(b);
  for (int32_t b = 0; b < top && holes.size() < srcs.size(); ++b)
    if (p->ref[b] == 0) holes.push_back(b);
  // Count the merged row moves before changing anything.
  int32_t nm = 0;
  for (size_t i = 0; i < srcs.size(); ++i)
    if (i == 0 || srcs[i] != srcs[i - 1] + 1 || holes[i] != holes[i - 1] + 1) ++nm;
  if (nm > 0 && (!moves_out || nm > max_moves))
    return perr(PKV_E_WORKSPACE, "moves_out is too small for the moves this defrag makes");
  if (srcs.empty()) return pok();
  std::vector<int32_t> where(p->n_blocks - top, -1);
  for (size_t i = 0; i < srcs.size(); ++i) where[srcs[i] - top] = holes[i];
  for (int32_t& e : p->table)
    if (e >= top) e = where[e - top];
  int32_t k = -1;
  const int64_t bs = p->bs;
  for (size_t i = 0; i < srcs.size(); ++i) {
    const int32_t a = srcs[i], d = holes[i];
    p->ref[d] = p->ref[a];
    p->ref[a] = 0;
    p->take(d);
    p->mark_free(a);
    if (i > 0 && a == srcs[i - 1] + 1 && d == holes[i - 1] + 1) {
      moves_out[3 * k + 2] += (int32_t)bs;
    } else {
      ++k;
      moves_out[3 * k] = (int32_t)(a * bs);
      moves_out[3 * k + 1] = (int32_t)(d * bs);
      moves_out[3 * k + 2] = (int32_t)bs;
    }
  }
  *n_moves = k + 1;
  return pok();
}

pkv_status pkv_pool_export(const pkv_block_pool* p, int32_t* table_out, int32_t* lens_out) {
  if (!p || !table_out) return perr(PKV_E_ARG, "pool or table_out is NULL");
  std::memcpy(table_out, p->table.data(), p->table.size() * sizeof(int32_t));
  if (lens_out) std::memcpy(lens_out, p->length.data(), p->length.size() * sizeof(int32_t));
  return pok();
}

}  // extern "C"
