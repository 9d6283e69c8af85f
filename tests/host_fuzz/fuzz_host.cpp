// Randomized host test of the copy planner and the block pool, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code.
//
// Copy planner: random move lists (overlapping slides, zero lengths, moves
// onto themselves) are planned into a buffer of exactly
// pkv_copy_cells_plan_words words; the plan, replayed on an index array as
// the device would apply it, must equal the moves applied one by one as
// memmoves in pkv_order_moves order ("KV Cache Design — cells, format,
// sessions", section 2: upward moves first, top-down, then downward ones,
// bottom-up).
// Block pool: random forks, removals, writes and defrags, with exactly
// sized output buffers; after each export every block's reference count
// must equal the number of table entries that name it.
// The device launches of copy_plan.cpp are stubbed out (never reached:
// nothing here applies a plan).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>
#include <algorithm>
#include "pkv.h"
#include "pkv_internal.hpp"
namespace pkv_host { void set_error(const char*) {} }
namespace pkv {

hipError_t launch_copy_rows(int, const PoolGeom&, unsigned char*, int, const int*, int, hipStream_t) { return hipSuccess; }
hipError_t launch_copy_runs(const PoolGeom&, const int*, const int*, int, int, hipStream_t) { return hipSuccess; }
}
static std::mt19937_64 R(12345);  // fixed seed: the same cases every run
static int rnd(int n) { return (int)(R() % (uint64_t)n); }

// naive model: apply effective moves in order_moves order as memmoves on an index array
static void check_plan(int iter) {
  const int rows = 1 + rnd(3000);
  const int n = rnd(60);
  std::vector<int32_t> mv(3 * (size_t)n);
  for (int i = 0; i < n; ++i) {
    int len = rnd(4) == 0 ? 0 : 1 + rnd(40);
    int src = rnd(rows), dst = rnd(rows);
    if (rnd(3) == 0) dst = src + rnd(9) - 4;
    if (src + len > rows) len = rows - src;
    if (dst < 0) dst = 0;
    if (dst + len > rows) len = std::max(0, rows - dst);
    mv[3 * i] = src; mv[3 * i + 1] = dst; mv[3 * i + 2] = len;
  }
  // order
  std::vector<int32_t> order((size_t)std::max(n, 1));
  int32_t no = 0;
  if (pkv_order_moves(n ? mv.data() : nullptr, n, order.data(), &no) != PKV_OK) { printf("order refused %d\n", iter); exit(1); }
  std::vector<int32_t> ref(rows);
  for (int r = 0; r < rows; ++r) ref[r] = r;
  for (int k = 0; k < no; ++k) {
    const int i = order[k];
    memmove(&ref[mv[3 * i + 1]], &ref[mv[3 * i]], sizeof(int32_t) * mv[3 * i + 2]);
  }
  const int64_t words = pkv_copy_cells_plan_words(n ? mv.data() : nullptr, n);
  if (words <= 0) {  // nothing to move: the model must be the identity
    for (int r = 0; r < rows; ++r) if (ref[r] != r) { printf("words 0 but rows move %d\n", iter); exit(1); }
    return;
  }
  int32_t* plan = (int32_t*)aligned_alloc(8, (size_t)((words * 4 + 7) / 8 * 8));
  pkv_copy_plan info;
  if (pkv_copy_cells_plan(mv.data(), n, rows, plan, words, &info) != PKV_OK) { printf("plan refused %d\n", iter); exit(1); }
  std::vector<int32_t> got(rows);
  for (int r = 0; r < rows; ++r) got[r] = r;
  if (info.kind == 1) {
    std::vector<int32_t> src0 = got;
    for (int i = 0; i < info.n_moves; ++i) {
      const int32_t s = plan[3 * i], d = plan[3 * i + 1], l = plan[3 * i + 2];
      for (int j = 0; j < l; ++j) got[d + j] = src0[s + j];
    }
  } else if (info.kind == 2) {
    std::vector<int32_t> stage(info.n_gather);
    const int32_t* g = plan;
    const int32_t* sc = plan + 2 * (int64_t)info.n_gather;
    for (int i = 0; i < info.n_gather; ++i) stage[g[2 * i + 1]] = got[g[2 * i]];
    std::vector<int32_t> src0 = got;
    for (int i = 0; i < info.n_scatter; ++i) {
      const int32_t row = sc[2 * i], s = sc[2 * i + 1];
      got[row] = s >= 0 ? src0[s] : stage[-s - 1];
    }
  }
  for (int r = 0; r < rows; ++r)
    if (got[r] != ref[r]) { printf("plan mismatch iter %d kind %d row %d\n", iter, info.kind, r); exit(1); }
  free(plan);
}

static void fuzz_pool(int iter) {
  const int nb = 8 + rnd(200), ns = 1 + rnd(20), mb = 1 + rnd(16), bs = rnd(2) ? 16 : 32;
  pkv_block_pool* p = nullptr;
  if (pkv_pool_create(nb, ns, mb, bs, rnd(3), &p) != PKV_OK) { printf("create failed\n"); exit(1); }
  for (int step = 0; step < 200; ++step) {
    const int op = rnd(5);
    if (op == 0) {
      const int n = rnd(8);
      std::vector<int32_t> s(n), p0(n), c(n);
      for (int i = 0; i < n; ++i) {
        s[i] = rnd(ns + 1) - (rnd(20) == 0);
        int len = pkv_pool_seq_len(p, std::max(0, std::min(s[i], ns - 1)));
        p0[i] = rnd(3) ? len : rnd(len + 2);
        c[i] = rnd(3 * bs);
      }
      int32_t cap = 0;
      for (int i = 0; i < n; ++i) cap += std::max(0, c[i]) / bs + 2;
      std::vector<int32_t> ops(3 * (size_t)std::max(cap, 1));
      int32_t nops = 0;
      pkv_pool_prepare_writes(p, n, n ? s.data() : nullptr, n ? p0.data() : nullptr, n ? c.data() : nullptr, ops.data(), cap, &nops);
    } else if (op == 1) {
      pkv_pool_fork(p, rnd(ns + 1) - 1, rnd(ns), rnd(4 * bs * mb));
    } else if (op == 2) {
      const int s = rnd(ns), len = pkv_pool_seq_len(p, s);
      const int a = rnd(len + 1);
      pkv_pool_remove(p, s, a, a + rnd(len + 2));
    } else if (op == 3) {
      const int cap = std::max(1, nb - pkv_pool_free_blocks(p));
      std::vector<int32_t> mvs(3 * (size_t)cap * 2);
      int32_t nm = 0;
      pkv_pool_defrag(p, rnd(3) ? -1 : rnd(nb), mvs.data(), cap * 2, &nm);
    } else {
      std::vector<int32_t> t((size_t)ns * mb), l(ns);
      pkv_pool_export(p, t.data(), l.data());
      // invariant: refcounts equal the number of table entries naming each block
      std::vector<int> cnt(nb, 0);
      for (int32_t b : t) if (b >= 0) { if (b >= nb) { printf("bad block\n"); exit(1); } ++cnt[b]; }
      for (int b = 0; b < nb; ++b)
        if (cnt[b] != pkv_pool_refcount(p, b)) { printf("refcount mismatch iter %d block %d: %d vs %d\n", iter, b, cnt[b], pkv_pool_refcount(p, b)); exit(1); }
    }
  }
  pkv_pool_destroy(p);
}

int main(int argc, char** argv) {
  const int n_plan = argc > 1 ? atoi(argv[1]) : 20000, n_pool = argc > 2 ? atoi(argv[2]) : 2000;
  for (int i = 0; i < n_plan; ++i) check_plan(i);
  printf("copy plan: %d cases ok\n", n_plan);
  for (int i = 0; i < n_pool; ++i) fuzz_pool(i);
  printf("pool: %d histories ok\n", n_pool);
  return 0;
}
