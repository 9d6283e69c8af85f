/*
 * pkv — grouped-query attention read through a paged KV cache, for AMD
 * Instinct MI355X (gfx950).  C ABI: plain pointers, sizes and status codes.
 *
 * Model of the cache ("Tiered KV cache — architecture", section "The
 * paged-attention block model"): tokens are stored in fixed-size physical
 * blocks; a per-sequence logical->physical block table says which block
 * holds which range of positions; an entry equal to PKV_INVALID_BLOCK_ID is
 * a hole whose positions score -infinity, i.e. do not exist (also section
 * "Kernel dispatch").  A block is block_size tokens x n_kv_heads x head_dim
 * of K and of V (section "The three-tier model").
 *
 * Windows ("KV Cache Design — cells, format, sessions", section 1
 * "Positions and cells"): causal positions, one [lo, hi) range per
 * sequence, or a map of up to PKV_KV_MAP_MAX_SPANS (cell, len) runs, read
 * in place, so a copy-on-write prefix shared by several sequences is read
 * through identical block ids without copies.
 *
 * Conventions for every call:
 *  - Device pointers are HIP device memory owned by the caller.  The library
 *    never allocates device memory and keeps no pointer after a call
 *    returns; scratch comes in through a caller-owned workspace whose size
 *    the matching *_workspace_bytes call returns.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL is the default
 *    stream) unless stated; inputs must stay alive until the stream passes.
 *  - Every argument the host can check is checked before anything is
 *    launched, so a refused call writes nothing ("KV Cache Design", section
 *    4: verify before apply).  Refusals return a status code and set a
 *    message readable with pkv_last_error() (per thread).  The library never
 *    aborts the process.
 *  - Device-resident integers (block ids, lengths, windows, positions) are
 *    not read back.  They are clamped where they are used: a window outside
 *    [0, seq_len) is clipped, seq_len is clipped to max_blocks_per_seq *
 *    block_size, and a block id outside [-1, n_pool_blocks) is treated as a
 *    hole, so no input makes a kernel read or write outside its buffers.
 *    With PKV_FLAG_CHECKED such ids are also reported: the call then waits
 *    for the stream and returns PKV_E_ARG.
 *  - No internal locking ("Tiered KV cache — architecture", section "The
 *    single-threading contract"): one caller mutates a pool at a time;
 *    calls on one stream are ordered.
 *  - Graph capture: the decode calls, pkv_paged_attn_prefill_window,
 *    pkv_kv_store, pkv_cow_apply, pkv_copy_cells_apply and the int4 codec
 *    only launch kernels on `stream` (no synchronization, allocation or
 *    memset), so they can be captured into a HIP graph and replayed.  With
 *    PKV_FLAG_CHECKED they wait for the stream and cannot; pkv_kv_copy_cells
 *    uploads its plan from the host, so it cannot either.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Sentinel for a wiped logical block (a hole). */
#define PKV_INVALID_BLOCK_ID (-1)
/* Most (cell, len) runs one kv_map window may hold. */
#define PKV_KV_MAP_MAX_SPANS 8
/* pkv_shape.flags: validate device ids and report bad ones (slow: syncs). */
#define PKV_FLAG_CHECKED 1u

typedef enum {
  PKV_OK = 0,
  PKV_E_ARG = 1,         /* malformed argument (null, negative, mismatch) */
  PKV_E_UNSUPPORTED = 2, /* well formed but outside the dispatch table   */
  PKV_E_WORKSPACE = 3,   /* workspace missing or too small                */
  PKV_E_DEVICE = 4,      /* a HIP call failed                             */
  PKV_E_CAPACITY = 5     /* the block pool has too few free blocks        */
} pkv_status;

/* KV storage formats ("KV Cache Design", section 3: f32, f16, q8_0). */
typedef enum { PKV_F32 = 0, PKV_F16 = 1, PKV_Q8_0 = 2 } pkv_fmt;

/* Window modes; the mode fixes the shape of the window input. */
typedef enum {
  PKV_WIN_CAUSAL = 0, /* window = NULL: positions [0, seq_len)                */
  PKV_WIN_SPAN = 1,   /* window = int32 [n_seqs][2] = (lo, hi)                */
  PKV_WIN_KV_MAP = 2  /* window = int32 [n_seqs][n_runs][2] = (cell, len);
                         len <= 0 marks an unused run; runs may overlap and a
                         position listed twice counts twice                   */
} pkv_win;

/*
 * Geometry of one attention call.
 *
 * Pools: k_pool and v_pool are [n_pool_blocks][n_kv_heads][block_size][seg]:
 * inside a block, each kv head's block_size token entries are contiguous.
 * seg is one token of one kv head: head_dim values for f32/f16, or for q8_0
 * head_dim/32 blocks of a little-endian f16 scale followed by 32 int8 codes
 * (value = scale * code), rounded up to whole 4-byte words.  Pool row
 * (token cell) r = block * block_size + slot is that slot of every kv head.
 * block_table: int32 [n_seqs][max_blocks_per_seq].  seq_lens: int32
 * [n_seqs].  q head h reads kv head h / (n_q_heads / n_kv_heads).
 * Scores are scale * q.k.
 *
 * Supported ("Tiered KV cache — architecture", sections "The
 * paged-attention block model" and "Kernel dispatch"): (head_dim,
 * block_size) in {(64,16), (128,16), (256,16), (128,32)}; n_q_heads /
 * n_kv_heads in {1, 2, 3, 4, 8}; (q, K, V) formats in {(f32, f32, f32),
 * (f16, f16, f16), (f16, q8_0, f16), (f32, q8_0, f32)}.  Anything else is
 * refused with PKV_E_UNSUPPORTED and a message naming the tuple.
 */
typedef struct {
  int32_t n_seqs;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t n_pool_blocks;
  int32_t max_blocks_per_seq;
  int32_t q_fmt; /* pkv_fmt: PKV_F32 or PKV_F16 */
  int32_t k_fmt; /* pkv_fmt */
  int32_t v_fmt; /* pkv_fmt: PKV_F32 or PKV_F16 */
  float scale;
  uint32_t flags;       /* PKV_FLAG_* */
  int32_t split_tokens; /* decode split size in tokens; 0 = automatic; else a
                           multiple of block_size, at most 64 blocks */
} pkv_shape;

/* Bytes of one pool row (one token cell: all kv heads) in format fmt, i.e.
 * n_kv_heads segments; 0 when the arguments are invalid.  A q8_0 segment is
 * rounded up to whole 4-byte words ("KV Cache Design", section 3). */
int64_t pkv_row_bytes(int32_t fmt, int32_t n_kv_heads, int32_t head_dim);

/* ---------------------------------------------------------------------------
 * Decode: one query per sequence, at position seq_len - 1, seeing
 * W_s intersected with [0, seq_len) minus holes ("KV cache" (sipllm),
 * section "Problem": a decode step dots the new query against the stored
 * history).  Split-K: each (sequence, kv head, split of the window) is a
 * separate work item producing (max, sum, unnormalised output); a second
 * pass merges the splits by log-sum-exp.  Calls with many possible items
 * first list the non-empty ones on the device (a one-workgroup plan pass)
 * and cut each sequence's last few full splits into shorter pieces, so the
 * split pass ends on short items.  The split size depends only on the
 * shape, and which splits are cut only on the shape and the sequence's own
 * length and window, so results are deterministic, do not depend on the
 * other sequences' lengths, and do not change when blocks move in the pool
 * and the table follows.
 *
 * q:   [n_seqs][n_q_heads][head_dim] in q_fmt.
 * out: float32 [n_seqs][n_q_heads][head_dim] = sum_t w_t v_t / sum_t w_t.
 * lse: float32 [n_seqs][n_q_heads] natural-log log-sum-exp of the scores,
 *      or NULL.  An empty visible set gives out = 0 and lse = -inf.
 * workspace: device, at least pkv_decode_workspace_bytes(...) bytes, 256-byte
 *      aligned; its contents need no initialisation.
 * ------------------------------------------------------------------------- */
size_t pkv_decode_workspace_bytes(const pkv_shape* shape, int32_t mode, int32_t n_runs);

/* Split size in tokens that a decode call with this shape uses (0 if the
 * shape is refused). */
int32_t pkv_decode_split_tokens(const pkv_shape* shape, int32_t mode, int32_t n_runs);

pkv_status pkv_paged_attn_decode(const pkv_shape* shape, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_table,
                                 const int32_t* seq_lens, int32_t mode, int32_t n_runs,
                                 const int32_t* window, float* out, float* lse, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* The two passes of pkv_paged_attn_decode as separate calls (same arguments;
 * the partials live in the workspace between them).  Lets a caller time or
 * overlap the passes; partials followed by merge equals the fused call. */
pkv_status pkv_paged_attn_decode_partials(const pkv_shape* shape, const void* q,
                                          const void* k_pool, const void* v_pool,
                                          const int32_t* block_table, const int32_t* seq_lens,
                                          int32_t mode, int32_t n_runs, const int32_t* window,
                                          void* workspace, size_t workspace_bytes, void* stream);

pkv_status pkv_paged_attn_decode_merge(const pkv_shape* shape, const int32_t* seq_lens,
                                       int32_t mode, int32_t n_runs, const int32_t* window,
                                       float* out, float* lse, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Decode without a caller workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and refusals as
 * pkv_paged_attn_decode; the workspace is a built-in device array of
 * PKV_NOALLOC_SCRATCH_BYTES bytes (each GPU holds its own copy from the
 * library's first use until the process ends; its address is looked up on
 * the first call on each device).  The call allocates nothing.  A call whose
 * pkv_decode_workspace_bytes exceeds the array is refused with
 * PKV_E_WORKSPACE before anything is launched (the 7B-class batch of 64
 * sequences of up to 32,768 tokens, 32/8 heads, head_dim 128, needs ~41 MB).
 * Every call on one GPU uses that GPU's one array: calls that overlap on one
 * GPU (two streams, or two threads) race on it and give undefined results;
 * calls ordered on one stream are safe.  The array needs no clearing between
 * calls (the decode passes write everything they read).
 * ------------------------------------------------------------------------- */
#define PKV_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

pkv_status pkv_paged_attn_decode_noalloc(const pkv_shape* shape, const void* q, const void* k_pool,
                                         const void* v_pool, const int32_t* block_table,
                                         const int32_t* seq_lens, int32_t mode, int32_t n_runs,
                                         const int32_t* window, float* out, float* lse, void* stream);

/* ---------------------------------------------------------------------------
 * Windowed prefill: a chunk of queries per sequence against its window,
 * causal inside the window ("KV Cache Design", section 1: the fast windowed
 * prefill families for more than one query, in _f32 and _f16 variants).
 * Query j of sequence s sees W_s intersected with
 * [0, min(seq_len_s, q_pos_j + 1)) minus holes.  f16 queries (K f16 or
 * q8_0, V f16): QK^T and PV run on the matrix cores (probabilities rounded
 * to f16 for PV).  f32 queries (K f32 or q8_0, V f32): every product and
 * sum stays in f32, computed by the decode kernels with each query as its
 * own decode sequence (its sequence's table and window, length
 * min(seq_len_s, q_pos_j + 1)); then n_q_total may be at most 65535.
 *
 * n_q_total: rows of q.  cu_q: int32 [n_seqs + 1], queries of sequence s are
 * rows cu_q[s] .. cu_q[s+1]-1 (non-decreasing, cu_q[0] = 0, cu_q[n_seqs] =
 * n_q_total; rows outside are left untouched).  max_q_per_seq: an upper
 * bound on cu_q[s+1] - cu_q[s] (queries past it are not computed).
 * q_pos: int32 [n_q_total] position of each query in its sequence.
 * q: [n_q_total][n_q_heads][head_dim] in q_fmt; out float32 same shape; lse
 * float32 [n_q_total][n_q_heads] or NULL.
 * ------------------------------------------------------------------------- */
size_t pkv_prefill_workspace_bytes(const pkv_shape* shape, int32_t n_q_total,
                                   int32_t max_q_per_seq, int32_t mode, int32_t n_runs);

pkv_status pkv_paged_attn_prefill_window(const pkv_shape* shape, int32_t n_q_total,
                                         int32_t max_q_per_seq, const void* q,
                                         const int32_t* cu_q, const int32_t* q_pos,
                                         const void* k_pool, const void* v_pool,
                                         const int32_t* block_table, const int32_t* seq_lens,
                                         int32_t mode, int32_t n_runs, const int32_t* window,
                                         float* out, float* lse, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Row moves ("KV Cache Design", section 2: a compaction changes only cells,
 * so rows move verbatim; whoever copies must apply the moves in order_moves
 * order — upward moves top-down, downward moves bottom-up, upward first —
 * because a destination may never land on a row not yet copied).
 *
 * A move is int32 (src, dst, len) in pool rows; dst > src is "up".  Upward
 * moves are ordered by descending src (then descending dst), downward moves
 * by ascending src (then ascending dst), ties by input index; moves with
 * dst == src or len <= 0 are no-ops and left out.  For move sets with no
 * safe order the result is defined as applying the ordered moves one after
 * another, each as a memmove.
 * ------------------------------------------------------------------------- */

/* Host only.  moves: host int32 [n][3].  order_out: host int32 [n]; receives
 * the indices of the effective moves in application order; *n_out their
 * count. */
pkv_status pkv_order_moves(const int32_t* moves, int32_t n, int32_t* order_out, int32_t* n_out);

/* copy_cells in two halves, so that the host work and the device work can
 * be placed (and overlapped) by the caller, and the device half captured
 * into a HIP graph:
 *  - pkv_copy_cells_plan (host only, no device calls): orders the moves and
 *    reduces them to a plan written into caller memory (any host memory;
 *    pinned memory lets the caller upload it asynchronously);
 *  - the caller copies the plan's n_words int32 words to device memory;
 *  - pkv_copy_cells_apply (device only: kernels on `stream`, nothing else):
 *    moves the rows.
 * Plan kinds: when no destination of a move overlaps another destination or
 * any source (every compaction the block pool plans), every application
 * order gives the same bytes and the plan is the moves themselves (kind 1:
 * [n_moves][3] (src, dst, len), then the n_moves + 1 prefix sums of the
 * lengths).  Otherwise the ordered moves are replayed on the host into the
 * final source of every changed row (kind 2: [n_gather][2] (source row,
 * stage slot) for rows that are read and also overwritten, then
 * [n_scatter][2] (row, source row or -(stage slot + 1))); the device first
 * copies the gathered rows into a stage, then writes every changed row. */
typedef struct {
  int32_t kind;       /* 0: nothing to copy; 1: disjoint runs; 2: staged rows */
  int32_t n_moves;    /* kind 1: runs (moves with len > 0 and src != dst)  */
  int32_t total_rows; /* kind 1: rows the runs copy                          */
  int32_t n_gather;   /* kind 2: rows copied into the stage first            */
  int32_t n_scatter;  /* kind 2: rows written                                */
  int32_t reserved;
  int64_t n_words;    /* int32 words of the plan                             */
} pkv_copy_plan;

/* Words of the plan buffer pkv_copy_cells_plan needs for these moves: room
 * for the plan and for the planner's working arrays, so that planning
 * allocates nothing (0 when there is nothing to move or on bad input). */
int64_t pkv_copy_cells_plan_words(const int32_t* moves, int32_t n);

/* Host only.  moves: host int32 [n][3] in pool rows; every effective move
 * must lie inside [0, n_pool_rows) or the call is refused.  plan: host int32
 * [plan_words], 8-byte aligned, at least pkv_copy_cells_plan_words; the
 * call works in it and leaves the plan in its first info->n_words words;
 * *info receives the kind and the counts.  No global state and no
 * allocation: safe to call from any thread, and callers that keep one
 * buffer (pinned, say) reuse it without page faults. */
pkv_status pkv_copy_cells_plan(const int32_t* moves, int32_t n, int64_t n_pool_rows, int32_t* plan,
                               int64_t plan_words, pkv_copy_plan* info);

/* Device stage bytes pkv_copy_cells_apply needs for this plan (kind 2:
 * n_gather rows of each pool; else 0). */
size_t pkv_copy_cells_stage_bytes(const pkv_copy_plan* info, int64_t row_bytes_k, int64_t row_bytes_v);

/* Device only.  Applies a plan to k_pool and, if not NULL, v_pool (both
 * [n_pool_blocks][n_kv_heads][block_size][seg], seg_bytes_* a multiple of
 * 4).  plan: device int32 [info->n_words], the words pkv_copy_cells_plan
 * wrote.  stage: device, pkv_copy_cells_stage_bytes bytes, 16-byte aligned
 * (may be NULL for kind 0 and 1).  Launches kernels on `stream` only (no
 * allocation, copy or synchronization), so it can be captured into a HIP
 * graph; a captured apply moves the rows again on every replay.  Rows or
 * stage slots in the device plan outside the pool or the stage are skipped
 * (the plan is device data the host does not read back). */
pkv_status pkv_copy_cells_apply(void* k_pool, void* v_pool, int32_t n_pool_blocks, int32_t block_size,
                                int32_t n_kv_heads, int64_t seg_bytes_k, int64_t seg_bytes_v,
                                const pkv_copy_plan* info, const int32_t* plan, void* stage,
                                size_t stage_bytes, void* stream);

/* Workspace for pkv_kv_copy_cells with these moves (an upper bound: the
 * plan and the stage); row_bytes_* = bytes of one token cell (all kv heads)
 * of each pool. */
size_t pkv_copy_cells_workspace_bytes(const int32_t* moves, int32_t n, int64_t row_bytes_k,
                                      int64_t row_bytes_v);

/* Plan, upload and apply in one call: moves (host int32 [n][3]) are planned
 * into memory the call allocates and frees on the host, the plan is copied
 * into the front of `workspace` on `stream` and the call waits for the
 * stream (so the plan's host memory can be freed), then the rows are moved
 * as by pkv_copy_cells_apply with the rest of the workspace as the stage
 * (asynchronously).  `moves` may be freed on return.  Not capturable;
 * callers that plan ahead, overlap the host plan with device work or
 * capture use the two halves. */
pkv_status pkv_kv_copy_cells(void* k_pool, void* v_pool, int32_t n_pool_blocks, int32_t block_size,
                             int32_t n_kv_heads, int64_t seg_bytes_k, int64_t seg_bytes_v,
                             const int32_t* moves, int32_t n, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Store: write the K and V rows of n_tok new tokens into the pools through
 * the block table, each in its pool's format — the write that precedes
 * every read ("KV Cache Design", section 2 names the store op of the fused
 * decode family; "Tiered KV cache — architecture", section "The
 * paged-attention block model": position p of sequence s lives in physical
 * block table[s][p / block_size] at slot p % block_size).
 *
 * Formats ("KV Cache Design", section 3: one quantizer for every store):
 *  - q8_0: per 32 values, d = amax / 127 in binary32; each code is x / d
 *    (binary32 division) rounded to nearest, ties to even, clamped to
 *    [-127, 127]; the stored scale is d rounded to binary16 (nearest-even).
 *    amax = 0 gives scale 0 and zero codes.  Codes are taken against d, so
 *    a block whose scale underflows binary16 keeps its codes with scale 0.
 *    Bytes past the last block of a segment (head_dim / 32 odd) are zero.
 *  - f16: the source rounded to binary16 (nearest-even); f32: exact.
 *  Inputs are finite, and amax / 127 fits binary16; other values are
 *  outside the format and give unspecified bytes.
 *
 * shape: n_seqs, n_kv_heads, head_dim (32, 64, 128 or 256), block_size,
 *   n_pool_blocks, max_blocks_per_seq, k_fmt and v_fmt are used; the other
 *   fields are ignored.
 * src_fmt: PKV_F32 or PKV_F16, the type of k_new and v_new.
 * k_new, v_new: device [n_tok][n_kv_heads][head_dim] of src_fmt, 16-byte
 *   aligned.  v_new and v_pool may both be NULL (store K only).
 * seq_ids: device int32 [n_tok], the sequence of each token, or NULL: token
 *   t belongs to sequence t (then n_tok <= n_seqs).
 * positions: device int32 [n_tok], the position of each token.
 * block_table: device int32 [n_seqs][max_blocks_per_seq].
 * k_pool, v_pool: device pools as for attention, 16-byte aligned.
 * skipped: device int32, or NULL.  A token whose sequence lies outside
 *   [0, n_seqs), whose position lies outside [0, max_blocks_per_seq *
 *   block_size), or whose table entry is not a block of the pool (the
 *   sentinel included) is not stored: its rows are left as they were and 1
 *   is added to *skipped (the caller clears it).
 * Destinations must be distinct: a row named by two tokens of one call
 * holds unspecified bytes.  Only the named rows are written.  n_tok = 0 is
 * a no-op whatever the pointers are.
 * ------------------------------------------------------------------------- */
pkv_status pkv_kv_store(const pkv_shape* shape, int32_t n_tok, int32_t src_fmt, const void* k_new,
                        const void* v_new, const int32_t* seq_ids, const int32_t* positions,
                        const int32_t* block_table, void* k_pool, void* v_pool, int32_t* skipped,
                        void* stream);

/* ---------------------------------------------------------------------------
 * Copy-on-write block pool (host).  Forking a sequence only raises the
 * reference counts of its blocks and copies its table; no K/V bytes move
 * until a fork writes ("Tiered KV cache — architecture", section "The
 * paged-attention block model").  A store may never land in a block another
 * sequence still reads, so a write into a shared block first copies it into
 * a fresh block ("KV Cache Design", sections 1 and 2); readers of the shared
 * prefix see no change.  A partial removal wipes whole logical blocks (their
 * entries become PKV_INVALID_BLOCK_ID).  The pool also keeps a watermark of
 * blocks that admission checks leave free (the same page's file list names a
 * physical allocator with reference counts and a watermark).
 *
 * The pool owns only host memory: per-block reference counts, the block
 * tables [n_seqs][max_blocks_per_seq] and sequence lengths.  Callers export
 * the tables to the device (pkv_pool_export) for attention and store.  Not
 * internally locked; one thread mutates a pool at a time.
 *
 * Rules:
 *  - allocation takes the free block with the smallest id; a block is free
 *    exactly when no table entry names it;
 *  - fork(src, dst, n): dst must be empty; it takes src's first
 *    ceil(n / block_size) entries (holes stay holes) and length n (n < 0:
 *    src's length); each block it names gains a reference;
 *  - remove(seq, p0, p1) on [p0, p1) clipped to [0, length): if it reaches
 *    the end, the length becomes p0 and every logical block starting at or
 *    after p0 is released; otherwise each logical block lying wholly inside
 *    is released and becomes a hole (removal is block-granular);
 *  - prepare_writes before writing positions [p0, p0 + count) of seq
 *    (p0 <= length, no gap), for each write in order and each logical block
 *    it touches: a block only this sequence names is written in place; a
 *    shared block is copied into a fresh block (the pair (src, dst) is
 *    returned, the shared block loses a reference); an empty entry gets a
 *    fresh block, whose rows other than the written ones hold whatever the
 *    pool held.  The length becomes max(length, p0 + count).  The returned
 *    ops must run (pkv_cow_apply) before the rows are stored; their copies
 *    read the blocks as they were before the batch.  The whole batch is checked
 *    before anything changes: a refused call changes nothing.
 * ------------------------------------------------------------------------- */
typedef struct pkv_block_pool pkv_block_pool;

pkv_status pkv_pool_create(int32_t n_blocks, int32_t n_seqs, int32_t max_blocks_per_seq,
                           int32_t block_size, int32_t watermark, pkv_block_pool** out);
void pkv_pool_destroy(pkv_block_pool* pool);

/* Free blocks; whether n more blocks can be taken with the watermark still
 * free (1/0); references to a block (-1 outside the pool); a sequence's
 * length (-1 outside the pool). */
int32_t pkv_pool_free_blocks(const pkv_block_pool* pool);
int32_t pkv_pool_can_allocate(const pkv_block_pool* pool, int32_t n);
int32_t pkv_pool_refcount(const pkv_block_pool* pool, int32_t block);
int32_t pkv_pool_seq_len(const pkv_block_pool* pool, int32_t seq);

pkv_status pkv_pool_fork(pkv_block_pool* pool, int32_t src, int32_t dst, int32_t n_tokens);
pkv_status pkv_pool_remove(pkv_block_pool* pool, int32_t seq, int32_t p0, int32_t p1);

/* n writes (host arrays seqs, p0s, counts; counts <= 0 are skipped).
 * ops_out: host int32 [max_ops][3] receiving one op per table entry the
 * writes change, in order: (src, dst, entry) = (the shared block to copy,
 * or -1 for a fresh block with nothing to copy; the new block; the entry's
 * index seq * max_blocks_per_seq + logical block).  *n_ops their number.
 * PKV_E_CAPACITY when the pool lacks free blocks, PKV_E_WORKSPACE when
 * max_ops is too small (at most one op per logical block a write touches). */
pkv_status pkv_pool_prepare_writes(pkv_block_pool* pool, int32_t n, const int32_t* seqs,
                                   const int32_t* p0s, const int32_t* counts, int32_t* ops_out,
                                   int32_t max_ops, int32_t* n_ops);

/* Compaction ("KV Cache Design", section 2: a compaction changes only cells,
 * so rows move verbatim through copy_cells in order_moves order, and the
 * defragmenter returns the moves for whoever caches block ids).  Makes the
 * top `need` block ids free (need < 0: as many as are free, so every live
 * block ends below the live count): the live blocks among them, ascending,
 * move into the lowest free blocks, ascending; tables and reference counts
 * follow at once.  A block-table sequence need not be contiguous, so holes
 * are filled instead of sliding everything down: the fewest blocks move and
 * every move goes down onto a free row (no destination is a source).
 * moves_out: host int32 [max_moves][3] (src_row, dst_row, len) in pool rows
 * (row = block * block_size + slot), consecutive blocks that land on
 * consecutive blocks merged; apply them to the K and V pools with
 * pkv_kv_copy_cells, and re-export the tables, before the next read.
 * PKV_E_CAPACITY if need exceeds the free blocks, PKV_E_WORKSPACE if
 * max_moves is too small (at most one move per moved block); a refused call
 * changes nothing. */
pkv_status pkv_pool_defrag(pkv_block_pool* pool, int32_t need, int32_t* moves_out, int32_t max_moves,
                           int32_t* n_moves);

/* Host copies of the tables (int32 [n_seqs][max_blocks_per_seq]) and, if
 * lens_out is not NULL, the lengths (int32 [n_seqs]). */
pkv_status pkv_pool_export(const pkv_block_pool* pool, int32_t* table_out, int32_t* lens_out);

/* Device: apply prepare_writes' ops (device int32 [n][3]).  For each op,
 * copy block src (when src >= 0) to block dst in k_pool and (if not NULL)
 * v_pool, both [n_pool_blocks][...] with k_block_bytes / v_block_bytes per
 * block (n_kv_heads * block_size * seg; multiples of 4; pools 16-byte
 * aligned), and, when table is not NULL, set table[entry] = dst (table:
 * device int32 of table_entries entries, the block tables [n_seqs]
 * [max_blocks_per_seq] that attention and store read).  An op whose src or
 * dst lies outside [0, n_pool_blocks), or with src == dst, copies nothing;
 * an entry outside the table is not patched.  Sources and destinations must
 * be disjoint, destinations distinct and entries distinct (prepare_writes
 * guarantees all three); otherwise the result is unspecified.
 * Run it before storing the batch's rows. */
pkv_status pkv_cow_apply(void* k_pool, void* v_pool, int32_t n_pool_blocks, int64_t k_block_bytes,
                         int64_t v_block_bytes, const int32_t* ops, int32_t n, int32_t* table,
                         int64_t table_entries, void* stream);

/* ---------------------------------------------------------------------------
 * int4 cold-block codec ("Tiered KV cache — architecture", section "The
 * three-tier model": a cold block is one f32 scale followed by ceil(n / 2)
 * bytes of packed int4 nibbles, one scale per block; about 0.99 cosine
 * similarity against the original).  A block is one pool block of one pool
 * taken flat in memory order: block_elems = n_kv_heads * block_size *
 * head_dim values (a multiple of 8, at most 65536).  Quantizer, in binary32:
 * scale = amax / 7; code = x / scale rounded to nearest, ties to even,
 * clamped to [-7, 7]; amax = 0 gives scale 0 and zero codes.  Blob: the
 * scale (little-endian f32), then byte j = code 2j (low nibble, two's
 * complement) | code 2j+1 (high nibble).  Decoding writes scale * code,
 * rounded to binary32 and then to the pool format (nearest-even).
 *
 * pool: device [n_pool_blocks][block_elems] of fmt (PKV_F16 or PKV_F32),
 * 16-byte aligned.  blocks: device int32 [n] pool block ids.  blobs: device
 * [n][blob_stride] bytes, 4-byte aligned, blob_stride >= blob bytes and a
 * multiple of 4; bytes past a blob's end are not touched.  Encode of a
 * block id outside the pool writes an all-zero blob; decode into one writes
 * nothing.  Destination block ids of one decode call are distinct.
 * ------------------------------------------------------------------------- */
int64_t pkv_int4_blob_bytes(int64_t n_elts);
pkv_status pkv_int4_encode(const void* pool, int32_t fmt, int32_t n_pool_blocks, int64_t block_elems,
                           const int32_t* blocks, int32_t n, void* blobs, int64_t blob_stride,
                           void* stream);
pkv_status pkv_int4_decode(const void* blobs, int64_t blob_stride, int32_t n, void* pool, int32_t fmt,
                           int32_t n_pool_blocks, int64_t block_elems, const int32_t* blocks,
                           void* stream);

/* ---------------------------------------------------------------------------
 * Debug export of the block-table/window resolver the attention kernels use.
 * rows_out: int32 [n_q_total][n_cand]: for query j and candidate index i of
 * its sequence's window enumeration (causal: positions 0..seq_len-1; span:
 * lo..hi-1; kv_map: the concatenation of its runs with len > 0) the pool
 * row that slot reads, or -1 when the index is past the enumeration, the
 * position is outside [0, min(seq_len, q_pos + 1)) or it lies in a hole.
 * Decode (cu_q == NULL and q_pos == NULL): n_q_total == n_seqs, query s at
 * position seq_len_s - 1.  Prefill: cu_q / q_pos as for prefill.
 * ------------------------------------------------------------------------- */
pkv_status pkv_resolve_rows(const pkv_shape* shape, int32_t n_q_total, const int32_t* cu_q,
                            const int32_t* q_pos, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t mode, int32_t n_runs,
                            const int32_t* window, int32_t n_cand, int32_t* rows_out,
                            void* stream);

/* Message of the last refused call on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
