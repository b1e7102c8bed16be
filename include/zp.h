/*
 * zp.h -- C ABI of the Compressed PagedAttention hot path for MI355X (gfx950).
 *
 * Compressed PagedAttention (Zipage) keeps every request's KV cache within a
 * fixed number of paged blocks.  Once a request holds N_max full blocks, a
 * compression pass scores every cached token per layer and per KV head,
 * drops the lowest-scoring ones, and relocates the survivors, in order, into
 * the first N_max-1 blocks; the last block is kept free for the tokens that
 * follow, and surplus blocks are released (gist.science/nl/paper/2603.08743,
 * "Technische samenvatting", Methodologie item 1; gist.science/ko/paper/
 * 2603.08743, "기술 요약", section 2.A).  Decode attention then reads the
 * compacted blocks through the usual block table (upskillscore.com guide
 * "Paged KV cache and continuous batching", "How it works").
 *
 * All entry points are plain C.  Device buffers are CALLER-owned (for
 * example PyTorch tensors); the library owns only the host-side block pool
 * (reference counts, free set, deferred frees), a few HIP events and a small
 * ring of pinned host staging buffers used to upload block tables.  Streams
 * are passed as `void*` holding a hipStream_t (NULL = the null stream).
 *
 * Errors: every call returns a zp_status; on any error other than ZP_ERR_HIP
 * the call has changed nothing (tables, reference counts, pool, device
 * memory).  zp_last_error() gives a human-readable reason for the calling
 * thread's last failure.  Work is enqueued asynchronously; a HIP failure
 * after the pool was updated marks the pool unusable (ZP_ERR_STATE from then
 * on).  The pool is not thread-safe: one scheduler thread owns it.
 *
 * Layouts (row-major, no padding):
 *   KV pool of one layer .... [num_blocks][H][b][d] elements, one pool for K
 *                             and one for V per layer; the (block, head) tile
 *                             is a contiguous b*d run.
 *   block table ............. int32 [R][n] physical block ids; logical slot j
 *                             of a request lives in block table[j / b] at
 *                             offset j % b.
 *   window queries .......... [R][w][Hq][d] per layer, the queries of the
 *                             last w cached slots, or a query-slot store
 *                             [S*w][Hq][d] the decode records into, read in
 *                             place (zp_compress_ex, window_slots).
 *   decode query ............ [R][Hq][d]; output float32 [R][Hq][d]
 *                             (bfloat16 through zp_paged_decode_ex).
 * Query head hq belongs to KV head hq / G with G = Hq / H (grouped queries).
 * Element type: float32 or bfloat16 for caches and queries alike.
 */
#ifndef ZP_H
#define ZP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZP_VERSION 2

typedef enum {
  ZP_OK = 0,
  ZP_ERR_INVALID = 1,   /* bad argument; nothing changed */
  ZP_ERR_NO_BLOCKS = 2, /* not enough free blocks; nothing changed */
  ZP_ERR_HIP = 3,       /* HIP runtime failure */
  ZP_ERR_STATE = 4      /* pool unusable after an earlier HIP failure */
} zp_status;

typedef enum { ZP_F32 = 0, ZP_BF16 = 1 } zp_dtype;

/* Reason for the calling thread's last failure ("" if none). */
const char* zp_last_error(void);
int32_t zp_version(void);

/* Geometry of a paged KV cache.  head_dim in {64, 128}, block_size in
 * {16, 32}, num_q_heads a multiple of num_kv_heads with G in {1, 2, 4, 8}.
 * k_cache / v_cache: host arrays of num_layers device pointers, each to a
 * [num_blocks][num_kv_heads][block_size][head_dim] pool (caller-owned). */
typedef struct zp_kv_cache {
  int32_t num_layers;
  int32_t num_kv_heads;
  int32_t num_q_heads;
  int32_t head_dim;
  int32_t block_size;
  int32_t num_blocks;
  int32_t dtype; /* zp_dtype */
  void* const* k_cache;
  void* const* v_cache;
} zp_kv_cache;

/* ------------------------------------------------------------------------
 * Block pool (host object): reference counts per physical block, a free set
 * handed out smallest id first, and blocks whose release waits for the GPU
 * work that still reads them.  Sharing through reference counts and
 * allocate-then-decrement follow the paged-cache guide ("How it works") and
 * the shared-prefix handling of the Zipage summaries (ko page section 2.C,
 * nl page Methodologie item 3).
 * ---------------------------------------------------------------------- */
typedef struct zp_block_pool zp_block_pool;

#define ZP_POOL_MANUAL_FENCE 1u /* deferred frees wait for zp_block_pool_fence()
                                   instead of HIP events (CPU-only use) */

/* Create a pool of num_blocks ids, all free (refcount 0). */
zp_status zp_block_pool_create(int32_t num_blocks, uint32_t flags, zp_block_pool** out);
void zp_block_pool_destroy(zp_block_pool* pool);
/* Allocate n blocks, smallest free ids first, refcount := 1; all or nothing
 * (ZP_ERR_NO_BLOCKS leaves the pool unchanged).  Completed deferred frees are
 * reclaimed first. */
zp_status zp_block_alloc(zp_block_pool* pool, int32_t n, int32_t* ids_out);
/* refcount += 1 for each id (prefix sharing); every id must be in use. */
zp_status zp_block_share(zp_block_pool* pool, const int32_t* ids, int32_t n);
/* refcount -= 1 for each id; ids reaching 0 are freed at once and listed in
 * freed_out (capacity n, may be NULL) / *n_freed (may be NULL).  The caller
 * guarantees no queued GPU work still reads them. */
zp_status zp_block_release(zp_block_pool* pool, const int32_t* ids, int32_t n,
                           int32_t* freed_out, int32_t* n_freed);
int32_t zp_block_refcount(const zp_block_pool* pool, int32_t id); /* -1 if out of range */
int32_t zp_block_num_free(const zp_block_pool* pool);    /* allocatable now */
int32_t zp_block_num_pending(const zp_block_pool* pool); /* freed, waiting for GPU work */
/* ZP_POOL_MANUAL_FENCE pools: mark every pending group complete. */
zp_status zp_block_pool_fence(zp_block_pool* pool);
/* Wait for the GPU work of every pending group and reclaim its blocks. */
zp_status zp_block_pool_sync(zp_block_pool* pool);

/* ------------------------------------------------------------------------
 * Compression planning (host only; also called by zp_compress).
 *
 * Trigger (decided by the caller): each of the num_reqs requests holds
 * exactly n_max full blocks (nl page Methodologie item 1: N_max blocks and
 * the last block full).  Reference counts are read as they stand at the
 * start of the call.  For each request, in order, and each logical block
 * n < n_max-1: a block held only by this request is compacted in place; a
 * shared block is replaced by a newly allocated target block (smallest free
 * id) and this request drops its reference to it (ko page section 2.C: new
 * target blocks keep the shared blocks intact).  The last logical block
 * becomes the reserved block: kept if private, replaced by a fresh block if
 * shared.  Blocks whose count reaches 0 are released once the GPU work of
 * the call is done (pending until then).
 *
 * block_tables: HOST int32 [num_reqs][n_max], rewritten on success.
 * src_out:      HOST int32 [num_reqs][n_max]   (the tables as they were).
 * dst_out:      HOST int32 [num_reqs][n_max-1] (compaction targets).
 * freed_ids:    HOST int32, capacity num_reqs*n_max; *num_freed entries.
 * Rejected (ZP_ERR_INVALID, nothing changed): n_max < 2, num_reqs < 0, ids
 * out of range, ids with refcount 0, an id twice in one table, an id listed
 * more often than its refcount.  ZP_ERR_NO_BLOCKS if fewer free blocks than
 * shared table entries.  The pending group of a plan made without
 * zp_compress is released by zp_block_pool_fence() / zp_block_pool_sync().
 * ---------------------------------------------------------------------- */
zp_status zp_compress_plan(zp_block_pool* pool, int32_t n_max, int32_t num_reqs,
                           int32_t* block_tables, int32_t* src_out, int32_t* dst_out,
                           int32_t* freed_ids, int32_t* num_freed);

/* zp_compress_plan for requests that hold n_src >= n_max full blocks: a
 * cache past the cap (a prompt longer than the budget, or a chunk of one)
 * is compressed to the same n_max-block shape, and its surplus blocks are
 * released (nl page Methodologie item 1: the surplus blocks are freed).
 * Blocks 0..n_max-2 become targets and block n_max-1 the reserved block as
 * in zp_compress_plan; for blocks n_max..n_src-1 the request drops its
 * reference (freed when it was the last).
 * block_tables: HOST int32 [num_reqs][n_src]; on success each row holds
 *               the n_max new ids followed by n_src-n_max entries of -1.
 * src_out:      HOST int32 [num_reqs][n_src].
 * dst_out:      HOST int32 [num_reqs][n_max-1].
 * freed_ids:    HOST int32, capacity num_reqs*n_src.
 * Rejected as zp_compress_plan, and n_src < n_max. */
zp_status zp_compress_plan_n(zp_block_pool* pool, int32_t n_src, int32_t n_max, int32_t num_reqs,
                             int32_t* block_tables, int32_t* src_out, int32_t* dst_out,
                             int32_t* freed_ids, int32_t* num_freed);

/* Optional device outputs of zp_compress for checking (any may be NULL).
 * T = n_src*block_size (n_src = n_max for zp_compress and zp_compress_lse),
 * K_keep = (n_max-1)*block_size. */
typedef struct zp_compress_debug {
  float* importance;  /* [L][R][H][T]: observation-window importance A */
  float* redundancy;  /* [L][R][H][T]: Lightning Redundancy Score R */
  float* score;       /* [L][R][H][T]: s = A*(1-R); slots >= T-w are not scored */
  int32_t* kept;      /* [L][R][H][K_keep]: surviving old slots, ascending */
  /* [L][R][H][5]: the device wall clock (zp_compress_info.wall_clock_khz)
   * read by each (layer, request, head) workgroup at its start, after the
   * softmax statistics (pass 1; right after the start when the
   * normalisers are supplied), after the scores (pass 2), after the selection, and at
   * its end (after its compaction when the same kernel compacts) -- where
   * the time of a compression goes, unit by unit. */
  int64_t* phase_times;
} zp_compress_debug;

/* Device workspace (caller-owned) needed by zp_compress / zp_compress_lse,
 * and by zp_compress_n with n_src source blocks (0 on invalid arguments). */
size_t zp_compress_workspace_bytes(const zp_kv_cache* cache, int32_t num_reqs, int32_t n_max,
                                   int32_t window);
size_t zp_compress_workspace_bytes_n(const zp_kv_cache* cache, int32_t num_reqs, int32_t n_src,
                                     int32_t n_max, int32_t window);

/* ------------------------------------------------------------------------
 * zp_compress: one compression call over every layer for num_reqs requests
 * that each hold n_max full blocks.
 *
 * Per layer l, request r and KV head h, with T = n_max*b cached slots, the
 * window slots C..T-1 (C = T-w), and the G query heads of h:
 *   importance  A[j] = mean over the G*w (query head, window row i) pairs of
 *               the causal softmax, over slots 0..C+i, of q.k_j/sqrt(d), at
 *               slot j (ko page section 2.A: scores from the queries of the
 *               last w tokens of the last block);
 *   redundancy  R[j] = mean cosine similarity of k_j with the other b-1 keys
 *               of its block, 0 for a zero-norm key (Lightning Redundancy
 *               Score: similarity only inside a block, nl page Methodologie
 *               item 5, ko page section 2.E);
 *   score       s[j] = A[j] * (1 - R[j]) for candidates j < C (the pages do
 *               not say how the two combine; this is the fixed reading);
 *   survivors   the window slots plus the K_sel = (n_max-1)*b - w candidates
 *               with the largest s (equal s: lower slot kept), moved in
 *               ascending slot order into logical slots 0..K_keep-1 of the
 *               targets from zp_compress_plan, for K and V alike.
 * Afterwards each request's table is [targets..., reserved block] and its
 * length is K_keep; the next token goes to slot K_keep.
 *
 * window_q:  host array [num_layers] of device pointers to [R][w][Hq][d].
 * workspace: device, >= zp_compress_workspace_bytes(), 256-byte aligned,
 *            must stay untouched until the stream has passed this call.
 * freed_ids / num_freed: as zp_compress_plan (blocks become allocatable
 *            only after this call's GPU work has completed).
 * stream:    hipStream_t; all device work is enqueued on it, with no
 *            device-to-host synchronisation.
 * Rejects (ZP_ERR_INVALID) everything zp_compress_plan rejects, plus bad
 * geometry, window < 1 or window > block_size, NULL pointers, a short or
 * misaligned workspace, and a pool created with ZP_POOL_MANUAL_FENCE.
 * ---------------------------------------------------------------------- */
zp_status zp_compress(const zp_kv_cache* cache, zp_block_pool* pool, int32_t n_max,
                      int32_t window, int32_t num_reqs, int32_t* block_tables,
                      const void* const* window_q, void* workspace, size_t workspace_bytes,
                      int32_t* freed_ids, int32_t* num_freed, void* stream,
                      const zp_compress_debug* debug);

/* ------------------------------------------------------------------------
 * zp_compress_lse: zp_compress with the softmax normalisers of the window
 * rows supplied by the caller, so the scoring reads K once instead of twice.
 *
 * The window queries are the queries of the last w decode steps of each
 * request (the "query slots" of the hybrid scheduling, nl page Methodologie
 * item 2, ko page section 2.B).  The decode step of window position i
 * already attended over exactly the slots 0..C+i that the importance
 * softmax of row i spans (causal window, no compression in between), so its
 * log-sum-exp is that row's normaliser; zp_paged_decode_lse returns it.
 *
 * window_lse: NULL (then exactly zp_compress), or a host array [num_layers]
 *   of device pointers to float [R][w][Hq]: for request r, window position i
 *   and query head hq, ln sum over j <= C+i of exp(q.k_j / sqrt(head_dim)),
 *   taken over the cache as it stands at this call.  Non-finite entries give
 *   that row probability 0.  Values that do not match the cache are not
 *   detected: the importances are then off by the per-row factor.
 * Everything else, including the results up to rounding, as zp_compress.
 * ---------------------------------------------------------------------- */
zp_status zp_compress_lse(const zp_kv_cache* cache, zp_block_pool* pool, int32_t n_max,
                          int32_t window, int32_t num_reqs, int32_t* block_tables,
                          const void* const* window_q, const void* const* window_lse,
                          void* workspace, size_t workspace_bytes, int32_t* freed_ids,
                          int32_t* num_freed, void* stream, const zp_compress_debug* debug);

/* ------------------------------------------------------------------------
 * zp_compress_n: zp_compress_lse for requests that each hold n_src >= n_max
 * full blocks (a cache past the cap: a long prompt, or a prefill chunk).
 * T = n_src*b slots are scored as in zp_compress (window = the last w
 * slots), E = (n_src - n_max + 1)*b candidates per (layer, head) are
 * evicted, and the K_keep = (n_max-1)*b survivors move in order into the
 * first n_max-1 blocks; the plan is zp_compress_plan_n's (surplus blocks
 * released once the GPU work is done).
 * block_tables: HOST int32 [num_reqs][n_src], rewritten as by
 *               zp_compress_plan_n.
 * window_lse:   as zp_compress_lse (may be NULL).
 * freed_ids:    HOST int32, capacity num_reqs*n_src.
 * Rejects everything zp_compress rejects, plus n_src < n_max, n_src > 512,
 * n_src*b > 8192 and more than 1024 evictions per head.
 * ---------------------------------------------------------------------- */
zp_status zp_compress_n(const zp_kv_cache* cache, zp_block_pool* pool, int32_t n_src,
                        int32_t n_max, int32_t window, int32_t num_reqs, int32_t* block_tables,
                        const void* const* window_q, const void* const* window_lse,
                        void* workspace, size_t workspace_bytes, int32_t* freed_ids,
                        int32_t* num_freed, void* stream, const zp_compress_debug* debug);

/* ------------------------------------------------------------------------
 * zp_compress_ex: every compression call above, with its options in one
 * struct, and one more: the caller's device copy of the block tables.
 *
 * Serving engines keep the block tables on the GPU for decode anyway.
 * Given that copy, a call whose plan compacts every request in place (no
 * shared block re-targeted -- the usual case) uploads nothing and records
 * no event: the kernels read the sources and, in place, the targets from
 * the device table, and the per-layer pointers travel in the kernel
 * arguments.  Plans that re-target shared blocks still upload their target
 * table (host staging ring, one event).  Without the device copy the source
 * table is uploaded, and the target table only when it differs from it.
 *
 * Fields (results exactly as the entry point each combination names):
 *   n_src, n_max    blocks each request holds (>= n_max; n_src = n_max is
 *                   zp_compress / zp_compress_lse, larger is zp_compress_n)
 *   window, num_reqs, block_tables (HOST int32 [num_reqs][n_src], rewritten
 *                   on success), window_q, window_lse (may be NULL),
 *                   workspace, workspace_bytes, freed_ids, num_freed,
 *                   stream, debug (may be NULL): as zp_compress_n.
 *   device_tables   NULL, or DEVICE int32 [num_reqs][n_src] (row stride
 *                   n_src, 4-byte aligned) holding the same ids as
 *                   block_tables at the call.  The library compares the
 *                   two only under ZP_DEBUG_VALIDATE: a copy that differs
 *                   gives wrong results (every id is still read as a block
 *                   of the pool).  Not written; after
 *                   a plan that re-targets blocks the caller refreshes it
 *                   from the rewritten host tables.
 *   flags           0, or ZP_COMPRESS_KEEP_PREFIX (zp_compress_keep_prefix).
 *   num_blocks      NULL (every request holds n_src blocks), or HOST int32
 *                   [num_reqs]: request r holds the first num_blocks[r]
 *                   entries of its row, n_max <= num_blocks[r] <= n_src, and
 *                   the rest of the row is -1 (in block_tables and in
 *                   device_tables alike: the kernels read each request's
 *                   count off its row).  Requests past the cap by different
 *                   amounts -- prompts compressed after chunks of their
 *                   prefill, say -- then share one call; each is scored on
 *                   its own T = num_blocks[r]*b slots and evicts
 *                   (num_blocks[r] - n_max + 1)*b per head.  Debug outputs
 *                   keep the row stride T = n_src*b; slots past a request's
 *                   own T are left as they were.
 *   window_slots    NULL (window_q[l] is [num_reqs][window][Hq][d] and
 *                   window_lse[l] [num_reqs][window][Hq]), or DEVICE int32
 *                   [num_reqs]: the query slot of each request.  window_q[l]
 *                   and window_lse[l] are then the query-slot stores the
 *                   decode records into (zp_paged_decode_lse's q_out and
 *                   lse_out), [window_store_slots*window][Hq][d] and
 *                   [window_store_slots*window][Hq], and request r's window
 *                   position i is their row window_slots[r]*window + i --
 *                   the hybrid scheduler's query slots (nl page Methodologie
 *                   item 2, ko page section 2.B) read in place, with nothing
 *                   gathered first.  A slot outside [0, window_store_slots)
 *                   is read as slot 0 (never outside the store); its
 *                   request's results are then meaningless.
 *   window_store_slots  slots in those stores (>= 1 when window_slots is set).
 * Rejects what the named entry points reject, unknown flags, a misaligned
 * device_tables or window_slots, window_store_slots < 1 with window_slots,
 * and num_blocks outside [n_max, n_src] or rows not padded with -1.  Kernels never follow an id outside the pool: a device table that
 * holds one reads that block as block 0 and never writes it.
 * ---------------------------------------------------------------------- */
#define ZP_COMPRESS_KEEP_PREFIX 1u

typedef struct zp_compress_args {
  int32_t n_src;
  int32_t n_max;
  int32_t window;
  int32_t num_reqs;
  int32_t* block_tables;
  const int32_t* device_tables;
  const void* const* window_q;
  const void* const* window_lse;
  void* workspace;
  size_t workspace_bytes;
  int32_t* freed_ids;
  int32_t* num_freed;
  void* stream;
  const zp_compress_debug* debug;
  uint32_t flags;
  const int32_t* num_blocks;
  const int32_t* window_slots;
  int32_t window_store_slots;
} zp_compress_args;

zp_status zp_compress_ex(const zp_kv_cache* cache, zp_block_pool* pool,
                         const zp_compress_args* args);

/* How zp_compress / zp_compress_lse / zp_compress_n run a call of this
 * shape on the current device (a host query; it enqueues nothing).  One
 * workgroup scores, selects and compacts each (layer, request, KV head)
 * unit; when every unit of the call is resident at once, the compaction
 * loads K normally (the scoring has just read it and much of it is still
 * cached), otherwise it streams K past the caches. */
typedef struct zp_compress_info {
  int32_t units;            /* num_layers * num_reqs * num_kv_heads workgroups */
  int32_t threads;          /* threads per workgroup */
  int32_t resident_per_cu;  /* such workgroups one compute unit holds at once */
  int32_t compute_units;    /* of the current device */
  int32_t k_cached;         /* 1: K loaded normally by the compaction; 0: streamed */
  int32_t wall_clock_khz;   /* rate of the clock in zp_compress_debug.phase_times */
} zp_compress_info;

/* Rejects (ZP_ERR_INVALID) the shapes zp_compress_n rejects; ZP_ERR_HIP
 * without a device. */
zp_status zp_compress_query(const zp_kv_cache* cache, int32_t num_reqs, int32_t n_src,
                            int32_t n_max, int32_t window, zp_compress_info* out);

/* ------------------------------------------------------------------------
 * zp_compress_keep_prefix: zp_compress_n that keeps shared blocks shared
 * when compression leaves them as they are.  New target blocks keep the
 * shared blocks intact for their other holders (ko page section 2.C, nl
 * page Methodologie item 3); a shared block that lies entirely below the
 * request's first evicted slot in every layer and head is not changed by
 * the compaction at all, so instead of a copy in a new block it stays in
 * the table, shared, and prefix caching keeps working after the
 * compression.  The plan therefore waits for the selection: the call
 * synchronises the host with `stream` once, after the scoring kernel.
 * Arguments, results and errors as zp_compress_n; ZP_ERR_NO_BLOCKS is
 * decided after the scoring (then only the workspace has changed).
 * ---------------------------------------------------------------------- */
zp_status zp_compress_keep_prefix(const zp_kv_cache* cache, zp_block_pool* pool, int32_t n_src,
                                  int32_t n_max, int32_t window, int32_t num_reqs,
                                  int32_t* block_tables, const void* const* window_q,
                                  const void* const* window_lse, void* workspace,
                                  size_t workspace_bytes, int32_t* freed_ids, int32_t* num_freed,
                                  void* stream, const zp_compress_debug* debug);

/* ------------------------------------------------------------------------
 * zp_append_kv: write one new token per request into layer `layer`.
 * k_new, v_new: device [R][H][d]; slot_mapping: device int32 [R], physical
 * slot block*b + offset (negative = skip).  The caller picks the slot:
 * the next free offset of the request's last block, the paged cache taking
 * a further block on demand once that one has filled (upskillscore.com
 * guide, "How it works").  A slot whose block lies outside the pool is
 * skipped.
 * ---------------------------------------------------------------------- */
zp_status zp_append_kv(const zp_kv_cache* cache, int32_t layer, int32_t num_reqs,
                       const void* k_new, const void* v_new, const int32_t* slot_mapping,
                       void* stream);

/* Device workspace for zp_paged_decode with tables of max_blocks columns. */
size_t zp_paged_decode_workspace_bytes(const zp_kv_cache* cache, int32_t num_reqs,
                                       int32_t max_blocks);

/* ------------------------------------------------------------------------
 * zp_paged_decode: attention of one new query per request over its cached
 * slots, read through the block table ("How it works": logical blocks map to
 * non-contiguous physical blocks).  For request r and query head hq:
 *   out[r][hq] = sum over j < seq_lens[r] of softmax_j(scale * q.k_j) v_j
 * with k_j, v_j of KV head hq/G at block block_tables[r][j/b], offset j%b.
 * q: device [R][Hq][d] (cache dtype); block_tables: device int32
 * [R][max_blocks]; seq_lens: device int32 [R], 0 <= seq_len <= max_blocks*b
 * (0 gives a zero output); out: device float32 [R][Hq][d]; workspace:
 * device, >= zp_paged_decode_workspace_bytes().  Entries of a table beyond
 * ceil(seq_len/b) are never read.  Device-side guards (the host cannot see
 * device tables): a seq_len outside [0, max_blocks*b] is clamped into it,
 * and a table entry outside [0, num_blocks) is skipped -- its slots add
 * nothing -- so no load ever leaves the pools.
 * ---------------------------------------------------------------------- */
zp_status zp_paged_decode(const zp_kv_cache* cache, int32_t layer, int32_t num_reqs,
                          const void* q, const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* seq_lens, float scale, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * zp_paged_decode_lse: zp_paged_decode that also records, per request, the
 * query and, per query head, the log-sum-exp of the scaled logits,
 *   lse[r][hq] = ln sum over j < seq_lens[r] of exp(scale * q.k_j)
 * (-inf for an empty request), into rows of caller-owned stores -- the
 * query slots of the hybrid scheduling (nl page Methodologie item 2).  With
 * scale = 1/sqrt(head_dim), a window row's recorded query and normaliser
 * are what zp_compress_lse takes.
 * lse_out:  NULL, or device float [capacity][Hq].
 * q_out:    NULL, or device [capacity][Hq][head_dim] in the cache dtype
 *           (16-byte aligned): a copy of q.
 * rows:     NULL (request r writes row r; then capacity >= num_reqs), or
 *           device int32 [num_reqs]: the row request r writes; rows outside
 *           [0, capacity) are skipped (e.g. -1 for requests that are not in
 *           their window).
 * Other arguments, layouts and errors as zp_paged_decode.
 * ---------------------------------------------------------------------- */
zp_status zp_paged_decode_lse(const zp_kv_cache* cache, int32_t layer, int32_t num_reqs,
                              const void* q, const int32_t* block_tables, int32_t max_blocks,
                              const int32_t* seq_lens, float scale, float* out, float* lse_out,
                              void* q_out, const int32_t* rows, int32_t capacity, void* workspace,
                              size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * zp_paged_decode_ex: zp_paged_decode_lse with its arguments in a struct,
 * and the output element type to choose.
 *   out_dtype   ZP_F32 (out: float [R][Hq][d], exactly zp_paged_decode_lse)
 *               or ZP_BF16 (out: bfloat16 [R][Hq][d], 2-byte aligned: the
 *               same float32 result rounded to nearest even).
 * Every other field, result and error as zp_paged_decode_lse (lse_out,
 * q_out and rows may be NULL); an unknown out_dtype is ZP_ERR_INVALID.
 * ---------------------------------------------------------------------- */
typedef struct zp_decode_args {
  int32_t layer;
  int32_t num_reqs;
  const void* q;
  const int32_t* block_tables;
  int32_t max_blocks;
  const int32_t* seq_lens;
  float scale;
  void* out;
  int32_t out_dtype; /* zp_dtype */
  float* lse_out;
  void* q_out;
  const int32_t* rows;
  int32_t capacity;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
} zp_decode_args;

zp_status zp_paged_decode_ex(const zp_kv_cache* cache, const zp_decode_args* args);

/* ------------------------------------------------------------------------
 * zp_paged_decode_noalloc: zp_paged_decode_lse for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  It takes no workspace: the
 * split partials go to a fixed 4 MiB device array inside the library, one
 * copy per GPU, held until the process ends; the call itself allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  Its
 * device address is looked up on the first call on each device.
 * Every argument, layout and result as zp_paged_decode_lse.  Calls on one
 * GPU share that array: two calls whose work overlaps on the GPU (on
 * different streams) race on it and must be ordered by the caller.
 * Rejects (ZP_ERR_INVALID) a batch whose partials would exceed the array
 * (none does at the library's split rule: at most about 2.1 MB at
 * head_dim 128), besides what zp_paged_decode_lse rejects.
 * ---------------------------------------------------------------------- */
zp_status zp_paged_decode_noalloc(const zp_kv_cache* cache, int32_t layer, int32_t num_reqs,
                                  const void* q, const int32_t* block_tables, int32_t max_blocks,
                                  const int32_t* seq_lens, float scale, float* out,
                                  float* lse_out, void* q_out, const int32_t* rows,
                                  int32_t capacity, void* stream);

/* ------------------------------------------------------------------------
 * zp_redundancy_all: the all-pairs redundancy that the Lightning Redundancy
 * Score replaces (nl page Methodologie item 5, ko page section 2.E: the
 * original score is O(N^2 b^2), the LRS O(N b^2)), for measuring that
 * replacement.  For request r, KV head h and each of the T = n_blocks*b
 * slots j of layer `layer`:
 *   out[r][h][j] = 1/(T-1) * sum over c != j of cos(k_j, k_c),
 * cos = 0 when either key is zero -- the LRS reduction over the whole
 * sequence instead of the block.  Every pair is formed (MFMA Gram tiles).
 * block_tables: device int32 [num_reqs][n_blocks], all blocks full (ids
 *               outside the pool read as zero keys).
 * out:          device float [num_reqs][H][T].
 * Rejects T < 2 or T > 8192 and what zp_paged_decode rejects for the cache.
 * ---------------------------------------------------------------------- */
zp_status zp_redundancy_all(const zp_kv_cache* cache, int32_t layer, int32_t num_reqs,
                            const int32_t* block_tables, int32_t n_blocks, float* out,
                            void* stream);

/* ------------------------------------------------------------------------
 * Hybrid scheduler (host object, not thread-safe).
 *
 * Requests below the block cap decode without any extra resource; a request
 * whose next token falls in the observation window [N_max*b - w, N_max*b)
 * needs a query slot (the storage for the queries -- and, with
 * zp_paged_decode_lse, the normalisers -- of its last w tokens) and waits
 * for one when none is free (slots go to the longest-waiting requests
 * first, then the earliest admitted); at the cap it compresses and rejoins decoding
 * in the next step; when blocks run out, running requests are preempted,
 * those without a query slot first (nl page "Technische samenvatting",
 * Methodologie item 2; ko page "기술 요약", section 2.B), the most recently
 * admitted first within each class, never one compressing in the step.  A
 * request that finds no free block waits for the step (blocks given back
 * become allocatable only after the fence below) and preempts one victim,
 * possibly itself, unless blocks given back earlier in the step already
 * cover it.  A preempted request returns its blocks and slot and goes back
 * to the front of the queue to start over (recompute).  Waiting requests
 * are admitted in arrival order while their prompt blocks and max_running
 * allow.
 *
 * Blocks a step gives back (finished or preempted requests) reach reference
 * count 0 but stay pending in the pool until zp_block_pool_fence(), which
 * the caller calls once the GPU work that last read them has completed.
 *
 * Chunked prefill (prefill_chunk > 0; the ko page, section 5, names chunked
 * prefilling as the next step): prompts of any length are written one
 * chunk per step, and a prompt longer than the budget is compressed as its
 * chunks go, so it never holds more than about a chunk past the cap.
 * Between steps a prefilling request's cache ends at or below the window
 * start T - w (T = N_max*b).  From cache position t, the next chunk of
 * c = min(prefill_chunk, rest of the prompt) tokens
 *   - ending at or below T - w is written as it is;
 *   - else, when the rest of the prompt reaches T, is cut or stretched to end
 *     at the block boundary max(T, floor((t + c)/b)*b), and the request
 *     compresses in the same step with n_src = that boundary / b blocks
 *     (zp_compress_n; window = the queries of the chunk's last w tokens),
 *     which leaves (N_max-1)*b cached tokens;
 *   - else (the rest ends inside (T - w, T)) is written whole, its positions
 *     p >= T - w recorded in a query slot (the request waits for a free one)
 *     at row prefill_record_row + p - (T - w), and decode follows.
 * ---------------------------------------------------------------------- */
typedef struct zp_sched zp_sched;

typedef struct zp_sched_config {
  int32_t n_max;           /* block cap per request (N_max) */
  int32_t block_size;      /* b, 16 or 32 */
  int32_t window;          /* w, 1..b */
  int32_t num_query_slots; /* query slots (each holds w rows), >= 1 */
  int32_t max_running;     /* concurrency cap, >= 1 */
  int32_t prefill_chunk;   /* 0: whole prompts at admission (length <= N_max*b - w);
                              else tokens per prefill chunk, a multiple of b */
} zp_sched_config;

/* One step's plan; arrays are owned by the scheduler and valid until the
 * next zp_sched_plan. */
typedef struct zp_sched_step {
  int32_t num_admitted;  /* admitted this step: whole prompt in the request's blocks, or
                            (chunked prefill) its first chunk, listed with the prefills */
  const int64_t* admitted;
  int32_t num_decode;    /* decode one token each, listed longest first: the
                            paged decode starts its workgroups in request
                            order, and a ragged batch finishes sooner when its
                            long requests start first */
  const int64_t* decode_ids;
  const int32_t* decode_slot;        /* physical slot (block*b + offset) of the new token */
  const int32_t* decode_seq_len;     /* length including the new token */
  const int32_t* decode_record_row;  /* query-slot row slot*w + i for window position i, or -1 */
  int32_t num_compress;  /* compress this step (zp_sched_tables, then commit) */
  const int64_t* compress_ids;
  const int32_t* compress_qslot;     /* their query slots, rows slot*w .. slot*w + w-1; -1 after
                                        a prefill chunk (window = the chunk's last w queries) */
  const int32_t* compress_n_src;     /* blocks each holds: N_max at the cap, more after a chunk
                                        (one zp_compress_ex call with these as num_blocks) */
  int32_t num_prefill;   /* prefill chunks of this step (after the decodes, before the
                            compressions of the requests that wrote them) */
  const int64_t* prefill_ids;
  const int32_t* prefill_start;      /* first cache position of the chunk */
  const int32_t* prefill_len;        /* its tokens (prompt tokens prefill_start.. of the cache) */
  const int32_t* prefill_record_row; /* query-slot row of position T - w, or -1 (see above) */
  int32_t num_preempted;
  const int64_t* preempted;
  int32_t num_finished;
  const int64_t* finished;
  int32_t num_released;  /* blocks now pending in the pool (fence after the GPU work) */
} zp_sched_step;

/* Rejects n_max < 2, block_size not in {16,32}, window outside [1, b],
 * num_query_slots < 1, max_running < 1, and a prefill_chunk that is
 * negative, not a multiple of b, or beyond the compression's limits
 * (n_max + prefill_chunk/b <= 512 blocks of at most 8192 tokens,
 * prefill_chunk + 2b <= 1024 evictions per head).  The pool is borrowed: it
 * must outlive the scheduler. */
zp_status zp_sched_create(zp_block_pool* pool, const zp_sched_config* cfg, zp_sched** out);
void zp_sched_destroy(zp_sched* sched);
/* Queue a request; max_new_tokens >= 1; prompt_len >= 1, and without
 * chunked prefill at most N_max*b - w (longer prompts then go through
 * zp_compress_n after their prefill). */
zp_status zp_sched_add(zp_sched* sched, int64_t id, int32_t prompt_len, int32_t max_new_tokens);
/* Plan the next step (see above).  ZP_ERR_STATE if the previous plan's
 * compressions were not committed; ZP_ERR_NO_BLOCKS if a request needs a
 * block and no other request can be preempted. */
zp_status zp_sched_plan(zp_sched* sched, zp_sched_step* out);
/* Block tables (HOST int32 [n][width], width >= n_max, -1 past a request's
 * blocks) and lengths (may be NULL) of the given requests. */
zp_status zp_sched_tables(const zp_sched* sched, const int64_t* ids, int32_t n, int32_t width,
                          int32_t* tables_out, int32_t* seq_lens_out);
/* After the step's compression calls (zp_compress / zp_compress_lse on
 * zp_sched_tables(ids, width = n_max) for the requests at the cap,
 * zp_compress_n on width = n_src for those past it after a prefill chunk,
 * which rewrote those tables): new_tables HOST int32 [num_compress][n_max]
 * in compress_ids order (the first n_max entries of each rewritten row);
 * each request's length becomes (N_max-1)*b and its query slot is free
 * again. */
zp_status zp_sched_compress_commit(zp_sched* sched, const int32_t* new_tables);
zp_status zp_sched_stats(const zp_sched* sched, int32_t* num_waiting, int32_t* num_running,
                         int32_t* free_query_slots);

/* ------------------------------------------------------------------------
 * Prefix index (host object, not thread-safe): full prompt blocks found
 * again by their tokens, so that requests starting with the same tokens
 * share the physical blocks (guide "How it works": shared blocks with
 * reference counts; ko page section 2.C and nl page Methodologie item 3:
 * prefix caching alongside compression).  An entry is one full block of
 * block_size tokens keyed by its tokens and by the entry of the block before
 * it (a block only matches after the same whole prefix); lookups hash and
 * then compare the tokens, so there are no false matches.  The index holds
 * one reference on each block it lists: listed blocks count as shared, so
 * compression never rewrites them in place (it re-targets them).
 * ---------------------------------------------------------------------- */
typedef struct zp_prefix_index zp_prefix_index;

/* The pool is borrowed (it must outlive the index); block_size >= 1. */
zp_status zp_prefix_index_create(zp_block_pool* pool, int32_t block_size, zp_prefix_index** out);
/* Gives back the index's references (blocks reaching 0 become free at
 * once, as with zp_block_release). */
void zp_prefix_index_destroy(zp_prefix_index* index);
/* List the full blocks of a prompt: block n holds tokens [n*b, (n+1)*b)
 * (HOST arrays; only min(num_tokens / b, num_blocks) blocks are full).
 * New entries take a reference on their block; entries already listed for
 * the same prefix are kept (their block wins).  Call it once the prefill
 * has written those blocks, and before any compression of the request.
 * ZP_ERR_INVALID (nothing changed) for ids that are not allocated. */
zp_status zp_prefix_insert(zp_prefix_index* index, const int32_t* tokens, int32_t num_tokens,
                           const int32_t* block_ids, int32_t num_blocks, int32_t* num_added);
/* Longest listed prefix of whole blocks of `tokens`: block_ids_out (HOST,
 * capacity num_tokens / b) gets its blocks, each with a new reference for
 * the caller (release it with zp_block_release), *num_matched their count. */
zp_status zp_prefix_match(zp_prefix_index* index, const int32_t* tokens, int32_t num_tokens,
                          int32_t* block_ids_out, int32_t* num_matched);
/* Drop up to max_entries least-recently-used entries without children,
 * giving back their references; freed_out (HOST, capacity max_entries, may
 * be NULL) gets the blocks that became free, *num_freed their count.  Like
 * zp_block_release, blocks reaching 0 are free at once: the caller
 * guarantees no queued GPU work still reads them. */
zp_status zp_prefix_evict(zp_prefix_index* index, int32_t max_entries, int32_t* freed_out,
                          int32_t* num_freed);
int32_t zp_prefix_size(const zp_prefix_index* index);  /* listed entries */

/* ------------------------------------------------------------------------
 * Debug switches.  The environment sets them when the library first needs
 * them (ZP_TRACE, ZP_DEBUG_POISON, ZP_VALIDATE: any value but "" and "0");
 * zp_set_debug_flags() replaces them at run time (not thread-safe against
 * calls in flight on other threads).
 *   ZP_DEBUG_TRACE     roctx ranges around the host side of every call (the
 *                      plan, each kernel launch), shown by rocprofv3's marker
 *                      trace; the roctx library is loaded on first use and
 *                      tracing stays off without one (zp_trace_available).
 *   ZP_DEBUG_POISON    after every compression, on its stream: NaN into the
 *                      blocks the call frees and into every slot of each
 *                      request's reserved block (all past the new length),
 *                      K and V of every layer, so that any later read of
 *                      stale rows turns outputs NaN.  Slow; checking only.
 *   ZP_DEBUG_VALIDATE  zp_compress_ex with device_tables reads that copy back
 *                      (one host synchronisation with the call's stream) and
 *                      returns ZP_ERR_INVALID, changing nothing, when it
 *                      differs from block_tables.
 * POISON fills with memset nodes and VALIDATE synchronises the host: keep
 * both off for calls made under HIP graph capture.
 * ---------------------------------------------------------------------- */
#define ZP_DEBUG_TRACE 1u
#define ZP_DEBUG_POISON 2u
#define ZP_DEBUG_VALIDATE 4u

uint32_t zp_debug_flags(void);
/* Rejects unknown bits (ZP_ERR_INVALID). */
zp_status zp_set_debug_flags(uint32_t flags);
/* 1 if a roctx library could be loaded (tracing can be shown), else 0. */
int32_t zp_trace_available(void);

/* ------------------------------------------------------------------------
 * Kernel timing.  While enabled, every kernel launch of the calls above is
 * bracketed by HIP events recorded on the caller's stream (a few events per
 * call, no synchronisation).  zp_profile_read() waits for the recorded
 * events, adds up the elapsed time per phase since the last read, and
 * forgets them.  Not thread-safe against concurrent calls of the entry
 * points on other threads.
 * ---------------------------------------------------------------------- */
typedef enum {
  ZP_PHASE_UPLOAD = 0,      /* table / pointer upload of zp_compress */
  ZP_PHASE_SCORE_STATS = 1, /* not used: the statistics pass is inside the scoring kernel */
  ZP_PHASE_SCORE = 2,       /* importance, redundancy, combined score and survivor selection */
  ZP_PHASE_SELECT = 3,      /* not used: the selection is inside the scoring kernel */
  ZP_PHASE_COMPACT = 4,     /* order-preserving gather of K and V */
  ZP_PHASE_APPEND = 5,      /* zp_append_kv */
  ZP_PHASE_DECODE = 6,      /* paged decode attention */
  ZP_PHASE_COMBINE = 7,     /* merge of the decode splits */
  ZP_PHASE_REDUNDANCY_ALL = 8, /* zp_redundancy_all */
  ZP_PHASE_SCORE_COMPACT = 9,  /* scoring, selection and compaction in one kernel */
  ZP_NUM_PHASES = 10
} zp_phase;

zp_status zp_profile_enable(int32_t on);
/* total_ms[ZP_NUM_PHASES], launches[ZP_NUM_PHASES] (either may be NULL). */
zp_status zp_profile_read(double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* ZP_H */
