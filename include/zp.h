/*
 * zp.h - C ABI of the compressed paged KV hot path for AMD Instinct MI355X
 * (gfx950): grouped-query decode attention over block tables, per-token
 * importance scoring, top-k selection with page compaction, and the host
 * block allocator / compression planner.
 *
 * Method: "Zipage: Maintain High Request Concurrency for LLM Reasoning
 * through Compressed PagedAttention" (Liao et al., arXiv 2603.08743), cited
 * below as "Zipage" with section, algorithm, equation or figure.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Plain C types only. Pointers marked [device] must point to GPU memory
 *    the caller owns (the library never allocates or frees device memory);
 *    pointers marked [host] are ordinary host memory.
 *  - GPU calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *    NULL is the null stream). They return after enqueueing work. Argument
 *    validation happens on the host before anything is enqueued: a call that
 *    returns an error has enqueued nothing and changed nothing.
 *  - No exception crosses the ABI. A failing call returns a negative
 *    zp_status and zp_last_error() returns a message for the calling thread.
 *  - Workspaces: every GPU call takes a caller-owned device workspace of at
 *    least the size its *_workspace_size function returns. Its first 256
 *    bytes are a header whose first uint32 collects device-side error bits
 *    (ZP_DEVERR_*). The caller zero-fills a workspace once before first use;
 *    the kernels leave every internal counter at zero when they finish, so a
 *    workspace can be reused by later calls on the same stream. Calls that
 *    share one workspace must not overlap in time.
 *  - Device-side validation: kernels never read or write outside the buffers
 *    the geometry describes. A block id outside [0, num_blocks), a sequence
 *    longer than its table or than the launch bound, or a query slot outside
 *    [0, max_slots) sets a ZP_DEVERR_* bit; the affected outputs are written
 *    as NaN (decode) or left unmodified (scoring, compaction). Read the bits
 *    with zp_workspace_errors().
 *
 * Cache layouts (row-major, innermost last)
 * -----------------------------------------
 *   K, V   [num_layers][num_blocks][num_kv_heads][block_size][head_dim]
 *   Qwin   [num_layers][max_slots][num_kv_heads][g][window][head_dim],
 *          g = num_q_heads / num_kv_heads; query head j belongs to kv-head
 *          j / g (contiguous grouping).
 *   F      [num_layers][num_blocks][num_kv_heads][block_size] float32
 *   Qlse   [num_layers][max_slots][num_kv_heads][g][window] float32
 * These hold the contents Zipage Sec. 3 (K, V), Sec. 4.2 (query cache) and
 * App. C.3 (global score cache F) define; only the axis order differs: one
 * (layer, block, kv-head) slice of K or V is contiguous.
 */
#ifndef ZP_H_
#define ZP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------ */
/* Status                                                                    */
/* ------------------------------------------------------------------------ */

typedef enum zp_status {
  ZP_OK = 0,
  ZP_EINVAL = -1,     /* invalid argument or unsupported geometry            */
  ZP_ENOBLOCKS = -2,  /* not enough free blocks; state unchanged             */
  ZP_EHIP = -3,       /* a HIP runtime call failed                           */
  ZP_ESTATE = -4      /* allocator misuse: double free, refcount underflow   */
} zp_status;

/* Device-side error bits (first uint32 of a workspace). */
#define ZP_DEVERR_BLOCK_ID 0x1u  /* block id outside [0, num_blocks)          */
#define ZP_DEVERR_SEQ_LEN 0x2u   /* sequence longer than its table / launch   */
#define ZP_DEVERR_SLOT 0x4u      /* query slot outside [0, max_slots)         */
#define ZP_DEVERR_KEEP 0x8u      /* keep > resident tokens of a request       */

/* Message of the last failed call on the calling thread ("" if none). */
const char* zp_last_error(void);
const char* zp_version(void);

/* ------------------------------------------------------------------------ */
/* Geometry                                                                  */
/* ------------------------------------------------------------------------ */

typedef enum zp_dtype { ZP_DTYPE_F32 = 0, ZP_DTYPE_BF16 = 1 } zp_dtype;

/* Shapes of the pre-allocated caches (Zipage Sec. 3 and Sec. 4.2).
 * Supported: head_dim in {64, 128}; block_size a power of two in
 * [16, 256]; num_q_heads a multiple of num_kv_heads with g in {1, 2, 4, 8};
 * 1 <= window <= block_size and g * window a multiple of 16, at most 128;
 * n_max >= 2. */
typedef struct zp_geom {
  int32_t num_layers;   /* L                                               */
  int32_t num_blocks;   /* N_total blocks in the pool                      */
  int32_t block_size;   /* b tokens per block                              */
  int32_t num_kv_heads; /* h_kv                                            */
  int32_t num_q_heads;  /* h_q                                             */
  int32_t head_dim;     /* d                                               */
  int32_t window;       /* w, observation window                           */
  int32_t max_slots;    /* M, query-cache slots                            */
  int32_t n_max;        /* N_max, blocks a request keeps after compression */
  int32_t dtype;        /* zp_dtype of K, V, Qwin, q, k/v_new and outputs  */
} zp_geom;

/* Device buffers of the caches, all [device], caller-owned. */
typedef struct zp_cache {
  void* k;         /* K cache                                            */
  void* v;         /* V cache                                            */
  void* qwin;      /* query cache of the observation window              */
  float* gscore;   /* global score cache F, or NULL when it is not used  */
  float* qwin_lse; /* log-sum-exp of each window query's attention row,
                      [num_layers][max_slots][num_kv_heads][g][window]
                      float32 (natural log, scale 1/sqrt(d)), written next
                      to Qwin by the attention calls; NULL when not kept   */
} zp_cache;

/* ------------------------------------------------------------------------ */
/* Decode attention (Zipage Sec. 3 block tables; Sec. 6: eviction leaves the */
/* attention forward an ordinary softmax attention over resident tokens)     */
/* ------------------------------------------------------------------------ */

/* Bytes of workspace zp_paged_decode needs for `batch` rows whose resident
 * lengths are at most `max_seq_len`. */
size_t zp_decode_workspace_size(const zp_geom* geom, int32_t batch, int32_t max_seq_len);

/* One decode step of one layer for `batch` requests.
 *
 * For each row i with n = seq_lens[i] > 0 (n counts the token being decoded):
 *   1. the token's k_new[i], v_new[i] are written to block
 *      block_tables[i*table_stride + (n-1)/b], slot (n-1)%b of layer `layer`;
 *   2. if qslot != NULL, qslot[i] >= 0 and (n-1)%b >= b-w, q[i] is written to
 *      row (n-1)%b-(b-w) of query-cache slot qslot[i] (Zipage Sec. 4.2: the
 *      window is the last w slots of the final block);
 *   3. out[i][j] = sum_t softmax_t(q[i][j] . k_t / sqrt(d)) v_t over the n
 *      resident tokens of kv-head j/g, and lse[i][j] = log sum_t exp(.) if
 *      lse != NULL.
 * Rows with seq_lens[i] <= 0 are skipped (nothing written).
 *
 *   q       [device] [batch][h_q][d] dtype
 *   k_new   [device] [batch][h_kv][d] dtype;  v_new likewise
 *   block_tables [device] int32 [batch][table_stride]
 *   seq_lens     [device] int32 [batch], each <= max_seq_len [host value]
 *   qslot        [device] int32 [batch] or NULL
 *   out     [device] [batch][h_q][d] dtype
 *   lse     [device] float32 [batch][h_q] or NULL
 * Errors: ZP_EINVAL for bad geometry/arguments or a short workspace.
 */
zp_status zp_paged_decode(const zp_geom* geom, const zp_cache* cache, int32_t layer,
                          int32_t batch, const void* q, const void* k_new, const void* v_new,
                          const int32_t* block_tables, int32_t table_stride,
                          const int32_t* seq_lens, int32_t max_seq_len, const int32_t* qslot,
                          void* out, float* lse, void* workspace, size_t workspace_bytes,
                          void* stream);

/* zp_paged_decode without a workspace, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, serving loops and
 * harnesses that forbid allocation. Same arguments, semantics and launch as
 * zp_paged_decode, except:
 *   - the split partials (needed when a small batch of long sequences is
 *     split over several workgroups) live in a static device array of
 *     ZP_DECODE_SCRATCH_BYTES owned by the library; each GPU the library
 *     runs on holds its own copy until the process ends. Nothing is
 *     allocated, by the library or through torch;
 *   - errors [device] uint32, caller-owned, zero-filled by the caller, or
 *     NULL: device-side ZP_DEVERR_* bits are OR-ed into it (dropped if NULL).
 * A call whose partials would exceed ZP_DECODE_SCRATCH_BYTES (zp_decode_
 * workspace_size - 256 bytes) fails with ZP_EINVAL before anything is
 * enqueued. The scratch of a GPU is shared by every call of this function
 * on it and keeps the last call's contents (every partial is written before
 * it is read, so nothing needs clearing): calls that overlap in time on one
 * GPU (different streams, or several host threads) race and must be
 * serialised by the caller. The device address of the array is looked up
 * (hipGetSymbolAddress) on the first call on each device, which can fail
 * with ZP_EHIP. */
#define ZP_DECODE_SCRATCH_BYTES (16 * 1024 * 1024)
zp_status zp_paged_decode_noalloc(const zp_geom* geom, const zp_cache* cache, int32_t layer,
                                  int32_t batch, const void* q, const void* k_new,
                                  const void* v_new, const int32_t* block_tables,
                                  int32_t table_stride, const int32_t* seq_lens,
                                  int32_t max_seq_len, const int32_t* qslot, void* out,
                                  float* lse, uint32_t* errors, void* stream);

/* ------------------------------------------------------------------------ */
/* Prefill attention (Zipage Sec. 3 block tables; Sec. 4.1 the prompt is     */
/* written in full and may exceed N_max blocks until its first compression;  */
/* Sec. 4.2 window queries; Sec. 4.4 a chunk may follow shared prefix        */
/* blocks; Sec. 6 attention is ordinary causal softmax attention)            */
/* ------------------------------------------------------------------------ */

size_t zp_prefill_workspace_size(const zp_geom* geom, int32_t nreq);

/* Causal attention of one layer for a ragged batch of `nreq` prompt chunks.
 *
 * Chunk r has q_len = cu_seqlens[r+1] - cu_seqlens[r] new tokens (rows
 * cu_seqlens[r] .. cu_seqlens[r+1]-1 of q, k_new, v_new, out, lse), which sit
 * at positions ctx_lens[r] .. ctx_lens[r]+q_len-1 of the request: the first
 * ctx_lens[r] tokens (for example shared prefix blocks) are already in the
 * cache. For each new token i at position p:
 *   1. k_new[i], v_new[i] are written to block block_tables[r][p/b], slot p%b;
 *   2. if qslot != NULL, qslot[r] >= 0 and p lies in the block of the
 *      chunk's last token at slot p%b >= b-w, q[i] is written to row
 *      p%b-(b-w) of query-cache slot qslot[r] (Zipage Sec. 4.2), and its
 *      log-sum-exp to cache->qwin_lse if that is not NULL (a negative slot:
 *      a request scheduled without a query slot, nothing is captured);
 *   3. out[i][j] = sum_{t<=p} softmax_t(q[i][j] . k_t / sqrt(d)) v_t over kv-head
 *      j/g, and lse[i][j] = log sum_{t<=p} exp(.) if lse != NULL.
 *
 *   q        [device] [T][h_q][d] dtype,  T = cu_seqlens[nreq]
 *   k_new    [device] [T][h_kv][d] dtype;  v_new likewise
 *   cu_seqlens [device] int32 [nreq+1], non-decreasing, cu_seqlens[0] = 0
 *   ctx_lens   [device] int32 [nreq]
 *   max_q_len  [host] upper bound of every q_len (sets the launch)
 *   block_tables [device] int32 [nreq][table_stride], covering ctx + q_len tokens
 *   qslot      [device] int32 [nreq] or NULL
 *   out        [device] [T][h_q][d] dtype;  lse [device] float32 [T][h_q] or NULL
 * Chunks whose geometry does not fit (q_len > max_q_len, ctx + q_len beyond
 * the table) set ZP_DEVERR_SEQ_LEN and are skipped. bf16 runs on MFMA
 * (tiles of 128/g tokens, all g heads of a kv-head per workgroup); fp32 runs
 * one workgroup per token.
 */
zp_status zp_paged_prefill(const zp_geom* geom, const zp_cache* cache, int32_t layer,
                           int32_t nreq, const void* q, const void* k_new, const void* v_new,
                           const int32_t* cu_seqlens, const int32_t* ctx_lens, int32_t max_q_len,
                           const int32_t* block_tables, int32_t table_stride,
                           const int32_t* qslot, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Importance scores (Zipage Sec. 4.2; App. C.2 Alg. 1, C.3 Alg. 2, C.4,     */
/* C.5 eq. (4), C.7 lightning redundancy, C.8 tempered softmax)              */
/* ------------------------------------------------------------------------ */

#define ZP_SCORE_GLOBAL 0x1u          /* decayed global score (Alg. 2)            */
#define ZP_SCORE_POOL 0x2u            /* max pooling along the sequence (eq. (3)) */
#define ZP_SCORE_POOL_FIRST_ONLY 0x4u /* pool only at a request's first compression */
#define ZP_SCORE_REDUNDANCY 0x8u      /* key redundancy, S - lambda R (lightning) */
#define ZP_SCORE_REDUNDANCY_FLASH 0x10u /* with ZP_SCORE_REDUNDANCY: similarities over the
                                           whole sequence (Zipage Alg. 3) instead of within
                                           each block (App. C.7); ignored without
                                           ZP_SCORE_REDUNDANCY. Needs 2*b*d*sizeof(elem)
                                           + 56*b bytes of LDS (<= 160 KiB), which
                                           holds wherever scoring itself fits        */
#define ZP_SCORE_GLOBAL_SUM 0x20u     /* with ZP_SCORE_GLOBAL: decayed sum-reduce,
                                         alpha*F + S, instead of Alg. 2's
                                         max(alpha*F, S) (App. C.3 names both);
                                         invalid without ZP_SCORE_GLOBAL             */
#define ZP_SCORE_WINDOW_LSE_ALL 0x40u /* every request's window rows carry their
                                         log-sum-exp in cache->qwin_lse, as if
                                         window_lse_valid[r] != 0 for all r (the
                                         array is then not read and may be NULL); the
                                         statistics pass is not launched at all.
                                         Needs cache->qwin_lse                       */

typedef struct zp_score_params {
  float alpha;         /* decay of the global score                          */
  float lambda_;       /* weight of the redundancy score                     */
  float tau;           /* softmax temperature of the redundancy score (> 0)  */
  float sim_threshold; /* p: cosine above which the last entry per column is
                          zeroed; must be >= 0                               */
  int32_t pool_kernel; /* odd pooling width >= 1                             */
  uint32_t flags;      /* ZP_SCORE_* bits                                    */
} zp_score_params;

size_t zp_score_workspace_size(const zp_geom* geom, int32_t layer_count, int32_t nreq,
                               int32_t max_blocks);

/* Final per-token scores of `nreq` requests whose blocks are all full, for
 * layers [layer_begin, layer_begin + layer_count) (the layer stride of
 * Zipage App. C.1) and every kv-head. For request r with N = num_blocks[r]
 * blocks (n = N*b tokens, N <= max_blocks) and window queries in query-cache
 * slot qslot[r]:
 *   S0 = mean over the window of the max over the g query heads of
 *        softmax_t(q.k_t/sqrt(d)), the last block causally masked;
 *   S1 = global score (when ZP_SCORE_GLOBAL; first_compression[r] != 0
 *        means the request was never compressed): on every block but the
 *        last, max(alpha*F, S0), or alpha*F + S0 with ZP_SCORE_GLOBAL_SUM;
 *        the cache's F is only read,
 *        the updated history (Alg. 2's new F, which equals S1) goes to f_new,
 *        and zp_select_compact moves it into the target blocks, so blocks
 *        shared between requests are never written;
 *   S2 = max-pooled S1 (when ZP_SCORE_POOL, and first_compression[r] if
 *        ZP_SCORE_POOL_FIRST_ONLY);
 *   S3 = S2 - lambda * softmax_t(r_t / n / tau), r_t the lightning row sums
 *        (or, with ZP_SCORE_REDUNDANCY_FLASH, the flash row sums over the
 *        whole sequence), when ZP_SCORE_REDUNDANCY;
 *   scores = S3 with +inf on the last w positions.
 *
 *   block_tables [device] int32 [nreq][table_stride]
 *   num_blocks   [device] int32 [nreq];  qslot [device] int32 [nreq]
 *   first_compression [device] uint8 [nreq]
 *   window_lse_valid  [device] uint8 [nreq] or NULL: nonzero when every
 *          window row of request r has its log-sum-exp in cache->qwin_lse
 *          (zp_paged_decode and zp_paged_prefill write it next to each
 *          window query they capture; the attention of a window query
 *          already covered exactly its causal row of Alg. 1). Those
 *          requests skip the pass that gathers the softmax statistics, and
 *          their keys are read once. Needs cache->qwin_lse.
 *   scores [device] float32 [layer_count][nreq][h_kv][scores_stride],
 *          scores_stride >= max_blocks*b; entries past n are not written.
 *   f_new  [device] float32, same layout as scores: S1 of every token; may be
 *          NULL when ZP_SCORE_GLOBAL is off.
 */
zp_status zp_score_tokens(const zp_geom* geom, const zp_cache* cache,
                          const zp_score_params* params, int32_t layer_begin,
                          int32_t layer_count, int32_t nreq, const int32_t* block_tables,
                          int32_t table_stride, const int32_t* num_blocks, int32_t max_blocks,
                          const int32_t* qslot, const uint8_t* first_compression,
                          const uint8_t* window_lse_valid, float* scores, float* f_new,
                          int64_t scores_stride, void* workspace, size_t workspace_bytes,
                          void* stream);

/* ------------------------------------------------------------------------ */
/* Top-k selection and compaction (Zipage Sec. 4.2, App. C.6 Alg. 4,         */
/* Sec. 4.4 target blocks)                                                   */
/* ------------------------------------------------------------------------ */

#define ZP_SELECT_NO_COMPACT 0x1u /* only select; leave K, V, F untouched */

/* Workspace bytes of zp_select_compact for `keep` kept tokens per (layer,
 * request, kv-head): error bits, per-item status and the kept indices. */
size_t zp_select_workspace_size(const zp_geom* geom, int32_t layer_count, int32_t nreq,
                                int32_t keep);

/* For every (layer, request, kv-head): keep the `keep` tokens with the
 * highest score (ties go to the higher token index), and move their K, V and
 * (if cache->gscore != NULL) global-score entries, in ascending token order,
 * to logical slots 0..keep-1 of the target blocks dst_tables[r][0..]. The
 * global score written for kept token t is f_new[t] (zp_score_tokens'
 * updated history) when f_new != NULL, else the cache's own F value of t.
 * keep is normally (N_max - 1) * b. kept_idx, if not NULL, receives the
 * ascending token indices.
 *
 * Precondition (in-place safety): each target block dst_tables[r][i] is
 * either src_tables[r][i] or a block that src_tables[r] does not contain.
 * zp_plan_compress produces targets of this form.
 *
 *   scores, f_new [device] float32 [layer_count][nreq][h_kv][scores_stride]
 *   src_tables [device] int32 [nreq][src_stride]; num_blocks [device] int32 [nreq]
 *   dst_tables [device] int32 [nreq][dst_stride], dst_stride*b >= keep
 *   kept_idx [device] int32 [layer_count][nreq][h_kv][keep] or NULL
 * keep must be in [1, 8192].
 */
zp_status zp_select_compact(const zp_geom* geom, const zp_cache* cache, int32_t layer_begin,
                            int32_t layer_count, int32_t nreq, const float* scores,
                            const float* f_new, int64_t scores_stride,
                            const int32_t* src_tables, int32_t src_stride,
                            const int32_t* num_blocks, int32_t max_blocks,
                            const int32_t* dst_tables, int32_t dst_stride, int32_t keep,
                            int32_t* kept_idx, uint32_t flags, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Waits for `stream`, then copies the workspace's device error bits to
 * *flags [host]. */
zp_status zp_workspace_errors(const void* workspace, uint32_t* flags, void* stream);
/* Clears the workspace's device error bits (enqueued on `stream`). */
zp_status zp_workspace_clear_errors(void* workspace, void* stream);

/* ------------------------------------------------------------------------ */
/* Host block allocator and compression planner (Zipage Sec. 3, Sec. 4.1,    */
/* Sec. 4.4). Host-only; one handle is not thread-safe (callers serialise,   */
/* like a single scheduler).                                                 */
/* ------------------------------------------------------------------------ */

typedef struct zp_alloc zp_alloc;

/* Pool of block ids 0..num_blocks-1, all free. NULL on bad size. */
zp_alloc* zp_alloc_create(int32_t num_blocks);
void zp_alloc_destroy(zp_alloc* a);

/* Takes n free blocks (refcount 1) into ids[0..n) [host], lowest ids first.
 * All or nothing: ZP_ENOBLOCKS leaves the pool unchanged. */
zp_status zp_block_alloc(zp_alloc* a, int32_t n, int32_t* ids);
/* Drops one reference of each listed block; a block whose count reaches 0
 * returns to the pool. ZP_ESTATE (state unchanged) if any listed block is
 * already free or would be released twice by this call. */
zp_status zp_block_free(zp_alloc* a, const int32_t* ids, int32_t n);
/* Adds one reference to each listed (allocated) block: prefix sharing. */
zp_status zp_block_share(zp_alloc* a, const int32_t* ids, int32_t n);
/* Reference count of a block (0 = free), or -1 for an id out of range. */
int32_t zp_block_refcount(const zp_alloc* a, int32_t id);
int32_t zp_num_free(const zp_alloc* a);
int32_t zp_num_blocks(const zp_alloc* a);

/* Plans one compression of a request holding table[0..n_blocks) [host]
 * (n_blocks >= n_max >= 2). Blocks with refcount > 1 are shared and must form
 * a prefix of the table. Target rule (Zipage Sec. 4.4): with N_prefix shared
 * blocks, if N_prefix >= n_max-1 all n_max-1 targets are new blocks, else the
 * shared positions get new blocks and the other positions keep the request's
 * own blocks; new blocks take the logical positions of the shared ones. The
 * reserved n_max-th block (Sec. 4.1) is the first own block not used as a
 * target, or a new block if there is none. Fresh blocks are allocated here,
 * all or nothing (ZP_ENOBLOCKS leaves everything unchanged: the request
 * stays uncompressed and the caller must wait or preempt).
 *   dst_table [host] int32 [n_max-1]  targets for zp_select_compact
 *   new_table [host] int32 [n_max]    table after the compression
 *   release   [host] int32 [n_blocks] own blocks that commit will free
 *   n_release [host] their count */
zp_status zp_plan_compress(zp_alloc* a, const int32_t* table, int32_t n_blocks, int32_t n_max,
                           int32_t* dst_table, int32_t* new_table, int32_t* release,
                           int32_t* n_release);
/* Finishes a planned compression once its compaction has completed on the
 * GPU: every block of old_table that is not in new_table loses one reference
 * (shared blocks drop by one, released own blocks return to the pool). */
zp_status zp_commit_compress(zp_alloc* a, const int32_t* old_table, int32_t n_blocks,
                             const int32_t* new_table, int32_t n_max);
/* Abandons a planned compression: frees the fresh blocks of new_table (those
 * not in old_table); the request keeps old_table. */
zp_status zp_abort_compress(zp_alloc* a, const int32_t* old_table, int32_t n_blocks,
                            const int32_t* new_table, int32_t n_max);

/* Capacity (Zipage Sec. 4.2 eq. (1); App. C.3 eq. (2)): with m_blk = m_kv +
 * m_f bytes per block (m_f = global-score bytes per block, 0 if unused) and
 * m_q query-cache bytes per request,
 *   M = floor(m_avail / (m_blk*n_max + m_q)),
 *   N_total = floor(m_avail / (m_blk + m_q/n_max)). */
zp_status zp_capacity(int64_t m_avail, int64_t m_kv, int64_t m_f, int64_t m_q, int32_t n_max,
                      int64_t* max_concurrency, int64_t* num_blocks);

/* ------------------------------------------------------------------------ */
/* Request scheduler (Zipage Sec. 4.3 constrained and hybrid scheduling,     */
/* Fig. 2; Sec. 4.4 shared prefixes and their preemption rule). Host-only,   */
/* deterministic, not thread-safe. It owns a block pool of num_blocks ids    */
/* and M = num_slots query-cache slots, and decides, step by step, which     */
/* requests are prefilled or decoded, which are compressed (with their       */
/* source and target tables) and which are preempted.                        */
/*                                                                           */
/* Policy, in the order one zp_sched_step applies it:                        */
/*  (a) requests that became due in an earlier step (n = N b tokens,         */
/*      N >= n_max, Sec. 4.1) get their compression planned with             */
/*      zp_plan_compress's target rule; if fresh targets cannot be allocated */
/*      (shared prefixes only) victims are preempted per (e), else it waits. */
/*      Compressions are listed in the step output and must run after the    */
/*      kernels of earlier steps and before those of this step;             */
/*  (b) free slots go to the foremost slot-less requests among the first M   */
/*      of the running queue (hybrid rules 1 and 3);                         */
/*  (c) admission, first come first served: the head of the waiting queue is */
/*      prefilled if its prompt (plus outputs, after a preemption) fits the  */
/*      free blocks; with a slot if fewer than M requests run, else (hybrid  */
/*      only) without one if its last prompt position needs no slot;         */
/*      admission stops at the first request that does not fit. If any is   */
/*      admitted, the step is a prefill step;                                */
/*  (d) otherwise every running request that is neither compressing nor due  */
/*      decodes one token, except a slot-less request whose next position    */
/*      needs a slot (position p needs one iff p / b >= n_max - 1 and        */
/*      p % b >= b - w: its query belongs to the window of a block whose end */
/*      can trigger a compression; hybrid rule 2), and a request that needs  */
/*      a new block while none is free and no victim remains (it waits:      */
/*      constrained scheduling);                                             */
/*  (e) victims of a block shortage, one at a time from the back of the      */
/*      running queue: with prefix_sharing, the last request never           */
/*      compressed and not being compressed (Sec. 4.4); otherwise, hybrid,   */
/*      the last request without a slot (hybrid rule 4); constrained, none.  */
/*      A preempted request frees its blocks and slot and goes to the front  */
/*      of the waiting queue keeping its outputs (it is prefilled again over */
/*      prompt + outputs).                                                   */
/* Token accounting: a prefill produces one output token, each decode step   */
/* appends the previous output token's K/V and produces one; a request       */
/* finishes after max_new outputs and its blocks and slot are freed at once. */
/* Shared prefixes: requests of one prefix group share their first           */
/* prefix_len / b blocks, written by the first member admitted; members      */
/* admitted in a later step take a reference and prefill only the rest       */
/* (ctx > 0). A member stops holding the prefix when its compression is      */
/* planned, when it finishes or when it is preempted. Block, slot and row    */
/* ids are always taken lowest first.                                        */
/* ------------------------------------------------------------------------ */

typedef struct zp_sched zp_sched;

enum { ZP_SCHED_CONSTRAINED = 0, ZP_SCHED_HYBRID = 1 };
enum { ZP_STEP_IDLE = 0, ZP_STEP_PREFILL = 1, ZP_STEP_DECODE = 2 };
enum { ZP_REQ_WAITING = 0, ZP_REQ_RUNNING = 1, ZP_REQ_COMPRESSING = 2, ZP_REQ_FINISHED = 3,
       ZP_REQ_UNKNOWN = -1 };

typedef struct {
  int32_t num_blocks;          /* block pool size */
  int32_t block_size;          /* b, a power of two */
  int32_t window;              /* w, 1..b */
  int32_t n_max;               /* N_max >= 2: the default and largest per-request cap */
  int32_t num_slots;           /* M, query-cache slots, >= 1 */
  int32_t max_running;         /* largest running queue (and batch), >= 1 */
  int32_t max_prefill_tokens;  /* tokens of one prefill step (a longer first request still runs alone) */
  int32_t table_cap;           /* largest block table, >= n_max */
  int32_t policy;              /* ZP_SCHED_CONSTRAINED or ZP_SCHED_HYBRID */
  int32_t prefix_sharing;      /* nonzero: share prefix blocks, preemption rule of Sec. 4.4 */
  int32_t nmax_growth;         /* adaptive N_max, tokens per extra block (0 = off); see
                                  zp_sched_add */
} zp_sched_config;

/* Output of one step. The caller provides every array with the capacity
 * noted (R = max_running, C = table_cap); the step fills the counts.
 * Batch entries (n of them) are in running-queue order:
 *   rid, slot (-1 = none), ctx (tokens resident before the entry's tokens),
 *   pos (index of the entry's first token in the request's token sequence,
 *   e.g. for position encodings; equal to ctx until the first compression),
 *   len (prefill: tokens to write, decode: 1), tables [R][C] (entry i's
 *   block table in row i, -1 beyond its length). A prefill entry writes
 *   cache positions ctx..ctx+len-1; a decode entry writes cache position
 *   ctx and attends over ctx + 1 tokens.
 * Compressions (n_comp): c_rid, c_slot, c_first (1 = first compression of
 *   the request), c_nblocks (source table length), c_nmax (the request's
 *   N_max: keep (c_nmax - 1) * b tokens), c_src [R][C] (-1 padded),
 *   c_dst [R][n_max-1] and c_new [R][n_max] (c_nmax - 1 and c_nmax entries,
 *   -1 padded).
 * finished / preempted: request ids (n_finished / n_preempted, <= R each).
 * n_blocked: requests that could not decode this step (slot or block wait). */
typedef struct {
  int32_t* rid;
  int32_t* slot;
  int32_t* ctx;
  int32_t* pos;
  int32_t* len;
  int32_t* tables;
  int32_t* c_rid;
  int32_t* c_slot;
  int32_t* c_first;
  int32_t* c_nblocks;
  int32_t* c_nmax;
  int32_t* c_src;
  int32_t* c_dst;
  int32_t* c_new;
  int32_t* finished;
  int32_t* preempted;
  int32_t kind;       /* ZP_STEP_* */
  int32_t n;
  int32_t n_comp;
  int32_t n_finished;
  int32_t n_preempted;
  int32_t n_blocked;
} zp_sched_step_out;

typedef struct {
  int64_t steps, prefill_steps, decode_steps, idle_steps;
  int64_t waiting, running, compressing, finished;
  int64_t free_blocks, slots_in_use;
  int64_t prefill_tokens, decode_tokens, compressions, preemptions, blocked;
} zp_sched_stats;

typedef struct {
  int32_t state;       /* ZP_REQ_* */
  int32_t n;           /* resident tokens */
  int32_t gen;         /* outputs produced */
  int32_t slot;        /* -1 = none */
  int32_t compressed;  /* 1 once a compression has committed */
  int32_t ntable;      /* block table length */
  int32_t n_max;       /* its N_max now (grows with nmax_growth) */
} zp_sched_req_info;

/* NULL (with zp_last_error) on an invalid configuration. */
zp_sched* zp_sched_create(const zp_sched_config* cfg);
void zp_sched_destroy(zp_sched* s);
/* Queues a request at the back of the waiting queue. prefix_group < 0: no
 * shared prefix; else 0 <= prefix_len < prompt_len, one prefix_len per group.
 * n_max: this request's N_max in [2, cfg.n_max], 0 for cfg.n_max (Zipage
 * names a per-request N_max, set from the request's expected length, as a
 * way to trade concurrency for quality; the choice is the caller's). Every
 * rule above uses the request's own N_max, and a slot is given only while
 * the N_max of all slot holders sums to at most num_blocks (the
 * per-request form of M <= N_total / N_max, Sec. 4.2; with one N_max and a
 * pool sized by that rule it never binds).
 * Adaptive N_max (cfg.nmax_growth = A > 0; Zipage, Limitations: N_max set
 * per request from its actual sequence length): after each step of a
 * request, its N_max becomes max(current, min(cfg.n_max, n_max_added +
 * floor(L / A))) with L = prompt_len + outputs so far, before the trigger
 * check; a slot holder's raise is cut to what keeps the holders' sum within
 * num_blocks (the remainder is taken at a later step). Compressions report
 * the N_max they keep (c_nmax).
 * ZP_EINVAL for a repeated rid, bad lengths or n_max, or a prompt longer
 * than table_cap blocks. */
zp_status zp_sched_add(zp_sched* s, int32_t rid, int32_t prompt_len, int32_t max_new,
                       int32_t prefix_group, int32_t prefix_len, int32_t n_max);
/* One scheduling step (policy above). ZP_ESTATE if a table would exceed
 * table_cap: the scheduler is then unusable and must be destroyed. */
zp_status zp_sched_step(zp_sched* s, zp_sched_step_out* out);
/* The compaction of request rid (listed by an earlier step) has completed:
 * its table becomes c_new, blocks it no longer lists lose its reference, it
 * holds (n_max - 1) b tokens and decodes again. ZP_ESTATE if rid is not
 * compressing. */
zp_status zp_sched_compress_done(zp_sched* s, int32_t rid);
zp_status zp_sched_get_stats(const zp_sched* s, zp_sched_stats* out);
/* State of request rid; table [host] (capacity table_cap) may be NULL. An
 * unknown rid gives state ZP_REQ_UNKNOWN. */
zp_status zp_sched_request(const zp_sched* s, int32_t rid, zp_sched_req_info* info,
                           int32_t* table);
/* Requests not finished yet. */
int32_t zp_sched_unfinished(const zp_sched* s);
/* The scheduler's block pool (read-only use: refcounts, free count). */
const zp_alloc* zp_sched_allocator(const zp_sched* s);

#ifdef __cplusplus
}
#endif

#endif /* ZP_H_ */
