/*
 * sparse_decode.h -- C ABI of libsparse_decode.so: top-k sparse decode
 * attention over a paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * One decode step, for every request b (one decode query per request):
 *   1. score every cached token t < kv_lens[b] from the paged K pool through
 *      the request's block table, one score per (request, KV head);
 *   2. keep the top-k token positions per (request, KV head), highest score
 *      first, lowest position first among equal scores;
 *   3. gather only the kept K/V rows and run softmax attention of every query
 *      head over its KV head's kept rows.
 *
 * Sources (page title and section of the pages this library follows):
 *   - "Add TriAttention KV-cache compression method" (TensorRT-LLM PR 16957),
 *     Summary and Key Design Decisions: score paged K directly through a
 *     batched page-table snapshot, per-head reduction, TopK with deterministic
 *     tie settlement, score scratch reused at a high-water mark.
 *   - "Overlap DSA heuristic prev_topk write-back on the aux stream"
 *     (TensorRT-LLM PR 16666), Description: the DSA indexer produces each
 *     decode step's top-k into a persistent buffer, which core sparse
 *     attention then consumes.
 *   - "Unify sparse attention framework with clean backend interfaces"
 *     (TensorRT-LLM PR 12733), Dev Engineer Review and Description: indices
 *     travel to the attention op with per-request lengths; global index
 *     conversion through block_table invalidates negative positions and
 *     out-of-range pages; buffers keep a stable address for graph capture.
 *   - "Add DSA Vanilla sparse attention" (TensorRT-LLM PR 16309),
 *     Walkthrough: selected-token attention over request-local selections,
 *     MLA latent rows read from a paged cache.
 *   - "Compact pseudo-KV/topological sparse attention benchmark evidence and
 *     backend gap" (TensorRT-LLM issue 15989), Misc discussion: a typed,
 *     fixed call shape, not a generic keyword carrier.
 *
 * Conventions shared by every entry point:
 *   - Pointers named "device" are HIP device memory owned by the caller; the
 *     library never allocates, frees, synchronizes or keeps state between
 *     calls, so calls may be captured into a HIP graph.  All work is enqueued
 *     on `stream` and runs asynchronously.
 *   - Pool element offsets are 64-bit: row (page p, KV head g, slot s) starts
 *     at element p*page_stride + g*head_stride + s*token_stride, and its
 *     head_dim elements are contiguous.  Rows must start on 16-byte boundaries.
 *   - Query head h belongs to KV head h / (q_heads / num_kv_heads).
 *   - Token t of request b lives in page block_table[b*max_pages + t/page_size]
 *     at slot t % page_size.  Device-side values cannot be checked on the host:
 *     kv_lens[b] is clamped to [0, min(max_kv_len, max_pages*page_size)], and a
 *     token whose page id is outside [0, num_pages) is treated as absent (it
 *     scores -inf, is never kept, and contributes nothing to attention).
 *   - bfloat16 data is passed as raw 16-bit patterns (SD_BF16).
 *   - SD_FP8_E4M3 pools (indexer K only) hold OCP FP8 E4M3 byte codes (sign,
 *     4 exponent bits with bias 7, 3 mantissa bits; no infinities, codes 0x7F
 *     and 0xFF are NaN, largest finite 448) plus one binary32 scale per row:
 *     row (page p, KV head g, slot s) stands for decode(code) * scale[(p *
 *     num_kv_heads + g) * page_size + s] ("Overlap DSA heuristic prev_topk
 *     write-back on the aux stream", Test Coverage: the block-scaled FP8
 *     indexer cache).
 *   - Every entry point validates its host-visible arguments first and
 *     returns a non-SD_OK status without enqueuing anything when they are
 *     wrong; sd_last_error() then names the argument.  No exception crosses
 *     the ABI.  A failed HIP launch returns SD_ERR_HIP.
 */
#ifndef SPARSE_DECODE_H
#define SPARSE_DECODE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SD_VERSION 2

typedef enum sd_status {
  SD_OK = 0,
  SD_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size or alignment          */
  SD_ERR_UNSUPPORTED = 2,      /* valid request the library has no kernel for */
  SD_ERR_WORKSPACE_TOO_SMALL = 3,
  SD_ERR_HIP = 4               /* a HIP launch or runtime call failed          */
} sd_status;

typedef enum sd_dtype { SD_F32 = 0, SD_BF16 = 1, SD_FP8_E4M3 = 2 } sd_dtype;

/* How the per-head dot products of one KV head's query heads become one
 * token score ("Add TriAttention ...", Summary: per-head reduction; the DSA
 * indexer of "Overlap DSA heuristic prev_topk write-back ...", Description).
 * dot_h = q_h . k_t accumulated in binary32; G = query heads per KV head. */
typedef enum sd_score_mode {
  SD_SCORE_GROUP_SUM = 0,     /* s = sum_h (dot_h * head_scale)                 */
  SD_SCORE_GROUP_MEAN = 1,    /* s = (sum_h dot_h) * (1/G)                      */
  SD_SCORE_RELU_WEIGHTED = 2  /* s = sum_h (w_h * max(dot_h, 0)): DSA indexer   */
} sd_score_mode;

/* SD_SCORE_EXACT computes every score with one fixed binary32 evaluation
 * order: each dot product left to right over the head dimension (each
 * product and each sum rounded once, no fused multiply-add), then the sum
 * over the group's heads left to right in head order, with the mode's scale
 * applied as written above.  Two calls, or this library and any other
 * implementation of that order, agree bit for bit.
 * An SD_FP8_E4M3 pool is scored as the binary32 pool of its dequantized
 * rows: each element is decoded and multiplied by its row scale (one
 * rounding), then the dot products follow the same order with every product
 * rounded once.
 * SD_SCORE_FAST may evaluate in another order (bf16 matrix cores for the
 * DSA mode) and reports a per-row bound on its distance from the exact score.
 * Modes without a fast kernel compute the exact scores in both settings. */
typedef enum sd_score_precision { SD_SCORE_EXACT = 0, SD_SCORE_FAST = 1 } sd_score_precision;

/* A paged pool (K, V, MLA latent or indexer K). */
typedef struct sd_pool {
  const void* data;        /* device                                           */
  sd_dtype dtype;
  int32_t num_pages;
  int32_t page_size;       /* tokens per page                                  */
  int32_t num_kv_heads;
  int32_t head_dim;        /* elements per row                                 */
  int64_t page_stride;     /* elements                                         */
  int64_t head_stride;     /* elements                                         */
  int64_t token_stride;    /* elements                                         */
  const float* scale;      /* SD_FP8_E4M3 only (else NULL): device row scales  */
                           /* [num_pages][num_kv_heads][page_size], contiguous */
} sd_pool;

/* The batch's page tables ("Add TriAttention ...", Key Design Decisions: a
 * batched page-table snapshot read directly by the scorer). */
typedef struct sd_pages {
  const int32_t* block_table; /* device [batch][max_pages]                     */
  const int32_t* kv_lens;     /* device [batch]                                */
  int32_t batch;
  int32_t max_pages;          /* row length of block_table                     */
  int32_t max_kv_len;         /* host bound on kv_lens; row length of scores   */
} sd_pages;

/* ------------------------------------------------------------------ step 1 */

/* Score every token t < kv_len of every (request, KV head) of k_pool.
 *   q            device [batch][q_heads][k_pool->head_dim], dtype q_dtype
 *                (must equal k_pool->dtype; SD_BF16 for an SD_FP8_E4M3 pool)
 *   head_weights device [batch][q_heads] float, RELU_WEIGHTED only (else NULL)
 *   head_scale   GROUP_SUM factor (ignored by the other modes)
 *   scores       device [batch][num_kv_heads][max_kv_len] float; entries at
 *                t >= kv_len (and absent tokens) are set to -inf
 *   row_bound    device [batch][num_kv_heads] float or NULL, caller-initialised
 *                (normally to 0).  SD_SCORE_FAST raises each entry to at
 *                least d >= 0 with |scores[t] - exact score(t)| <= d for
 *                every t < kv_len of the row (a max into the existing value,
 *                so one zero fill serves any number of calls on the same
 *                inputs); SD_SCORE_EXACT leaves it unchanged.
 * Follows "Add TriAttention ...", Key Design Decisions (direct paged-pool
 * scoring) and, for RELU_WEIGHTED, the DSA indexer of "Overlap DSA heuristic
 * prev_topk write-back ...", Description. */
sd_status sd_sparse_score_paged(const sd_pages* pages, const sd_pool* k_pool, const void* q,
                                sd_dtype q_dtype, int32_t q_heads, const float* head_weights,
                                sd_score_mode mode, float head_scale,
                                sd_score_precision precision, float* scores, float* row_bound,
                                hipStream_t stream);

/* ------------------------------------------------------------------ step 2 */

/* Top-k per row: the min(k, kv_len) positions t < kv_lens[b] that come first
 * in (score descending, position ascending) order ("Add TriAttention ...",
 * Summary and Test Plan: TopK with deterministic heavy-tie settlement).  A row
 * with kv_len <= k keeps every token (dense-equivalent).  -0 and +0 compare
 * equal; NaN scores inside kv_len are outside the contract.
 *   scores  device [batch][groups][row_stride] float
 *   indices device [batch][groups][k] int32: kept positions in ascending
 *           order, then -1 padding
 *   counts  device [batch][groups] int32 (number kept), or NULL
 *   workspace device, at least sd_topk_workspace_size() bytes (may be NULL
 *           when that size is 0). */
sd_status sd_topk_workspace_size(int32_t batch, int32_t groups, int32_t row_stride, int32_t k,
                                 size_t* bytes);
sd_status sd_topk_select(const float* scores, int32_t batch, int32_t groups, int32_t row_stride,
                         const int32_t* kv_lens, int32_t k, int32_t* indices, int32_t* counts,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Top-k with a previous step's selection as a hint, and its write-back ("Overlap
 * DSA heuristic prev_topk write-back on the aux stream", Description: each
 * decode step's top-k is written back as the next step's hint).  The result
 * is exactly sd_topk_select's for any hint contents: the hint only narrows
 * the search.  A hint entry counts when it is a position in [0, kv_len)
 * larger than every counted entry before it (an ascending hint, as the
 * write-back produces, counts in full); when at least k entries of a row
 * count, the smallest of their scores is a floor under the k-th largest and
 * no token below it is examined further.  A row whose hint certifies
 * nothing is selected without a floor.
 *   hint       device [batch][groups][hint_stride] int32 request-local
 *              positions (may be NULL: no hint); the first hint_len of each
 *              row are read (hint_stride >= hint_len >= 0)
 *   writeback  device [batch][groups][writeback_stride] int32 or NULL: gets
 *              the same k entries as indices (writeback_stride >= k), from
 *              the same kernel stores.  It may be the hint buffer itself:
 *              the hint is read completely before any write-back store.
 * Other arguments, workspace and errors as sd_topk_select. */
sd_status sd_topk_select_hinted(const float* scores, int32_t batch, int32_t groups, int32_t row_stride,
                                const int32_t* kv_lens, int32_t k, const int32_t* hint, int32_t hint_len,
                                int64_t hint_stride, int32_t* indices, int32_t* counts,
                                int32_t* writeback, int64_t writeback_stride, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ modes */

/* TriAttention selection modes ("Add TriAttention KV-cache compression
 * method", Summary: normalize/reduce before TopK / tie settlement; union,
 * per_head and per_layer_perhead eviction modes; Main Files: score
 * normalization and union reduction).  The pages give no formula; the
 * library's evaluation, bit-identical on every call:
 *   per member row (layer l, request b, KV head g), over its finite scores
 *   at t < kv_len[b] (n of them), binary64 statistics summed in a fixed
 *   order -- 256 partials P_c over t % 256 == c (t ascending), then
 *   P_0..P_255 in order -- mu = sum / n, var = (the same sums of
 *   ((double)s_t - mu)^2) / n, and z_t = (float)(((double)s_t - mu) /
 *   sqrt(var)) (0 when var == 0; -inf for a non-finite score or t >= kv_len);
 *   reduced row r_t = max of z_t over the mode's members (layers, then
 *   heads, ascending; a later member wins only when strictly larger);
 *   then the top-k of sd_topk_select on each reduced row. */
typedef enum sd_select_mode {
  SD_SELECT_PER_LAYER_PERHEAD = 0, /* one row per (layer, b, g): its own z      */
  SD_SELECT_PER_HEAD = 1,          /* one row per (b, g): max over layers       */
  SD_SELECT_UNION = 2              /* one row per b: max over layers and heads  */
} sd_select_mode;

/*   scores      device [layers][batch][groups][row_stride] float (the
 *               scorer's output for each layer, stacked)
 *   indices     device [out_rows][k] int32, out_rows = layers*batch*groups,
 *               batch*groups or batch by mode; ascending, -1 padded
 *   counts      device [out_rows] int32 or NULL
 *   reduced_out device [out_rows][row_stride] float or NULL: the reduced rows
 *   workspace   device, at least sd_triattention_select_workspace_size() bytes
 * NaN scores inside kv_len are outside the contract. */
sd_status sd_triattention_select_workspace_size(int32_t layers, int32_t batch, int32_t groups,
                                                int32_t row_stride, sd_select_mode mode, int32_t k,
                                                size_t* bytes);
sd_status sd_triattention_select(const float* scores, int32_t layers, int32_t batch, int32_t groups,
                                 int32_t row_stride, const int32_t* kv_lens, sd_select_mode mode,
                                 int32_t k, int32_t* indices, int32_t* counts, float* reduced_out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ step 3 */

/* Softmax attention of every query head over its KV head's selected rows
 * ("Add DSA Vanilla sparse attention", Walkthrough: selected-token attention;
 * "Unify sparse attention framework ...", Description: the op consumes
 * predicted indices).  For query head h of request b with KV head g:
 *   x_t = softmax_scale * (q_h . k_t),  o_h = sum_t e^{x_t - max x} v_t /
 *   sum_t e^{x_t - max x}, over the kept t of indices[b][g][0..k_sel).
 *   q        device [batch][q_heads][k_pool->head_dim], dtype q_dtype
 *   k_pool   key rows; v_pool value rows whose first v_dim elements are the
 *            value (MLA: pass the latent pool as both, v_dim = 512); F32 or
 *            BF16 (FP8 pools are scored, not attended)
 *   indices  device [batch][num_kv_heads][k_sel] int32 request-local
 *            positions, -1 = unused slot; a position >= kv_len or on an absent
 *            page is skipped
 *   out      device [batch][q_heads][v_dim] in out_dtype; a head with no kept
 *            row gets zeros
 *   workspace device, at least sd_sparse_decode_attn_workspace_size() bytes. */
sd_status sd_sparse_decode_attn_workspace_size(const sd_pages* pages, int32_t q_heads,
                                               const sd_pool* k_pool, int32_t v_dim,
                                               int32_t k_sel, size_t* bytes);
sd_status sd_sparse_decode_attn(const sd_pages* pages, const void* q, sd_dtype q_dtype,
                                int32_t q_heads, const sd_pool* k_pool, const sd_pool* v_pool,
                                int32_t v_dim, const int32_t* indices, int32_t k_sel,
                                float softmax_scale, void* out, sd_dtype out_dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Attention over block-granular selections ("Unify sparse attention
 * framework with clean backend interfaces", review of the runtime carrier:
 * the indices travel with an indices block size).  Entry e >= 0 of a row
 * names the tokens [e*block_size, (e+1)*block_size) that lie below kv_len;
 * a negative entry names none.  The result is sd_sparse_decode_attn over the
 * token list the entries name, in order (an entry given twice counts twice).
 *   block_indices device [batch][num_kv_heads][k_blocks] int32
 *   block_size    >= 1; k_blocks * block_size <= 2^24
 *   workspace     device, at least sd_sparse_decode_attn_blocks_workspace_size()
 * Other arguments and errors as sd_sparse_decode_attn. */
sd_status sd_sparse_decode_attn_blocks_workspace_size(const sd_pages* pages, int32_t q_heads,
                                                      const sd_pool* k_pool, int32_t v_dim,
                                                      int32_t k_blocks, int32_t block_size,
                                                      size_t* bytes);
sd_status sd_sparse_decode_attn_blocks(const sd_pages* pages, const void* q, sd_dtype q_dtype,
                                       int32_t q_heads, const sd_pool* k_pool, const sd_pool* v_pool,
                                       int32_t v_dim, const int32_t* block_indices, int32_t k_blocks,
                                       int32_t block_size, float softmax_scale, void* out,
                                       sd_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/* ------------------------------------------------------------------ fused */

/* One whole decode step: score -> top-k -> attention on one stream, with no
 * host round trip.  With precision = SD_SCORE_FAST the DSA scores come from
 * matrix cores and the selection is still exactly the SD_SCORE_EXACT top-k:
 * tokens whose fast score lies within twice the row's error bound of the
 * k-th fast score are re-scored in the exact order before the final choice.
 * The score side and the attention side may use different pools (DSA: the
 * indexer K pool scores, the MLA latent pool is attended), with the same
 * block table and page size.  The selection is per score-side KV head; the
 * attention side must have the same number of KV heads. */
typedef struct sd_sparse_decode_args {
  sd_pages pages;
  /* scoring (step 1) */
  sd_pool score_k;
  const void* score_q;           /* device [batch][score_heads][score_k.head_dim] */
  sd_dtype score_q_dtype;
  int32_t score_heads;
  const float* head_weights;     /* device [batch][score_heads] or NULL        */
  sd_score_mode mode;
  float head_scale;
  sd_score_precision precision;
  /* selection (step 2) */
  int32_t topk;
  /* attention (step 3) */
  const void* q;                 /* device [batch][q_heads][k.head_dim]        */
  sd_dtype q_dtype;
  int32_t q_heads;
  sd_pool k;
  sd_pool v;
  int32_t v_dim;
  float softmax_scale;
  void* out;                     /* device [batch][q_heads][v_dim]             */
  sd_dtype out_dtype;
  /* optional outputs (NULL to skip) */
  int32_t* indices_out;          /* device [batch][groups][topk]               */
  int32_t* counts_out;           /* device [batch][groups]                     */
  /* optional hint and write-back, as sd_topk_select_hinted (NULL to skip);
   * with fast scores the floor is the hint's smallest fast score minus twice
   * the row bound, so selection stays exact */
  const int32_t* topk_hint;      /* device [batch][groups][hint_stride]        */
  int32_t hint_len;
  int64_t hint_stride;
  int32_t* topk_writeback;       /* device [batch][groups][writeback_stride]   */
  int64_t writeback_stride;
  /* multi-query decode (0 or 1: one query per request).  With next_n > 1
   * every request carries next_n consecutive query tokens (a decode token
   * and its draft tokens), the last next_n positions of its kv_len tokens;
   * query j (0-based) sees tokens t < kv_len - (next_n - 1 - j) (causal).
   * Each query token is scored, selected and attended on its own: score_q,
   * head_weights, q, out, indices_out, counts_out, topk_hint and
   * topk_writeback gain a next_n dimension after batch ([batch][next_n]...).
   * ("Overlap DSA heuristic prev_topk write-back on the aux stream",
   * Performance: the MTP=3 end-to-end setting; next_n <= 64.) */
  int32_t next_n;
} sd_sparse_decode_args;

sd_status sd_sparse_decode_workspace_size(const sd_sparse_decode_args* args, size_t* bytes);
sd_status sd_sparse_decode(const sd_sparse_decode_args* args, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* The fused step without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, kernels and results as
 * sd_sparse_decode; its scratch is a fixed array inside the library, one per
 * device (sd_sparse_decode_noalloc_max_bytes() bytes = 64 MiB, held by each
 * GPU the library runs on until the process ends).  The call allocates and
 * frees nothing.  A call whose workspace (sd_sparse_decode_workspace_size)
 * would exceed the scratch returns SD_ERR_WORKSPACE_TOO_SMALL and launches
 * nothing.  stream must belong to the current device (else
 * SD_ERR_INVALID_ARGUMENT).  The first call on a device looks up the
 * scratch's device address there (no allocation).  Every call on one device
 * shares that device's scratch: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialized by the caller; the scratch keeps
 * the last call's contents, and nothing in the step depends on them. */
size_t sd_sparse_decode_noalloc_max_bytes(void);
sd_status sd_sparse_decode_noalloc(const sd_sparse_decode_args* args, hipStream_t stream);

/* ------------------------------------------------------------------ indices */

/* Request-local position -> flat pool slot page*page_size + t%page_size, -1
 * for a negative position, a position past the block table, or a page id
 * outside [0, num_pages) ("Unify sparse attention framework ...", Dev
 * Engineer Review: global index conversion).  local and global_out are
 * device [batch][groups][k]. */
sd_status sd_local_to_global(const sd_pages* pages, int32_t page_size, int32_t num_pages,
                             const int32_t* local, int32_t groups, int32_t k,
                             int64_t* global_out, hipStream_t stream);

/* ------------------------------------------------------------------ misc */

const char* sd_status_string(sd_status status);
/* Text of the last failed call's reason on this host thread ("" if none). */
const char* sd_last_error(void);
int32_t sd_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPARSE_DECODE_H */
