/*
 * oracle.h -- plain CPU oracle for top-k sparse decode attention over a paged
 * KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this code; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the HIP
 * library: every definition here is written out again from the statement of
 * the method.
 *
 * What it computes (each function below cites the passage it follows):
 *   1. scores   -- every cached token of every request is scored through the
 *                  page table ("Add TriAttention KV-cache compression method",
 *                  Key Design Decisions: the scorer reads paged K directly
 *                  through a page-table snapshot);
 *   2. top-k    -- a full sort by (score descending, token index ascending):
 *                  deterministic tie settlement ("Add TriAttention ...", Summary
 *                  and Test Plan);
 *   3. attention-- exact softmax attention over the selected rows of each
 *                  request's logical cache, in float64 ("Add DSA Vanilla sparse
 *                  attention", Walkthrough: the eager golden reference that
 *                  rebuilds each request's logical cache and attends over the
 *                  selected tokens).
 *
 * Floating point: compiled with -O2 -ffp-contract=off and without
 * -ffast-math, so every written float operation rounds separately (IEEE-754
 * binary32, round to nearest even, no flush to zero).
 */
#ifndef TSD_ORACLE_H
#define TSD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
#define ORC_F32 0   /* IEEE binary32                                  */
#define ORC_BF16 1  /* bfloat16 bits stored as uint16 (upper half of f32) */
#define ORC_FP8 2   /* OCP FP8 E4M3 byte codes with one binary32 scale per row */

/* score modes */
#define ORC_GROUP_SUM 0      /* s = sum_{h in group} (dot_h * head_scale)       */
#define ORC_GROUP_MEAN 1     /* s = (sum_{h in group} dot_h) * (1/G)            */
#define ORC_RELU_WEIGHTED 2  /* s = sum_{h in group} (w_h * max(dot_h, +0))     */

/* error codes */
#define ORC_OK 0
#define ORC_EARG 1      /* bad argument (null pointer, bad size)            */
#define ORC_EPAGE 2     /* a referenced page id is outside [0, num_pages)   */
#define ORC_ENAN 3      /* a score that takes part in selection is NaN      */
#define ORC_EINDEX 4    /* a selected index is outside [0, kv_len)          */

typedef struct {
  const void* data;  /* host memory                                          */
  int32_t dtype;     /* ORC_F32 or ORC_BF16                                  */
  int32_t num_pages, page_size, num_kv_heads, head_dim;
  int64_t page_stride, head_stride, token_stride;  /* in elements            */
  /* ORC_FP8 only: the scale of each row, [num_pages][num_kv_heads][page_size]
   * contiguous; row (page, g, slot) stands for the values
   * decode(code) * scale[(page * num_kv_heads + g) * page_size + slot]. */
  const float* scale;
} orc_pool;

/* Scores for every (request b, KV head g, token t < kv_lens[b]); entries
 * t >= kv_lens[b] of a row are set to -inf.  q is [batch][q_heads][head_dim],
 * query head h belongs to KV head h / (q_heads / num_kv_heads).  weights is
 * [batch][q_heads] (RELU_WEIGHTED only).  scores is [batch][num_kv_heads][row_len].
 * An ORC_FP8 pool is dequantized first (each element decoded and multiplied
 * by its row scale, one binary32 rounding) and the binary32 row is then
 * scored exactly as an ORC_F32 row: the block-scaled FP8 indexer cache of
 * "Overlap DSA heuristic prev_topk write-back on the aux stream" (Test
 * Coverage: the FP8 block-scale end-to-end test). */
int orc_score(const int32_t* block_table, int32_t max_pages, const int32_t* kv_lens,
              int32_t batch, const orc_pool* k, const void* q, int32_t q_dtype,
              int32_t q_heads, const float* weights, int32_t mode, float head_scale,
              float* scores, int32_t row_len);

/* Top-k of each row over t < kv_lens[b]: the min(k, kv_len) tokens that come
 * first in (score descending, index ascending) order, written in ascending
 * token order and padded with -1.  indices is [batch][groups][k], counts is
 * [batch][groups] (may be NULL). */
int orc_topk(const float* scores, int32_t batch, int32_t groups, int32_t row_len,
             const int32_t* kv_lens, int32_t k, int32_t* indices, int32_t* counts);

/* Softmax attention over the selected rows, float64.  q is
 * [batch][q_heads][qk_dim] (qk_dim == k->head_dim), the value row is the first
 * v_dim elements of the v pool row (v may describe the same memory as k).
 * indices is [batch][num_kv_heads][k_sel] of request-local token positions,
 * -1 entries are skipped.  out is [batch][q_heads][v_dim]; a head with no
 * selected row gets zeros. */
int orc_attention(const int32_t* block_table, int32_t max_pages, const int32_t* kv_lens,
                  int32_t batch, const void* q, int32_t q_dtype, int32_t q_heads,
                  const orc_pool* k, const orc_pool* v, int32_t v_dim,
                  const int32_t* indices, int32_t k_sel, float scale, double* out);

/* Request-local token position -> flat pool slot page*page_size + t%page_size,
 * or -1 when the position is negative, past the table, or names a page outside
 * [0, num_pages).  local is [batch][groups][k], global the same shape. */
int orc_local_to_global(const int32_t* block_table, int32_t max_pages, int32_t batch,
                        int32_t page_size, int32_t num_pages, const int32_t* local,
                        int32_t groups, int32_t k, int64_t* global_out);

/* TriAttention selection modes ("Add TriAttention KV-cache compression
 * method", Summary: a normalize/reduce step between paged-K scoring and
 * TopK / tie settlement, with union, per_head and per_layer_perhead eviction
 * modes; Main Files: score normalization and union reduction).  The pages
 * name these steps only; the arithmetic below is this oracle's reading of
 * them, written out in full.
 *
 * scores is [layers][batch][groups][row_len].  Normalization, per member row
 * (layer, b, g), over its finite scores at t < kv_lens[b] (n of them), every
 * binary64 operation rounded on its own and each sum exactly rounded (the
 * exact real sum of its terms, rounded once to the nearest binary64, ties to
 * even; no order of summation enters):
 *   mu  = S1 / n, S1 = the exactly rounded sum of the finite s_t, each
 *         widened exactly to binary64;
 *   var = S2 / n, S2 = the exactly rounded sum of the d_t * d_t (each product
 *         rounded), d_t = (double)s_t - mu;
 *   sigma = sqrt(var);
 *   z_t = (float)(((double)s_t - mu) / sigma)  (0 when sigma == 0),
 *   z_t = -inf for a non-finite score and for t >= kv_lens[b].
 * Reduction: r_t = max over the mode's members of z_t (binary32 max).
 *   ORC_PER_LAYER_PERHEAD: one output row per (layer, b, g), its own z;
 *   ORC_PER_HEAD:          one row per (b, g), the max over layers;
 *   ORC_UNION:             one row per b, the max over layers and groups.
 * Selection: orc_topk on the reduced rows with kv_lens[b].
 * z (optional) receives every member's z, shape of scores; reduced
 * (optional) the reduced rows [out_rows][row_len]; indices [out_rows][k],
 * counts [out_rows] (may be NULL). */
/* Threads used by the row loops above (OpenMP over independent (request,
 * head group) rows; every result is bit-identical for any thread count).
 * n > 0 sets the count; returns the count now in effect. */
int orc_set_threads(int32_t n);

#define ORC_PER_LAYER_PERHEAD 0
#define ORC_PER_HEAD 1
#define ORC_UNION 2
/* The exactly rounded sum of n finite binary64 values (the sums of the
 * normalization above): *out = the nearest binary64 to their exact real sum,
 * ties to even.  ORC_EARG for a non-finite value. */
int orc_exact_sum(const double* v, int64_t n, double* out);

int orc_tri_select(const float* scores, int32_t layers, int32_t batch, int32_t groups, int32_t row_len,
                   const int32_t* kv_lens, int32_t mode, int32_t k, float* z, float* reduced,
                   int32_t* indices, int32_t* counts);

#ifdef __cplusplus
}
#endif
#endif
