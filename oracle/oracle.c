/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for top-k sparse
 * decode attention over a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): used by the tests, the smoke check
 * and the benchmark's CPU-baseline leg, never by the product path.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared.  Every float
 * expression below is written one rounding per operation; with contraction
 * off and SSE arithmetic on x86-64 that is exactly what executes.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------ threads */

int orc_set_threads(int32_t n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
  return omp_get_max_threads();
#else
  (void)n;
  return 1;
#endif
}

/* ------------------------------------------------------------------ helpers */

/* bfloat16 is the upper 16 bits of a binary32: widening is exact. */
static float bf16_bits_to_float(uint16_t b) {
  uint32_t u = ((uint32_t)b) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* OCP FP8 E4M3 ("E4M3FN"): sign bit, 4 exponent bits with bias 7, 3
 * mantissa bits.  Exponent field 0 holds the subnormals m * 2^-9; the two
 * codes with every exponent and mantissa bit set are NaN; there is no
 * infinity, the largest finite value is 448. */
static float fp8_e4m3_to_float(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  /* (1 + m/8) * 2^(e-7) = (8 + m) * 2^(e-10) for normals */
  const float v = e == 0 ? ldexpf((float)m, -9) : ldexpf((float)(8 + m), e - 10);
  return s ? -v : v;
}

static float load_elem(const void* base, int32_t dtype, int64_t off) {
  if (dtype == ORC_F32) return ((const float*)base)[off];
  if (dtype == ORC_FP8) return fp8_e4m3_to_float(((const uint8_t*)base)[off]);
  return bf16_bits_to_float(((const uint16_t*)base)[off]);
}

/* Logical token t of request b lives in physical page block_table[b][t/P] at
 * slot t%P ("Unify sparse attention framework ...", Dev Engineer Review: the
 * global index conversion goes through block_table with a page-range check).
 * Returns the element offset of the first element of that row for KV head g,
 * or -1 when the page id is outside [0, num_pages). */
static int64_t row_offset(const orc_pool* p, const int32_t* block_table, int32_t max_pages,
                          int32_t b, int32_t g, int32_t t) {
  int32_t lp = t / p->page_size;
  int32_t slot = t % p->page_size;
  if (lp >= max_pages) return -1;
  int32_t page = block_table[(int64_t)b * max_pages + lp];
  if (page < 0 || page >= p->num_pages) return -1;
  return (int64_t)page * p->page_stride + (int64_t)g * p->head_stride +
         (int64_t)slot * p->token_stride;
}

/* The FP8 row scale of token t (same page lookup as row_offset, which the
 * caller has already checked). */
static float row_scale(const orc_pool* p, const int32_t* block_table, int32_t max_pages, int32_t b,
                       int32_t g, int32_t t) {
  const int32_t page = block_table[(int64_t)b * max_pages + t / p->page_size];
  return p->scale[((int64_t)page * p->num_kv_heads + g) * p->page_size + t % p->page_size];
}

/* q . k accumulated in binary32 in ascending d, each product and each sum
 * rounded on its own:  (((+0 + q0*k0) + q1*k1) + ...) + q_{D-1}*k_{D-1}.
 * (For bfloat16 operands every product is exact in binary32.) */
static float dot_f32_sequential(const float* qv, const float* kv, int32_t D) {
  float acc = 0.0f;
  for (int32_t d = 0; d < D; ++d) {
    float prod = qv[d] * kv[d];
    acc = acc + prod;
  }
  return acc;
}

/* ------------------------------------------------------------------ scores */

/* Scoring of every cached token through the page table ("Add TriAttention
 * KV-cache compression method", Key Design Decisions: direct paged-pool
 * scoring; Summary: per-head scores are then reduced to one score per KV
 * head).  Modes:
 *   GROUP_SUM      s = sum_h (dot_h * head_scale),  h ascending
 *   GROUP_MEAN     s = (sum_h dot_h) * (1/G),       h ascending
 *   RELU_WEIGHTED  s = sum_h (w_h * max(dot_h, +0)), h ascending
 * The last one is the DSA indexer score: a ReLU-weighted sum over the indexer
 * heads of q_I,h . k_I, with one indexer key row per token shared by all
 * indexer heads ("Overlap DSA heuristic prev_topk write-back on the aux
 * stream", Description: the indexer produces each decode step's top-k). */
int orc_score(const int32_t* block_table, int32_t max_pages, const int32_t* kv_lens,
              int32_t batch, const orc_pool* k, const void* q, int32_t q_dtype,
              int32_t q_heads, const float* weights, int32_t mode, float head_scale,
              float* scores, int32_t row_len) {
  if (!block_table || !kv_lens || !k || !k->data || !q || !scores) return ORC_EARG;
  if (batch < 0 || max_pages < 0 || row_len < 0 || q_heads <= 0) return ORC_EARG;
  const int32_t Hkv = k->num_kv_heads, D = k->head_dim;
  if (Hkv <= 0 || D <= 0 || k->page_size <= 0 || q_heads % Hkv != 0) return ORC_EARG;
  if (mode == ORC_RELU_WEIGHTED && !weights) return ORC_EARG;
  if (mode < ORC_GROUP_SUM || mode > ORC_RELU_WEIGHTED) return ORC_EARG;
  if (k->dtype == ORC_FP8 && !k->scale) return ORC_EARG;
  const int32_t G = q_heads / Hkv;
  const float inv_g = (float)(1.0 / (double)G);

  /* rows (b, g) are independent: with OpenMP they run on several threads,
   * each row's arithmetic unchanged (the result does not depend on the
   * thread count); the first failing row in row order decides the status */
  const int64_t nrows = (int64_t)batch * Hkv;
  int* row_rc = (int*)calloc((size_t)(nrows > 0 ? nrows : 1), sizeof(int));
  if (!row_rc) return ORC_EARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int32_t b = (int32_t)(r / Hkv), g = (int32_t)(r % Hkv);
    float* qf = (float*)malloc(sizeof(float) * (size_t)G * (size_t)D);
    float* kf = (float*)malloc(sizeof(float) * (size_t)D);
    int rc = ORC_OK;
    const int32_t L = kv_lens[b];
    float* row = scores + r * row_len;
    if (!qf || !kf) rc = ORC_EARG;
    else if (L < 0 || L > row_len || L > max_pages * k->page_size) rc = ORC_EARG;
    if (rc == ORC_OK) {
      for (int32_t j = 0; j < G; ++j)
        for (int32_t d = 0; d < D; ++d)
          qf[(int64_t)j * D + d] = load_elem(q, q_dtype, ((int64_t)b * q_heads + g * G + j) * D + d);
      for (int32_t t = 0; t < row_len; ++t) row[t] = -INFINITY;
      for (int32_t t = 0; t < L; ++t) {
        int64_t off = row_offset(k, block_table, max_pages, b, g, t);
        if (off < 0) { rc = ORC_EPAGE; break; }
        for (int32_t d = 0; d < D; ++d) kf[d] = load_elem(k->data, k->dtype, off + d);
        if (k->dtype == ORC_FP8) {
          /* dequantize first, one binary32 rounding per element, then score
           * the binary32 row exactly as an F32 pool */
          const float sc = row_scale(k, block_table, max_pages, b, g, t);
          for (int32_t d = 0; d < D; ++d) kf[d] = kf[d] * sc;
        }
        float s = 0.0f;
        for (int32_t j = 0; j < G; ++j) {
          int32_t h = g * G + j;
          float dh = dot_f32_sequential(qf + (int64_t)j * D, kf, D);
          if (mode == ORC_GROUP_SUM) {
            float term = dh * head_scale;
            s = s + term;
          } else if (mode == ORC_GROUP_MEAN) {
            s = s + dh;
          } else {
            float rl = dh > 0.0f ? dh : 0.0f;
            float term = weights[(int64_t)b * q_heads + h] * rl;
            s = s + term;
          }
        }
        if (mode == ORC_GROUP_MEAN) s = s * inv_g;
        row[t] = s;
      }
    }
    row_rc[r] = rc;
    free(qf);
    free(kf);
  }
  int rc = ORC_OK;
  for (int64_t r = 0; r < nrows && rc == ORC_OK; ++r) rc = row_rc[r];
  free(row_rc);
  return rc;
}

/* ------------------------------------------------------------------ top-k */

typedef struct {
  float s;
  int32_t t;
} scored_tok;

/* (score descending, token index ascending); IEEE comparison, so -0 == +0. */
static int cmp_rank(const void* a, const void* b) {
  const scored_tok* x = (const scored_tok*)a;
  const scored_tok* y = (const scored_tok*)b;
  if (x->s > y->s) return -1;
  if (x->s < y->s) return 1;
  return (x->t < y->t) ? -1 : (x->t > y->t);
}

static int cmp_int(const void* a, const void* b) {
  int32_t x = *(const int32_t*)a, y = *(const int32_t*)b;
  return (x > y) - (x < y);
}

/* Selection of the k best tokens per row with deterministic tie settlement:
 * a full sort by (score descending, index ascending), lowest index first
 * among equal scores ("Add TriAttention KV-cache compression method", Summary:
 * TopK / tie settlement; Test Plan: deterministic heavy-tie settlement).  A row
 * with kv_len <= k keeps every token (the dense-equivalent case).  The kept
 * set is emitted in ascending token order and padded with -1; counts gets the
 * number kept, the per-request selected length the attention op consumes
 * ("Unify sparse attention framework ...", Description: the runtime carries
 * indices plus per-request lengths to the attention op). */
int orc_topk(const float* scores, int32_t batch, int32_t groups, int32_t row_len,
             const int32_t* kv_lens, int32_t k, int32_t* indices, int32_t* counts) {
  if (!scores || !kv_lens || !indices || batch < 0 || groups <= 0 || row_len < 0 || k <= 0)
    return ORC_EARG;
  const int64_t nrows = (int64_t)batch * groups;
  int* row_rc = (int*)calloc((size_t)(nrows > 0 ? nrows : 1), sizeof(int));
  if (!row_rc) return ORC_EARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int32_t b = (int32_t)(r / groups);
    scored_tok* buf = (scored_tok*)malloc(sizeof(scored_tok) * (size_t)(row_len > 0 ? row_len : 1));
    int32_t* keep = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
    int rc = ORC_OK;
    const int32_t L = kv_lens[b];
    if (!buf || !keep || L < 0 || L > row_len) rc = ORC_EARG;
    if (rc == ORC_OK) {
      const float* row = scores + r * row_len;
      for (int32_t t = 0; t < L; ++t) {
        if (isnan(row[t])) { rc = ORC_ENAN; break; }
        buf[t].s = row[t];
        buf[t].t = t;
      }
    }
    if (rc == ORC_OK) {
      qsort(buf, (size_t)L, sizeof(scored_tok), cmp_rank);
      int32_t n = L < k ? L : k;
      for (int32_t i = 0; i < n; ++i) keep[i] = buf[i].t;
      qsort(keep, (size_t)n, sizeof(int32_t), cmp_int);
      int32_t* out = indices + r * k;
      for (int32_t i = 0; i < k; ++i) out[i] = i < n ? keep[i] : -1;
      if (counts) counts[r] = n;
    }
    row_rc[r] = rc;
    free(buf);
    free(keep);
  }
  int rc = ORC_OK;
  for (int64_t r = 0; r < nrows && rc == ORC_OK; ++r) rc = row_rc[r];
  free(row_rc);
  return rc;
}

/* ------------------------------------------------------------------ attention */

/* Softmax attention of every query head over its KV head's selected rows, in
 * float64 throughout: x_t = scale * sum_d q_d k_td, p_t = exp(x_t - max x),
 * o = sum_t p_t v_t / sum_t p_t.  This is the eager golden reference's
 * selected-token attention ("Add DSA Vanilla sparse attention", Walkthrough:
 * it rebuilds each request's logical cache and performs selected-token
 * attention).  For sparse MLA the value row is the leading v_dim elements of
 * the same latent row. */
int orc_attention(const int32_t* block_table, int32_t max_pages, const int32_t* kv_lens,
                  int32_t batch, const void* q, int32_t q_dtype, int32_t q_heads,
                  const orc_pool* k, const orc_pool* v, int32_t v_dim,
                  const int32_t* indices, int32_t k_sel, float scale, double* out) {
  if (!block_table || !kv_lens || !q || !k || !v || !k->data || !v->data || !indices || !out)
    return ORC_EARG;
  const int32_t Hkv = k->num_kv_heads, D = k->head_dim;
  if (batch < 0 || q_heads <= 0 || Hkv <= 0 || q_heads % Hkv != 0 || k_sel <= 0) return ORC_EARG;
  if (v->num_kv_heads != Hkv || v_dim <= 0 || v_dim > v->head_dim) return ORC_EARG;
  if (v->page_size != k->page_size) return ORC_EARG;
  if (k->dtype == ORC_FP8 || v->dtype == ORC_FP8) return ORC_EARG;  /* indexer pools only */
  const int32_t G = q_heads / Hkv;

  const int64_t nrows = (int64_t)batch * Hkv;
  int* row_rc = (int*)calloc((size_t)(nrows > 0 ? nrows : 1), sizeof(int));
  if (!row_rc) return ORC_EARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < nrows; ++r) {
    const int32_t b = (int32_t)(r / Hkv), g = (int32_t)(r % Hkv);
    double* x = (double*)malloc(sizeof(double) * (size_t)k_sel);
    int64_t* koff = (int64_t*)malloc(sizeof(int64_t) * (size_t)k_sel);
    int64_t* voff = (int64_t*)malloc(sizeof(int64_t) * (size_t)k_sel);
    double* acc = (double*)malloc(sizeof(double) * (size_t)v_dim);
    int rc = (!x || !koff || !voff || !acc) ? ORC_EARG : ORC_OK;
    const int32_t L = kv_lens[b];
    const int32_t* sel = indices + r * k_sel;
    int32_t n = 0;
    for (int32_t i = 0; i < k_sel && rc == ORC_OK; ++i) {
      int32_t t = sel[i];
      if (t < 0) continue;
      if (t >= L) { rc = ORC_EINDEX; break; }
      int64_t ko = row_offset(k, block_table, max_pages, b, g, t);
      int64_t vo = row_offset(v, block_table, max_pages, b, g, t);
      if (ko < 0 || vo < 0) { rc = ORC_EPAGE; break; }
      koff[n] = ko;
      voff[n] = vo;
      ++n;
    }
    for (int32_t j = 0; j < G && rc == ORC_OK; ++j) {
      int32_t h = g * G + j;
      double* o = out + ((int64_t)b * q_heads + h) * v_dim;
      if (n == 0) {
        for (int32_t d = 0; d < v_dim; ++d) o[d] = 0.0;
        continue;
      }
      int64_t qo = ((int64_t)b * q_heads + h) * D;
      double m = -INFINITY;
      for (int32_t i = 0; i < n; ++i) {
        double sd = 0.0;
        for (int32_t d = 0; d < D; ++d)
          sd += (double)load_elem(q, q_dtype, qo + d) *
                (double)load_elem(k->data, k->dtype, koff[i] + d);
        x[i] = (double)scale * sd;
        if (x[i] > m) m = x[i];
      }
      double l = 0.0;
      for (int32_t d = 0; d < v_dim; ++d) acc[d] = 0.0;
      for (int32_t i = 0; i < n; ++i) {
        double p = exp(x[i] - m);
        l += p;
        for (int32_t d = 0; d < v_dim; ++d)
          acc[d] += p * (double)load_elem(v->data, v->dtype, voff[i] + d);
      }
      for (int32_t d = 0; d < v_dim; ++d) o[d] = acc[d] / l;
    }
    row_rc[r] = rc;
    free(x);
    free(koff);
    free(voff);
    free(acc);
  }
  int rc = ORC_OK;
  for (int64_t r = 0; r < nrows && rc == ORC_OK; ++r) rc = row_rc[r];
  free(row_rc);
  return rc;
}

/* ------------------------------------------------------------------ indices */

/* Global index conversion: request-local position -> pool slot through the
 * block table, invalid (-1) for a negative position or a page outside the
 * pool ("Unify sparse attention framework ...", Dev Engineer Review). */
int orc_local_to_global(const int32_t* block_table, int32_t max_pages, int32_t batch,
                        int32_t page_size, int32_t num_pages, const int32_t* local,
                        int32_t groups, int32_t k, int64_t* global_out) {
  if (!block_table || !local || !global_out || batch < 0 || groups <= 0 || k <= 0 ||
      page_size <= 0 || max_pages < 0)
    return ORC_EARG;
  for (int32_t b = 0; b < batch; ++b)
    for (int32_t g = 0; g < groups; ++g)
      for (int32_t i = 0; i < k; ++i) {
        int64_t idx = ((int64_t)b * groups + g) * k + i;
        int32_t t = local[idx];
        int64_t r = -1;
        if (t >= 0 && t / page_size < max_pages) {
          int32_t page = block_table[(int64_t)b * max_pages + t / page_size];
          if (page >= 0 && page < num_pages) r = (int64_t)page * page_size + t % page_size;
        }
        global_out[idx] = r;
      }
  return ORC_OK;
}

/* ------------------------------------------------------------------ TriAttention modes */

/* Exactly rounded sums.  A long accumulator holds a non-negative multiple of
 * 2^-1074 (the smallest binary64 step) in 64-bit words, word 0 lowest; 35
 * words (2240 bits) take any finite binary64 magnitude (below 2^1024, so
 * bit 2098 is the highest) 2^31 times over.  Positive and negative terms go to
 * two accumulators; the sum is their difference, rounded once to the nearest
 * binary64, ties to even. */
#define ORC_ACC_WORDS 35
typedef struct {
  uint64_t w[ORC_ACC_WORDS];
} orc_acc;

/* acc += |v| for a finite v */
static void acc_add_magnitude(orc_acc* a, double v) {
  uint64_t bits;
  memcpy(&bits, &v, sizeof bits);
  const int ef = (int)((bits >> 52) & 0x7FF);
  uint64_t m = bits & ((1ull << 52) - 1);
  int pos; /* the bit of 2^-1074 multiples that m's lowest bit stands for */
  if (ef == 0) {
    pos = 0; /* subnormal: frac * 2^-1074 */
  } else {
    m |= 1ull << 52;
    pos = ef - 1; /* (2^52 + frac) * 2^(ef - 1075) */
  }
  if (m == 0) return;
  const int wi = pos / 64, sh = pos % 64;
  /* m << sh spans words wi and wi + 1 */
  const uint64_t lo = m << sh;
  const uint64_t hi = sh == 0 ? 0 : m >> (64 - sh);
  uint64_t old = a->w[wi];
  a->w[wi] = old + lo;
  uint64_t carry = a->w[wi] < old ? 1u : 0u;
  uint64_t add = hi + carry; /* hi < 2^53: no overflow */
  for (int j = wi + 1; add != 0 && j < ORC_ACC_WORDS; ++j) {
    old = a->w[j];
    a->w[j] = old + add;
    add = a->w[j] < old ? 1u : 0u;
  }
}

/* bit i of the accumulator */
static int acc_bit(const orc_acc* a, int i) { return (int)((a->w[i / 64] >> (i % 64)) & 1u); }

/* the nearest binary64 to p - n (ties to even) */
static double acc_round(const orc_acc* p, const orc_acc* n) {
  int cmp = 0;
  for (int j = ORC_ACC_WORDS - 1; j >= 0 && cmp == 0; --j)
    if (p->w[j] != n->w[j]) cmp = p->w[j] > n->w[j] ? 1 : -1;
  if (cmp == 0) return 0.0;
  const orc_acc* big = cmp > 0 ? p : n;
  const orc_acc* small = cmp > 0 ? n : p;
  orc_acc d; /* big - small */
  uint64_t borrow = 0;
  for (int j = 0; j < ORC_ACC_WORDS; ++j) {
    const uint64_t x = big->w[j], y = small->w[j];
    d.w[j] = x - y - borrow;
    borrow = (x < y || (x == y && borrow)) ? 1u : 0u;
  }
  int top = ORC_ACC_WORDS * 64 - 1;
  while (!acc_bit(&d, top)) --top;
  double mag;
  if (top <= 52) {
    mag = ldexp((double)d.w[0], -1074); /* fits in 53 bits: exact */
  } else {
    const int lowbit = top - 52; /* the 53 kept bits are top .. lowbit */
    uint64_t mant = 0;
    for (int i = top; i >= lowbit; --i) mant = (mant << 1) | (uint64_t)acc_bit(&d, i);
    const int round = acc_bit(&d, lowbit - 1);
    int sticky = 0;
    for (int i = lowbit - 2; i >= 0 && !sticky; --i) sticky = acc_bit(&d, i);
    int e = lowbit;
    if (round && (sticky || (mant & 1u))) {
      ++mant;
      if (mant == (1ull << 53)) {
        mant >>= 1;
        ++e;
      }
    }
    mag = ldexp((double)mant, e - 1074);
  }
  return cmp > 0 ? mag : -mag;
}

int orc_exact_sum(const double* v, int64_t n, double* out) {
  if ((!v && n > 0) || n < 0 || n > 2147483647 || !out) return ORC_EARG;
  orc_acc p, m;
  memset(&p, 0, sizeof p);
  memset(&m, 0, sizeof m);
  for (int64_t i = 0; i < n; ++i) {
    if (!isfinite(v[i])) return ORC_EARG;
    if (v[i] > 0.0) acc_add_magnitude(&p, v[i]);
    else if (v[i] < 0.0) acc_add_magnitude(&m, v[i]);
  }
  *out = acc_round(&p, &m);
  return ORC_OK;
}

/* Normalization of one member row (see oracle.h): the population mean and
 * standard deviation of the row's finite scores, each sum exactly rounded. */
static void tri_normalize_row(const float* row, int32_t L, int32_t row_len, float* z) {
  int64_t n = 0;
  orc_acc pos, neg;
  memset(&pos, 0, sizeof pos);
  memset(&neg, 0, sizeof neg);
  for (int32_t t = 0; t < L; ++t)
    if (isfinite(row[t])) {
      const double x = (double)row[t];
      if (x > 0.0) acc_add_magnitude(&pos, x);
      else if (x < 0.0) acc_add_magnitude(&neg, x);
      ++n;
    }
  const double s1 = acc_round(&pos, &neg);
  const double mu = n > 0 ? s1 / (double)n : 0.0;
  memset(&pos, 0, sizeof pos);
  memset(&neg, 0, sizeof neg);
  for (int32_t t = 0; t < L; ++t)
    if (isfinite(row[t])) {
      const double d = (double)row[t] - mu;
      const double dd = d * d;
      acc_add_magnitude(&pos, dd);
    }
  const double s2 = acc_round(&pos, &neg);
  const double sigma = n > 0 ? sqrt(s2 / (double)n) : 0.0;
  for (int32_t t = 0; t < row_len; ++t) {
    if (t >= L || !isfinite(row[t])) {
      z[t] = -INFINITY;
    } else if (sigma == 0.0) {
      z[t] = 0.0f;
    } else {
      const double d = (double)row[t] - mu;
      z[t] = (float)(d / sigma);
    }
  }
}

int orc_tri_select(const float* scores, int32_t layers, int32_t batch, int32_t groups, int32_t row_len,
                   const int32_t* kv_lens, int32_t mode, int32_t k, float* z, float* reduced,
                   int32_t* indices, int32_t* counts) {
  if (!scores || !kv_lens || !indices || layers <= 0 || batch < 0 || groups <= 0 || row_len < 0 || k <= 0)
    return ORC_EARG;
  if (mode != ORC_PER_LAYER_PERHEAD && mode != ORC_PER_HEAD && mode != ORC_UNION) return ORC_EARG;
  const int64_t members = (int64_t)layers * batch * groups;
  for (int32_t b = 0; b < batch; ++b)
    if (kv_lens[b] < 0 || kv_lens[b] > row_len) return ORC_EARG;
  for (int64_t m = 0; m < members; ++m) {
    const int32_t b = (int32_t)((m / groups) % batch);
    for (int32_t t = 0; t < kv_lens[b]; ++t)
      if (isnan(scores[m * row_len + t])) return ORC_ENAN;
  }
  float* zz = (float*)malloc(sizeof(float) * (size_t)(members * row_len > 0 ? members * row_len : 1));
  if (!zz) return ORC_EARG;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t m = 0; m < members; ++m) {
    const int32_t b = (int32_t)((m / groups) % batch);
    tri_normalize_row(scores + m * row_len, kv_lens[b], row_len, zz + m * row_len);
  }
  if (z) memcpy(z, zz, sizeof(float) * (size_t)(members * row_len));

  /* reduced rows and the batch / group shape the top-k sees */
  int32_t out_batch, out_groups;
  int32_t* lens;
  if (mode == ORC_PER_LAYER_PERHEAD) { out_batch = layers * batch; out_groups = groups; }
  else if (mode == ORC_PER_HEAD) { out_batch = batch; out_groups = groups; }
  else { out_batch = batch; out_groups = 1; }
  const int64_t out_rows = (int64_t)out_batch * out_groups;
  float* r = (float*)malloc(sizeof(float) * (size_t)(out_rows * row_len > 0 ? out_rows * row_len : 1));
  lens = (int32_t*)malloc(sizeof(int32_t) * (size_t)(out_batch > 0 ? out_batch : 1));
  if (!r || !lens) { free(zz); free(r); free(lens); return ORC_EARG; }
  for (int32_t ob = 0; ob < out_batch; ++ob) lens[ob] = kv_lens[ob % batch];
  for (int64_t o = 0; o < out_rows; ++o)
    for (int32_t t = 0; t < row_len; ++t) r[o * row_len + t] = -INFINITY;
  for (int32_t l = 0; l < layers; ++l)
    for (int32_t b = 0; b < batch; ++b)
      for (int32_t g = 0; g < groups; ++g) {
        const float* src = zz + (((int64_t)l * batch + b) * groups + g) * row_len;
        int64_t o;
        if (mode == ORC_PER_LAYER_PERHEAD) o = ((int64_t)l * batch + b) * groups + g;
        else if (mode == ORC_PER_HEAD) o = (int64_t)b * groups + g;
        else o = b;
        float* dst = r + o * row_len;
        for (int32_t t = 0; t < row_len; ++t)
          if (src[t] > dst[t]) dst[t] = src[t];
      }
  if (reduced) memcpy(reduced, r, sizeof(float) * (size_t)(out_rows * row_len));
  const int rc = orc_topk(r, out_batch, out_groups, row_len, lens, k, indices, counts);
  free(zz);
  free(r);
  free(lens);
  return rc;
}
