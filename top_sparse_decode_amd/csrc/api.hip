// api.hip -- the C ABI of libsparse_decode (declared in
// include/sparse_decode.h): host-side validation, workspace layout and
// kernel dispatch.  The library allocates nothing, never synchronizes, and
// keeps no state between calls, so every entry point can be captured into a
// HIP graph ("Unify sparse attention framework with clean backend
// interfaces", Dev Engineer Review: buffer identity and stability under graph
// capture; "Add TriAttention KV-cache compression method", Key Design
// Decisions: score scratch reused, sized at the high-water mark).
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "common.h"
#include "kernels.h"
#include "sparse_decode.h"

// Device scratch of sd_sparse_decode_noalloc (64 MiB per device, see below).
static __device__ __align__(256) unsigned char sd_noalloc_scratch[size_t(64) << 20];

namespace {

thread_local std::string g_err;

sd_status fail(sd_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sd_status fail(sd_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sd_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return SD_OK;
  return fail(SD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_size(sd_dtype t) { return t == SD_F32 ? 4 : (t == SD_BF16 ? 2 : 1); }
bool dtype_ok(sd_dtype t) { return t == SD_F32 || t == SD_BF16 || t == SD_FP8_E4M3; }
int dtype_code(sd_dtype t) { return t == SD_F32 ? 0 : (t == SD_BF16 ? 1 : 2); }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

sd_status check_pages(const sd_pages* p, int32_t page_size) {
  if (!p) return fail(SD_ERR_INVALID_ARGUMENT, "pages is NULL");
  if (p->batch < 0 || p->max_pages < 0 || p->max_kv_len < 0)
    return fail(SD_ERR_INVALID_ARGUMENT, "negative batch / max_pages / max_kv_len");
  if (p->batch > 0 && (!p->block_table || !p->kv_lens))
    return fail(SD_ERR_INVALID_ARGUMENT, "block_table or kv_lens is NULL");
  if (p->batch > 0 && p->max_pages == 0 && p->max_kv_len > 0)
    return fail(SD_ERR_INVALID_ARGUMENT, "max_pages is 0 but max_kv_len > 0");
  if ((int64_t)p->max_pages * page_size < p->max_kv_len)
    return fail(SD_ERR_INVALID_ARGUMENT, "max_kv_len %d exceeds max_pages*page_size", p->max_kv_len);
  return SD_OK;
}

sd_status check_pool(const sd_pool* k, const char* name) {
  if (!k) return fail(SD_ERR_INVALID_ARGUMENT, "%s pool is NULL", name);
  if (!dtype_ok(k->dtype)) return fail(SD_ERR_INVALID_ARGUMENT, "%s: bad dtype", name);
  if (!k->data) return fail(SD_ERR_INVALID_ARGUMENT, "%s: data is NULL", name);
  if (k->num_pages <= 0 || k->page_size <= 0 || k->num_kv_heads <= 0 || k->head_dim <= 0)
    return fail(SD_ERR_INVALID_ARGUMENT, "%s: non-positive size", name);
  if (k->page_stride < 0 || k->head_stride < 0 || k->token_stride < 0)
    return fail(SD_ERR_INVALID_ARGUMENT, "%s: negative stride", name);
  const int es = elem_size(k->dtype);
  if (!aligned16(k->data) || ((int64_t)k->head_dim * es) % 16 || (k->page_stride * es) % 16 ||
      (k->head_stride * es) % 16 || (k->token_stride * es) % 16)
    return fail(SD_ERR_INVALID_ARGUMENT, "%s: rows must be 16-byte aligned", name);
  if (k->dtype == SD_FP8_E4M3) {
    if (!k->scale) return fail(SD_ERR_INVALID_ARGUMENT, "%s: FP8 pool needs row scales", name);
    if (!aligned16(k->scale)) return fail(SD_ERR_INVALID_ARGUMENT, "%s: scales must be 16-byte aligned", name);
  } else if (k->scale) {
    return fail(SD_ERR_INVALID_ARGUMENT, "%s: scales are for FP8 pools only", name);
  }
  return SD_OK;
}

sd::ScoreArgs make_score_args(const sd_pages* pg, const sd_pool* k, const void* q, int32_t q_heads,
                              const float* w, sd_score_mode mode, float head_scale, float* scores,
                              float* row_bound) {
  sd::ScoreArgs a{};
  a.block_table = pg->block_table;
  a.kv_lens = pg->kv_lens;
  a.batch = pg->batch;
  a.max_pages = pg->max_pages;
  a.max_kv_len = pg->max_kv_len;
  a.k = k->data;
  a.dtype = dtype_code(k->dtype);
  a.k_scale = k->scale;
  a.num_pages = k->num_pages;
  a.page_size = k->page_size;
  a.num_kv_heads = k->num_kv_heads;
  a.head_dim = k->head_dim;
  a.page_stride = k->page_stride;
  a.head_stride = k->head_stride;
  a.token_stride = k->token_stride;
  a.q = q;
  a.q_heads = q_heads;
  a.head_weights = w;
  a.mode = (int32_t)mode;
  a.head_scale = head_scale;
  const int G = q_heads / k->num_kv_heads;
  a.inv_g = (float)(1.0 / (double)G);
  a.scores = scores;
  a.row_bound = row_bound;
  return a;
}

// need_ptrs = false for size queries, which check shapes only.
sd_status check_score(const sd_pages* pg, const sd_pool* k, const void* q, sd_dtype q_dtype,
                      int32_t q_heads, const float* w, sd_score_mode mode, const float* scores,
                      bool need_ptrs) {
  sd_status st = check_pool(k, "score k");
  if (st != SD_OK) return st;
  if ((st = check_pages(pg, k->page_size)) != SD_OK) return st;
  if (k->dtype == SD_FP8_E4M3 ? q_dtype != SD_BF16 : q_dtype != k->dtype)
    return fail(SD_ERR_UNSUPPORTED, "score q dtype must equal the K pool dtype (BF16 for an FP8 pool)");
  if (need_ptrs) {
    if (!q) return fail(SD_ERR_INVALID_ARGUMENT, "score q is NULL");
    if (!aligned16(q)) return fail(SD_ERR_INVALID_ARGUMENT, "score q must be 16-byte aligned");
  }
  if (q_heads <= 0 || q_heads % k->num_kv_heads)
    return fail(SD_ERR_INVALID_ARGUMENT, "q_heads %d is not a multiple of num_kv_heads %d", q_heads,
                k->num_kv_heads);
  if (mode != SD_SCORE_GROUP_SUM && mode != SD_SCORE_GROUP_MEAN && mode != SD_SCORE_RELU_WEIGHTED)
    return fail(SD_ERR_INVALID_ARGUMENT, "bad score mode %d", (int)mode);
  if (need_ptrs && mode == SD_SCORE_RELU_WEIGHTED && !w)
    return fail(SD_ERR_INVALID_ARGUMENT, "RELU_WEIGHTED needs head_weights");
  if (!sd::score_exact_supported(q_heads / k->num_kv_heads))
    return fail(SD_ERR_UNSUPPORTED, "query heads per KV head must be 1, 2, 4, 8, 16, 32 or 64");
  if (need_ptrs && !scores && pg->batch > 0 && pg->max_kv_len > 0)
    return fail(SD_ERR_INVALID_ARGUMENT, "scores is NULL");
  return SD_OK;
}

sd_status run_score(const sd::ScoreArgs& a, sd_score_precision precision, hipStream_t st) {
  // the fast scorer max-accumulates its bound into row_bound (zeroed by the
  // caller, or by the selection's init kernel in the fused path); exact
  // scores carry no error and leave it alone
  if (precision == SD_SCORE_FAST && sd::score_fast_supported(a))
    return hip_status(sd::launch_score_fast(a, st), "score_fast");
  sd::ScoreArgs e = a;
  e.row_bound = nullptr;
  return hip_status(sd::launch_score_exact(e, st), "score_exact");
}

// ---------------------------------------------------------------- attention

struct AttnPlan {
  sd::AttnArgs a;
  bool mla;
  size_t ws_bytes;
};

sd_status plan_attn(const sd_pages* pg, const void* q, sd_dtype q_dtype, int32_t q_heads,
                    const sd_pool* k, const sd_pool* v, int32_t v_dim, const int32_t* indices,
                    int32_t k_sel, float scale, void* out, sd_dtype out_dtype, bool need_ptrs,
                    AttnPlan* plan) {
  sd_status st;
  if ((st = check_pool(k, "attention k")) != SD_OK) return st;
  if ((st = check_pool(v, "attention v")) != SD_OK) return st;
  if ((st = check_pages(pg, k->page_size)) != SD_OK) return st;
  if (v->page_size != k->page_size || v->num_kv_heads != k->num_kv_heads)
    return fail(SD_ERR_INVALID_ARGUMENT, "k and v pools must share page_size and num_kv_heads");
  if (k->dtype == SD_FP8_E4M3 || v->dtype == SD_FP8_E4M3)
    return fail(SD_ERR_UNSUPPORTED, "attention pools must be F32 or BF16 (FP8 pools are scored only)");
  if (k->dtype != v->dtype || q_dtype != k->dtype)
    return fail(SD_ERR_UNSUPPORTED, "q, k and v must have one dtype");
  if (q_heads <= 0 || q_heads % k->num_kv_heads)
    return fail(SD_ERR_INVALID_ARGUMENT, "q_heads %d is not a multiple of num_kv_heads", q_heads);
  if (v_dim <= 0 || v_dim > v->head_dim) return fail(SD_ERR_INVALID_ARGUMENT, "bad v_dim %d", v_dim);
  if (k_sel <= 0) return fail(SD_ERR_INVALID_ARGUMENT, "k_sel must be >= 1");
  if (out_dtype != SD_F32 && out_dtype != SD_BF16) return fail(SD_ERR_INVALID_ARGUMENT, "bad out dtype");
  if (need_ptrs) {
    if (!q || !indices || !out) return fail(SD_ERR_INVALID_ARGUMENT, "q, indices or out is NULL");
    if (!aligned16(q)) return fail(SD_ERR_INVALID_ARGUMENT, "q must be 16-byte aligned");
  }
  sd::AttnArgs a{};
  a.block_table = pg->block_table;
  a.kv_lens = pg->kv_lens;
  a.batch = pg->batch;
  a.max_pages = pg->max_pages;
  a.max_kv_len = pg->max_kv_len;
  a.q = q;
  a.q_heads = q_heads;
  a.dtype = k->dtype == SD_F32 ? 0 : 1;
  a.k = k->data;
  a.k_num_pages = k->num_pages;
  a.page_size = k->page_size;
  a.num_kv_heads = k->num_kv_heads;
  a.head_dim = k->head_dim;
  a.k_page_stride = k->page_stride;
  a.k_head_stride = k->head_stride;
  a.k_token_stride = k->token_stride;
  a.v = v->data;
  a.v_num_pages = v->num_pages;
  a.v_page_stride = v->page_stride;
  a.v_head_stride = v->head_stride;
  a.v_token_stride = v->token_stride;
  a.v_dim = v_dim;
  a.indices = indices;
  a.k_sel = k_sel;
  a.scale = scale;
  a.out = out;
  a.out_dtype = out_dtype == SD_F32 ? 0 : 1;
  const bool mla = sd::attn_mla_supported(a);
  if (!mla && !sd::attn_vec_supported(a))
    return fail(SD_ERR_UNSUPPORTED,
                "attention shape not supported: head_dim %d, v_dim %d, %d query heads per KV head "
                "(vector path: head_dim 64/128 = v_dim, 1/2/4/8 heads; MLA path: bf16 576/512, "
                "one shared latent pool, 32/64/128 heads)",
                k->head_dim, v_dim, q_heads / k->num_kv_heads);
  a.chunk = sd::attn_rows_per_split(a, mla);
  a.splits = (k_sel + a.chunk - 1) / a.chunk;
  const size_t parts = (size_t)pg->batch * q_heads * a.splits;
  // partial outputs: fp32, bf16 on the MLA path
  plan->ws_bytes = align_up(parts * (size_t)v_dim * (mla ? 2 : 4)) + align_up(parts * 2 * 4);
  plan->a = a;
  plan->mla = mla;
  return SD_OK;
}

void bind_attn_ws(AttnPlan* p, void* ws) {
  const size_t parts = (size_t)p->a.batch * p->a.q_heads * p->a.splits;
  char* base = static_cast<char*>(ws);
  p->a.part_o = reinterpret_cast<float*>(base);
  p->a.part_ml = reinterpret_cast<float*>(base + align_up(parts * (size_t)p->a.v_dim * (p->mla ? 2 : 4)));
}

// ---------------------------------------------------------------- fused plan

struct FusedPlan {
  sd::ScoreArgs score;
  bool fast;
  AttnPlan attn;
  int32_t groups;
  size_t off_scores, off_bound, off_slots, off_keys, off_idx, off_attn, total;
};

// Selection over finished scores: one launch for short exact rows, else
// statistics, histogram, classification and emission.
sd_status run_select(const sd::SelectArgs& a, hipStream_t stream) {
  if (sd::select_short_path(a)) return hip_status(sd::launch_select_short(a, stream), "select_short");
  sd_status s;
  if ((s = hip_status(sd::launch_select_init(a, stream), "select_init")) != SD_OK) return s;
  if ((s = hip_status(sd::launch_select_stats(a, stream), "select_stats")) != SD_OK) return s;
  return hip_status(sd::launch_select(a, stream), "select");
}

sd_status check_hint(const int32_t* hint, int32_t hint_len, int64_t hint_stride, const int32_t* writeback,
                     int64_t wb_stride, int32_t k) {
  if (hint && (hint_len < 0 || hint_stride < hint_len))
    return fail(SD_ERR_INVALID_ARGUMENT, "bad hint length %d / stride %lld", hint_len, (long long)hint_stride);
  if (writeback && wb_stride < k)
    return fail(SD_ERR_INVALID_ARGUMENT, "write-back stride %lld below k %d", (long long)wb_stride, k);
  return SD_OK;
}

sd_status topk_select_impl(const float* scores, int32_t batch, int32_t groups, int32_t row_stride,
                           const int32_t* kv_lens, int32_t k, const int32_t* hint, int32_t hint_len,
                           int64_t hint_stride, int32_t* indices, int32_t* counts, int32_t* writeback,
                           int64_t wb_stride, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  if (batch < 0 || groups <= 0 || row_stride < 0 || k <= 0)
    return fail(SD_ERR_INVALID_ARGUMENT, "bad sizes (batch %d, groups %d, row_stride %d, k %d)", batch,
                groups, row_stride, k);
  if (row_stride > sd::select_max_row())
    return fail(SD_ERR_UNSUPPORTED, "rows longer than %d tokens", sd::select_max_row());
  if (batch > 0 && (!scores || !kv_lens || !indices))
    return fail(SD_ERR_INVALID_ARGUMENT, "scores, kv_lens or indices is NULL");
  sd_status s = check_hint(hint, hint_len, hint_stride, writeback, wb_stride, k);
  if (s != SD_OK) return s;
  const size_t need = align_up(sd::select_workspace_bytes(batch * groups, row_stride));
  if (batch > 0 && (workspace_bytes < need || !workspace))
    return fail(SD_ERR_WORKSPACE_TOO_SMALL, "topk needs %zu workspace bytes", need);
  if (batch > 0 && !aligned16(workspace)) return fail(SD_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (batch == 0) return SD_OK;
  sd::SelectArgs a{};
  a.scores = scores;
  a.batch = batch;
  a.groups = groups;
  a.row_stride = row_stride;
  a.kv_lens = kv_lens;
  a.k = k;
  a.indices = indices;
  a.counts = counts;
  a.row_bound = nullptr;
  a.hint = hint;
  a.hint_len = hint ? hint_len : 0;
  a.hint_stride = hint_stride;
  a.writeback = writeback;
  a.wb_stride = wb_stride;
  sd::select_bind_workspace(&a, workspace);
  return run_select(a, stream);
}

struct TriPlan {
  int out_rows, out_batch, out_groups;
  size_t off_stats, off_lens, off_reduced, off_select, total;
};
sd_status plan_tri(int32_t layers, int32_t batch, int32_t groups, int32_t row_stride, sd_select_mode mode,
                   int32_t k, bool own_reduced, TriPlan* p) {
  if (layers <= 0 || batch < 0 || groups <= 0 || row_stride < 0 || k <= 0)
    return fail(SD_ERR_INVALID_ARGUMENT, "bad sizes (layers %d, batch %d, groups %d, row_stride %d, k %d)",
                layers, batch, groups, row_stride, k);
  if (mode != SD_SELECT_PER_LAYER_PERHEAD && mode != SD_SELECT_PER_HEAD && mode != SD_SELECT_UNION)
    return fail(SD_ERR_INVALID_ARGUMENT, "bad selection mode %d", (int)mode);
  if (row_stride > sd::select_max_row())
    return fail(SD_ERR_UNSUPPORTED, "rows longer than %d tokens", sd::select_max_row());
  if ((int64_t)layers * batch * groups > INT32_MAX / 2) return fail(SD_ERR_UNSUPPORTED, "too many rows");
  p->out_rows = sd::tri_out_rows(layers, batch, groups, (int)mode);
  p->out_batch = mode == SD_SELECT_PER_LAYER_PERHEAD ? layers * batch : batch;
  p->out_groups = mode == SD_SELECT_UNION ? 1 : groups;
  size_t off = 0;
  p->off_stats = off; off += align_up((size_t)layers * batch * groups * 32);
  p->off_lens = off; off += align_up((size_t)layers * batch * 4);
  p->off_reduced = off; off += own_reduced ? 0 : align_up((size_t)p->out_rows * row_stride * 4);
  p->off_select = off; off += align_up(sd::select_workspace_bytes(p->out_rows, row_stride));
  p->total = off;
  return SD_OK;
}

sd_status plan_fused(const sd_sparse_decode_args* x, bool need_ptrs, FusedPlan* f) {
  if (!x) return fail(SD_ERR_INVALID_ARGUMENT, "args is NULL");
  // the fused call scores into its own workspace: no scores pointer to check
  static const float kNonNull = 0.0f;
  sd_status st = check_score(&x->pages, &x->score_k, x->score_q, x->score_q_dtype, x->score_heads,
                             x->head_weights, x->mode, &kNonNull, need_ptrs);
  if (st != SD_OK) return st;
  if (x->topk <= 0) return fail(SD_ERR_INVALID_ARGUMENT, "topk must be >= 1");
  if ((st = check_hint(x->topk_hint, x->hint_len, x->hint_stride, x->topk_writeback, x->writeback_stride,
                       x->topk)) != SD_OK)
    return st;
  if (x->pages.max_kv_len > sd::select_max_row())
    return fail(SD_ERR_UNSUPPORTED, "max_kv_len above %d tokens", sd::select_max_row());
  if (x->precision != SD_SCORE_EXACT && x->precision != SD_SCORE_FAST)
    return fail(SD_ERR_INVALID_ARGUMENT, "bad precision");
  if (x->k.page_size != x->score_k.page_size)
    return fail(SD_ERR_INVALID_ARGUMENT, "score and attention pools must share the page size");
  if (x->k.num_kv_heads != x->score_k.num_kv_heads)
    return fail(SD_ERR_INVALID_ARGUMENT, "score and attention pools must have the same KV heads");
  const int32_t groups = x->score_k.num_kv_heads;
  // indices come from the selection step (caller buffer or workspace)
  static const int32_t kIdx = 0;
  st = plan_attn(&x->pages, x->q, x->q_dtype, x->q_heads, &x->k, &x->v, x->v_dim,
                 x->indices_out ? x->indices_out : &kIdx, x->topk, x->softmax_scale, x->out,
                 x->out_dtype, need_ptrs, &f->attn);
  if (st != SD_OK) return st;
  f->score = make_score_args(&x->pages, &x->score_k, x->score_q, x->score_heads, x->head_weights,
                             x->mode, x->head_scale, nullptr, nullptr);
  f->fast = x->precision == SD_SCORE_FAST && sd::score_fast_supported(f->score);
  f->groups = groups;
  const size_t rows = (size_t)x->pages.batch * groups;
  const size_t sc = align_up(rows * (size_t)x->pages.max_kv_len * 4);
  size_t off = 0;
  f->off_scores = off; off += sc;
  f->off_bound = off; off += align_up(rows * 4);
  f->off_slots = off;
  off += f->fast ? align_up(rows * (size_t)sd::score_fast_max_spans(x->pages.max_kv_len) * 16) : 0;
  f->off_keys = off; off += align_up(sd::select_workspace_bytes((int)rows, x->pages.max_kv_len));
  f->off_idx = off; off += x->indices_out ? 0 : align_up(rows * (size_t)x->topk * 4);
  f->off_attn = off; off += f->attn.ws_bytes;
  f->total = off;
  return SD_OK;
}

// Multi-query decode: next_n query tokens per request become next_n decode
// rows of one request each, row (b, j) seeing the first kv_len - (next_n - 1
// - j) tokens through request b's page table.  *y is the single-query call
// over those rows; with `expand` NULL its tables are placeholders (sizing).
// *mq = the bytes of the expanded tables, placed after f->total.
sd_status plan_multi_query(const sd_sparse_decode_args* x, bool need_ptrs, char* expand,
                           sd_sparse_decode_args* y, FusedPlan* f, size_t* mq) {
  if (!x) return fail(SD_ERR_INVALID_ARGUMENT, "args is NULL");
  if (x->next_n < 0 || x->next_n > 64) return fail(SD_ERR_INVALID_ARGUMENT, "next_n %d outside [0, 64]", x->next_n);
  *y = *x;
  *mq = 0;
  if (x->next_n <= 1) return plan_fused(y, need_ptrs, f);
  sd_status st = check_pages(&x->pages, x->score_k.page_size);
  if (st != SD_OK) return st;
  if (need_ptrs && x->pages.batch > 0 && (!x->pages.block_table || !x->pages.kv_lens))
    return fail(SD_ERR_INVALID_ARGUMENT, "block_table or kv_lens is NULL");
  const int64_t rows = (int64_t)x->pages.batch * x->next_n;
  if (rows > INT32_MAX / 2) return fail(SD_ERR_UNSUPPORTED, "too many decode rows");
  static const int32_t kPlaceholder[1] = {0};
  const size_t bt_bytes = align_up((size_t)rows * x->pages.max_pages * 4);
  y->pages.batch = (int32_t)rows;
  y->pages.block_table = expand ? reinterpret_cast<const int32_t*>(expand) : kPlaceholder;
  y->pages.kv_lens = expand ? reinterpret_cast<const int32_t*>(expand + bt_bytes) : kPlaceholder;
  y->next_n = 1;
  st = plan_fused(y, need_ptrs, f);
  if (st != SD_OK) return st;
  *mq = bt_bytes + align_up((size_t)rows * 4);
  return SD_OK;
}


}  // namespace

// ====================================================================== ABI

extern "C" {

const char* sd_status_string(sd_status s) {
  switch (s) {
    case SD_OK: return "ok";
    case SD_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SD_ERR_UNSUPPORTED: return "unsupported";
    case SD_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SD_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* sd_last_error(void) { return g_err.c_str(); }

int32_t sd_version(void) { return SD_VERSION; }

sd_status sd_sparse_score_paged(const sd_pages* pages, const sd_pool* k_pool, const void* q,
                                sd_dtype q_dtype, int32_t q_heads, const float* head_weights,
                                sd_score_mode mode, float head_scale,
                                sd_score_precision precision, float* scores, float* row_bound,
                                hipStream_t stream) {
  g_err.clear();
  sd_status st = check_score(pages, k_pool, q, q_dtype, q_heads, head_weights, mode, scores, true);
  if (st != SD_OK) return st;
  if (precision != SD_SCORE_EXACT && precision != SD_SCORE_FAST)
    return fail(SD_ERR_INVALID_ARGUMENT, "bad precision");
  const sd::ScoreArgs a = make_score_args(pages, k_pool, q, q_heads, head_weights, mode, head_scale,
                                          scores, row_bound);
  return run_score(a, precision, stream);
}

sd_status sd_topk_workspace_size(int32_t batch, int32_t groups, int32_t row_stride, int32_t k,
                                 size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(SD_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (batch < 0 || groups <= 0 || row_stride < 0 || k <= 0)
    return fail(SD_ERR_INVALID_ARGUMENT, "bad sizes");
  *bytes = align_up(sd::select_workspace_bytes(batch * groups, row_stride));
  return SD_OK;
}



sd_status sd_triattention_select_workspace_size(int32_t layers, int32_t batch, int32_t groups,
                                                int32_t row_stride, sd_select_mode mode, int32_t k,
                                                size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(SD_ERR_INVALID_ARGUMENT, "bytes is NULL");
  TriPlan p;
  sd_status st = plan_tri(layers, batch, groups, row_stride, mode, k, false, &p);
  if (st != SD_OK) return st;
  *bytes = p.total;
  return SD_OK;
}

sd_status sd_triattention_select(const float* scores, int32_t layers, int32_t batch, int32_t groups,
                                 int32_t row_stride, const int32_t* kv_lens, sd_select_mode mode,
                                 int32_t k, int32_t* indices, int32_t* counts, float* reduced_out,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  TriPlan p;
  sd_status st = plan_tri(layers, batch, groups, row_stride, mode, k, reduced_out != nullptr, &p);
  if (st != SD_OK) return st;
  if (batch > 0 && (!scores || !kv_lens || !indices))
    return fail(SD_ERR_INVALID_ARGUMENT, "scores, kv_lens or indices is NULL");
  if (batch > 0 && (workspace_bytes < p.total || !workspace))
    return fail(SD_ERR_WORKSPACE_TOO_SMALL, "triattention select needs %zu workspace bytes", p.total);
  if (batch > 0 && !aligned16(workspace)) return fail(SD_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (reduced_out && !aligned16(reduced_out))
    return fail(SD_ERR_INVALID_ARGUMENT, "reduced_out must be 16-byte aligned");
  if (batch == 0 || row_stride == 0) return SD_OK;
  char* ws = static_cast<char*>(workspace);
  sd::TriArgs t{};
  t.scores = scores;
  t.layers = layers;
  t.batch = batch;
  t.groups = groups;
  t.row_stride = row_stride;
  t.kv_lens = kv_lens;
  t.mode = (int32_t)mode;
  t.stats = reinterpret_cast<double*>(ws + p.off_stats);
  t.lens = mode == SD_SELECT_PER_LAYER_PERHEAD ? reinterpret_cast<int32_t*>(ws + p.off_lens) : nullptr;
  t.reduced = reduced_out ? reduced_out : reinterpret_cast<float*>(ws + p.off_reduced);
  t.want_reduced = reduced_out ? 1 : 0;
  // per layer and head, rows of one wave's registers are selected by the
  // normalization kernel itself
  // (SD_TRI_FUSE_SELECT=0, tests: the separate selection pass)
  const char* fuse_env = getenv("SD_TRI_FUSE_SELECT");
  const bool fused_select = sd::tri_fuses_select(t) && !(fuse_env && fuse_env[0] == '0');
  if (fused_select) {
    t.sel_k = k;
    t.sel_indices = indices;
    t.sel_counts = counts;
  }
  if ((st = hip_status(sd::launch_tri(t, stream), "triattention normalize/reduce")) != SD_OK) return st;
  if (fused_select) return SD_OK;
  sd::SelectArgs a{};
  a.scores = t.reduced;
  a.batch = p.out_batch;
  a.groups = p.out_groups;
  a.row_stride = row_stride;
  a.kv_lens = t.lens ? t.lens : kv_lens;
  a.k = k;
  a.indices = indices;
  a.counts = counts;
  sd::select_bind_workspace(&a, ws + p.off_select);
  return run_select(a, stream);
}

sd_status sd_topk_select(const float* scores, int32_t batch, int32_t groups, int32_t row_stride,
                         const int32_t* kv_lens, int32_t k, int32_t* indices, int32_t* counts,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return topk_select_impl(scores, batch, groups, row_stride, kv_lens, k, nullptr, 0, 0, indices, counts,
                          nullptr, 0, workspace, workspace_bytes, stream);
}

sd_status sd_topk_select_hinted(const float* scores, int32_t batch, int32_t groups, int32_t row_stride,
                                const int32_t* kv_lens, int32_t k, const int32_t* hint, int32_t hint_len,
                                int64_t hint_stride, int32_t* indices, int32_t* counts,
                                int32_t* writeback, int64_t writeback_stride, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return topk_select_impl(scores, batch, groups, row_stride, kv_lens, k, hint, hint_len, hint_stride, indices,
                          counts, writeback, writeback_stride, workspace, workspace_bytes, stream);
}

sd_status sd_sparse_decode_attn_workspace_size(const sd_pages* pages, int32_t q_heads,
                                               const sd_pool* k_pool, int32_t v_dim,
                                               int32_t k_sel, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(SD_ERR_INVALID_ARGUMENT, "bytes is NULL");
  AttnPlan p;
  sd_status st = plan_attn(pages, nullptr, k_pool ? k_pool->dtype : SD_F32, q_heads, k_pool, k_pool,
                           v_dim, nullptr, k_sel, 1.0f, nullptr, SD_F32, false, &p);
  if (st != SD_OK) return st;
  *bytes = p.ws_bytes;
  return SD_OK;
}

sd_status sd_sparse_decode_attn(const sd_pages* pages, const void* q, sd_dtype q_dtype,
                                int32_t q_heads, const sd_pool* k_pool, const sd_pool* v_pool,
                                int32_t v_dim, const int32_t* indices, int32_t k_sel,
                                float softmax_scale, void* out, sd_dtype out_dtype,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  AttnPlan p;
  sd_status st = plan_attn(pages, q, q_dtype, q_heads, k_pool, v_pool, v_dim, indices, k_sel,
                           softmax_scale, out, out_dtype, true, &p);
  if (st != SD_OK) return st;
  if (workspace_bytes < p.ws_bytes || (p.ws_bytes && !workspace))
    return fail(SD_ERR_WORKSPACE_TOO_SMALL, "attention needs %zu workspace bytes", p.ws_bytes);
  if (!aligned16(workspace)) return fail(SD_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  bind_attn_ws(&p, workspace);
  return hip_status(sd::launch_attn(p.a, stream), "attention");
}

sd_status sd_sparse_decode_attn_blocks_workspace_size(const sd_pages* pages, int32_t q_heads,
                                                      const sd_pool* k_pool, int32_t v_dim, int32_t k_blocks,
                                                      int32_t block_size, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(SD_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (k_blocks <= 0 || block_size <= 0 || (int64_t)k_blocks * block_size > (1 << 24))
    return fail(SD_ERR_INVALID_ARGUMENT, "bad k_blocks %d / block_size %d", k_blocks, block_size);
  if (!pages || !k_pool) return fail(SD_ERR_INVALID_ARGUMENT, "pages or k_pool is NULL");
  AttnPlan p;
  sd_status st = plan_attn(pages, nullptr, k_pool->dtype, q_heads, k_pool, k_pool, v_dim, nullptr,
                           k_blocks * block_size, 1.0f, nullptr, SD_F32, false, &p);
  if (st != SD_OK) return st;
  *bytes = align_up((size_t)pages->batch * k_pool->num_kv_heads * k_blocks * block_size * 4) + p.ws_bytes;
  return SD_OK;
}

sd_status sd_sparse_decode_attn_blocks(const sd_pages* pages, const void* q, sd_dtype q_dtype,
                                       int32_t q_heads, const sd_pool* k_pool, const sd_pool* v_pool,
                                       int32_t v_dim, const int32_t* block_indices, int32_t k_blocks,
                                       int32_t block_size, float softmax_scale, void* out, sd_dtype out_dtype,
                                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err.clear();
  if (k_blocks <= 0 || block_size <= 0 || (int64_t)k_blocks * block_size > (1 << 24))
    return fail(SD_ERR_INVALID_ARGUMENT, "bad k_blocks %d / block_size %d", k_blocks, block_size);
  if (!pages || !k_pool) return fail(SD_ERR_INVALID_ARGUMENT, "pages or k_pool is NULL");
  if (pages->batch > 0 && !block_indices) return fail(SD_ERR_INVALID_ARGUMENT, "block_indices is NULL");
  const int32_t k_sel = k_blocks * block_size;
  const size_t tok_bytes = align_up((size_t)pages->batch * k_pool->num_kv_heads * k_sel * 4);
  static const int32_t kIdx = 0;
  AttnPlan p;
  sd_status st = plan_attn(pages, q, q_dtype, q_heads, k_pool, v_pool, v_dim, &kIdx, k_sel, softmax_scale,
                           out, out_dtype, true, &p);
  if (st != SD_OK) return st;
  if (workspace_bytes < tok_bytes + p.ws_bytes || !workspace)
    return fail(SD_ERR_WORKSPACE_TOO_SMALL, "block attention needs %zu workspace bytes", tok_bytes + p.ws_bytes);
  if (!aligned16(workspace)) return fail(SD_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (pages->batch == 0) return SD_OK;
  // block entry i -> its tokens i*block_size + r (those below kv_len), -1 otherwise
  char* ws = static_cast<char*>(workspace);
  int32_t* tok = reinterpret_cast<int32_t*>(ws);
  st = hip_status(sd::launch_expand_blocks(block_indices, pages->kv_lens, pages->batch, k_pool->num_kv_heads,
                                           k_blocks, block_size, pages->max_kv_len, tok, stream),
                  "block expand");
  if (st != SD_OK) return st;
  p.a.indices = tok;
  bind_attn_ws(&p, ws + tok_bytes);
  return hip_status(sd::launch_attn(p.a, stream), "attention");
}

sd_status sd_sparse_decode_workspace_size(const sd_sparse_decode_args* args, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(SD_ERR_INVALID_ARGUMENT, "bytes is NULL");
  sd_sparse_decode_args y;
  FusedPlan f;
  size_t mq = 0;
  sd_status st = plan_multi_query(args, false, nullptr, &y, &f, &mq);
  if (st != SD_OK) return st;
  *bytes = f.total + mq;
  return SD_OK;
}

}  // extern "C"

namespace {

// The fused step on a validated plan (plan_multi_query with pointers) and a
// workspace of at least f.total + mq bytes.
sd_status run_sparse_decode(const sd_sparse_decode_args* args, sd_sparse_decode_args y, FusedPlan f,
                            size_t mq, char* ws, hipStream_t stream) {
  sd_status st = SD_OK;
  if (args->pages.batch == 0) return SD_OK;
  if (mq) {
    // one decode row per (request, query token): the page tables repeated
    // and the causal lengths, at the end of the workspace; then plan again
    // with those pointers
    if ((st = plan_multi_query(args, true, ws + f.total, &y, &f, &mq)) != SD_OK) return st;
    const int n = args->next_n;
    st = hip_status(sd::launch_mq_expand(args->pages.block_table, args->pages.kv_lens, args->pages.batch,
                                         args->pages.max_pages, n, const_cast<int32_t*>(y.pages.block_table),
                                         const_cast<int32_t*>(y.pages.kv_lens), stream),
                    "multi-query expand");
    if (st != SD_OK) return st;
  }
  const sd_sparse_decode_args* x = &y;
  float* scores = reinterpret_cast<float*>(ws + f.off_scores);
  float* bound = reinterpret_cast<float*>(ws + f.off_bound);
  int32_t* idx = x->indices_out ? x->indices_out : reinterpret_cast<int32_t*>(ws + f.off_idx);

  // 1. score (also the row min / max keys and the selection statistics
  // cleared: by the fast scorer's blocks, else a small init pass first)
  sd::SelectArgs t{};
  t.scores = scores;
  t.batch = x->pages.batch;
  t.groups = f.groups;
  t.row_stride = x->pages.max_kv_len;
  t.kv_lens = x->pages.kv_lens;
  t.k = x->topk;
  t.indices = idx;
  t.counts = x->counts_out;
  t.row_bound = f.fast ? bound : nullptr;
  t.hint = x->topk_hint;
  t.hint_len = x->topk_hint ? x->hint_len : 0;
  t.hint_stride = x->hint_stride;
  t.writeback = x->topk_writeback;
  t.wb_stride = x->writeback_stride;
  sd::select_bind_workspace(&t, ws + f.off_keys);
  // short exact rows are selected in one launch that needs no statistics
  const bool short_rows = sd::select_short_path(t);
  f.score.scores = scores;
  f.score.row_bound = nullptr;
  f.score.row_stats = short_rows ? nullptr : t.stats;
  f.score.span_slots = nullptr;
  if (f.fast && x->pages.max_kv_len > 0) {
    // per-block slots that the histogram pass reduces into the row's keys and bound
    f.score.span_slots = reinterpret_cast<int32_t*>(ws + f.off_slots);
    t.span_slots = f.score.span_slots;
    t.nspans = sd::score_fast_spans(f.score);
  } else if (!short_rows) {
    if ((st = hip_status(sd::launch_select_init(t, stream), "select_init")) != SD_OK) return st;
    f.score.row_bound = f.fast ? bound : nullptr;
  }
  st = run_score(f.score, f.fast ? SD_SCORE_FAST : SD_SCORE_EXACT, stream);
  if (st != SD_OK) return st;
  // 2. select (exactly, also from fast scores)
  t.score = f.score;
  st = short_rows ? hip_status(sd::launch_select_short(t, stream), "select_short")
                  : hip_status(sd::launch_select(t, stream), "select");
  if (st != SD_OK) return st;
  // 3. attend
  f.attn.a.indices = idx;
  bind_attn_ws(&f.attn, ws + f.off_attn);
  return hip_status(sd::launch_attn(f.attn.a, stream), "attention");
}

// Scratch of the allocation-free fused step: one array per device (each GPU
// the library runs on holds its own copy until the process ends), shared by
// every call on that device.  In host code `sd_noalloc_scratch` names a
// host-side stand-in, not device memory: the kernels get the device address
// that hipGetSymbolAddress returns for the current device, looked up once
// per device and kept.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

sd_status noalloc_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (stream) {
    hipDevice_t sdev = -1;
    if ((e = hipStreamGetDevice(stream, &sdev)) != hipSuccess) return hip_status(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(SD_ERR_INVALID_ARGUMENT, "stream belongs to device %d but device %d is current", (int)sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(SD_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(sd_noalloc_scratch))) != hipSuccess)
      return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SD_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SD_OK;
}

}  // namespace

extern "C" {

sd_status sd_sparse_decode(const sd_sparse_decode_args* args, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  g_err.clear();
  sd_sparse_decode_args y;
  FusedPlan f;
  size_t mq = 0;
  sd_status st = plan_multi_query(args, true, nullptr, &y, &f, &mq);
  if (st != SD_OK) return st;
  if (workspace_bytes < f.total + mq || (f.total + mq && !workspace))
    return fail(SD_ERR_WORKSPACE_TOO_SMALL, "sparse_decode needs %zu workspace bytes", f.total + mq);
  if (!aligned16(workspace)) return fail(SD_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  return run_sparse_decode(args, y, f, mq, static_cast<char*>(workspace), stream);
}

size_t sd_sparse_decode_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

sd_status sd_sparse_decode_noalloc(const sd_sparse_decode_args* args, hipStream_t stream) {
  g_err.clear();
  sd_sparse_decode_args y;
  FusedPlan f;
  size_t mq = 0;
  sd_status st = plan_multi_query(args, true, nullptr, &y, &f, &mq);
  if (st != SD_OK) return st;
  if (f.total + mq > kNoAllocScratchBytes)
    return fail(SD_ERR_WORKSPACE_TOO_SMALL,
                "sparse_decode_noalloc: this call needs %zu bytes of scratch, more than the %zu the library holds "
                "per device; use sd_sparse_decode with a caller workspace",
                f.total + mq, kNoAllocScratchBytes);
  if (args->pages.batch == 0) return SD_OK;
  void* scratch = nullptr;
  if ((st = noalloc_scratch(stream, &scratch)) != SD_OK) return st;
  return run_sparse_decode(args, y, f, mq, static_cast<char*>(scratch), stream);
}

sd_status sd_local_to_global(const sd_pages* pages, int32_t page_size, int32_t num_pages,
                             const int32_t* local, int32_t groups, int32_t k, int64_t* global_out,
                             hipStream_t stream) {
  g_err.clear();
  if (!pages) return fail(SD_ERR_INVALID_ARGUMENT, "pages is NULL");
  if (page_size <= 0 || num_pages < 0 || groups <= 0 || k <= 0 || pages->batch < 0 || pages->max_pages < 0)
    return fail(SD_ERR_INVALID_ARGUMENT, "bad sizes");
  if (pages->batch > 0 && (!pages->block_table || !local || !global_out))
    return fail(SD_ERR_INVALID_ARGUMENT, "block_table, local or global_out is NULL");
  return hip_status(sd::launch_local_to_global(pages->block_table, pages->max_pages, pages->batch, page_size,
                                               num_pages, local, groups, k, global_out, stream),
                    "local_to_global");
}

}  // extern "C"

// ====================================================================== small kernels

namespace sd {

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ void mq_expand_kernel(const int32_t* bt, const int32_t* kv_lens, int32_t max_pages, int32_t n,
                                 int32_t* bt_out, int32_t* kv_out) {
  const int r = blockIdx.x, b = r / n, j = r % n;
  for (int i = threadIdx.x; i < max_pages; i += blockDim.x)
    bt_out[(int64_t)r * max_pages + i] = bt[(int64_t)b * max_pages + i];
  if (threadIdx.x == 0) kv_out[r] = max(kv_lens[b] - (n - 1 - j), 0);
}

hipError_t launch_mq_expand(const int32_t* bt, const int32_t* kv_lens, int32_t batch, int32_t max_pages,
                            int32_t n, int32_t* bt_out, int32_t* kv_out, hipStream_t st) {
  if (batch == 0) return hipSuccess;
  mq_expand_kernel<<<batch * n, 256, 0, st>>>(bt, kv_lens, max_pages, n, bt_out, kv_out);
  return hipGetLastError();
}

__global__ void expand_blocks_kernel(const int32_t* blocks, const int32_t* kv_lens, int32_t groups,
                                     int32_t k_blocks, int32_t bs, int32_t cap, int64_t total, int32_t* tok) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // token slot
  if (i >= total) return;
  const int64_t per_row = (int64_t)k_blocks * bs;
  const int64_t row = i / per_row;
  const int slot = (int)(i % per_row);
  const int b = (int)(row / groups);
  const int L = clamp_len(kv_lens[b], cap);
  const int e = blocks[row * k_blocks + slot / bs];
  const int64_t t = (int64_t)e * bs + slot % bs;
  tok[i] = (e >= 0 && t < L) ? (int32_t)t : -1;
}

hipError_t launch_expand_blocks(const int32_t* blocks, const int32_t* kv_lens, int32_t batch, int32_t groups,
                                int32_t k_blocks, int32_t block_size, int32_t cap, int32_t* tok, hipStream_t st) {
  const int64_t total = (int64_t)batch * groups * k_blocks * block_size;
  if (total == 0) return hipSuccess;
  expand_blocks_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(blocks, kv_lens, groups, k_blocks,
                                                                        block_size, cap, total, tok);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  fill_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(p, n, v);
  return hipGetLastError();
}

__global__ void local_to_global_kernel(const int32_t* bt, int32_t max_pages, int32_t page_size,
                                       int32_t num_pages, const int32_t* local, int32_t per_req,
                                       int64_t total, int64_t* out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int b = (int)(i / per_req);
  const int t = local[i];
  int64_t r = -1;
  if (t >= 0 && t / page_size < max_pages) {
    const int page = bt[(int64_t)b * max_pages + t / page_size];
    if (page >= 0 && page < num_pages) r = (int64_t)page * page_size + t % page_size;
  }
  out[i] = r;
}

hipError_t launch_local_to_global(const int32_t* bt, int32_t max_pages, int32_t batch,
                                  int32_t page_size, int32_t num_pages, const int32_t* local,
                                  int32_t groups, int32_t k, int64_t* out, hipStream_t st) {
  const int64_t per_req = (int64_t)groups * k;
  const int64_t total = (int64_t)batch * per_req;
  if (total == 0) return hipSuccess;
  local_to_global_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(
      bt, max_pages, page_size, num_pages, local, (int32_t)per_req, total, out);
  return hipGetLastError();
}

}  // namespace sd
