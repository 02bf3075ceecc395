// topk.hip -- per-row top-k selection with deterministic tie settlement.
//
// Selection keeps, per (request, KV head) row, the min(k, kv_len) positions
// that come first in (score descending, position ascending) order, and
// writes them in ascending position order padded with -1 ("Add TriAttention
// KV-cache compression method", Summary: TopK / tie settlement; Test Plan:
// deterministic heavy-tie settlement; the indices feed core sparse attention
// as in "Overlap DSA heuristic prev_topk write-back on the aux stream",
// Description).
//
// Method: radix select on order-preserving 32-bit keys (11 + 11 + 10 bits)
// finds the k-th largest key K* and how many of the keys equal to K* are
// kept (the lowest positions first); an ordered compaction then emits every
// position with key > K* plus the first `need` positions with key == K*.
//
// Exact selection from fast scores: given fast scores s~ with |s~ - s| <= d
// for every token of a row (s the exact score) and T~ the k-th largest s~,
// the exact k-th score T lies in [T~ - d, T~ + d].  Tokens with s~ > T~ + 2d
// are certainly kept, tokens with s~ < T~ - 2d certainly dropped; the rest
// (the band) are re-scored in the exact order.  Replacing kept scores by
// +inf and dropped ones by -inf and running the exact selection above on the
// result gives exactly the top-k of the exact scores.
#include "common.h"
#include "kernels.h"

namespace sd {

constexpr int kTopkThreads = 1024;

struct RadixResult {
  uint32_t key;  // k-th largest key
  int need;      // how many keys equal to `key` are kept
};

// Block-wide radix select of the k-th largest key among s[0..L).  Requires
// k <= L.  hist needs 2048 ints; tmp 16 ints; win 2 ints.
__device__ RadixResult radix_select_kth(const float* __restrict__ s, int L, int k, int* hist,
                                        int* tmp, int* win) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;
  const int shifts[3] = {21, 10, 0};
  const int nbits[3] = {11, 11, 10};
#pragma unroll 1
  for (int p = 0; p < 3; ++p) {
    const int shift = shifts[p];
    const int nb = 1 << nbits[p];
    for (int i = tid; i < 2048; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    for (int t = tid; t < L; t += kTopkThreads) {
      const uint32_t key = score_key(s[t]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (nb - 1)], 1);
    }
    __syncthreads();
    // bins in descending order: thread i owns bins nb-1-2i and nb-2-2i
    int c0 = 0, c1 = 0;
    const int b0 = nb - 1 - 2 * tid, b1 = nb - 2 - 2 * tid;
    if (b0 >= 0) c0 = hist[b0];
    if (b1 >= 0) c1 = hist[b1];
    int total;
    const int excl = block_excl_scan<kTopkThreads>(c0 + c1, tmp, &total);
    if (b0 >= 0 && excl < remaining && remaining <= excl + c0) {
      win[0] = b0;
      win[1] = excl;
    }
    if (b1 >= 0 && excl + c0 < remaining && remaining <= excl + c0 + c1) {
      win[0] = b1;
      win[1] = excl + c0;
    }
    __syncthreads();
    const int bin = win[0];
    remaining -= win[1];
    prefix |= (uint32_t)bin << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    __syncthreads();
  }
  return RadixResult{prefix, remaining};
}

// Ordered compaction of the kept positions of one row into out[0..k).
__device__ void emit_selected(const float* __restrict__ s, int L, uint32_t kth, int need,
                              int32_t* __restrict__ out, int* tmp) {
  const int tid = threadIdx.x;
  const int seg = (L + kTopkThreads - 1) / kTopkThreads;
  const int t0 = min(L, tid * seg), t1 = min(L, t0 + seg);
  int gt = 0, eq = 0;
  for (int t = t0; t < t1; ++t) {
    const uint32_t key = score_key(s[t]);
    gt += key > kth;
    eq += key == kth;
  }
  int total;
  const int eq_before = block_excl_scan<kTopkThreads>(eq, tmp, &total);
  const int take_eq = max(0, min(eq, need - eq_before));
  int pos = block_excl_scan<kTopkThreads>(gt + take_eq, tmp, &total);
  int taken = 0;
  for (int t = t0; t < t1; ++t) {
    const uint32_t key = score_key(s[t]);
    if (key > kth) {
      out[pos++] = t;
    } else if (key == kth && taken < take_eq) {
      out[pos++] = t;
      ++taken;
    }
  }
}

__global__ __launch_bounds__(kTopkThreads) void topk_row_kernel(TopkArgs a) {
  __shared__ int hist[2048];
  __shared__ int tmp[16];
  __shared__ int win[2];
  const int row = blockIdx.x;
  const int b = row / a.groups;
  const int L = clamp_len(a.kv_lens[b], a.row_stride);
  const int k = a.k;
  int32_t* out = a.indices + (int64_t)row * k;
  if (L <= k) {
    for (int i = threadIdx.x; i < k; i += kTopkThreads) out[i] = i < L ? i : -1;
    if (a.counts && threadIdx.x == 0) a.counts[row] = L;
    return;
  }
  const float* s = a.scores + (int64_t)row * a.row_stride;
  const RadixResult r = radix_select_kth(s, L, k, hist, tmp, win);
  emit_selected(s, L, r.key, r.need, out, tmp);
  if (a.counts && threadIdx.x == 0) a.counts[row] = k;
}

// k-th largest fast score per row (rows with kv_len <= k need none).
__global__ __launch_bounds__(kTopkThreads) void topk_threshold_kernel(TopkArgs a, float* thr) {
  __shared__ int hist[2048];
  __shared__ int tmp[16];
  __shared__ int win[2];
  const int row = blockIdx.x;
  const int b = row / a.groups;
  const int L = clamp_len(a.kv_lens[b], a.row_stride);
  if (L <= a.k) {
    if (threadIdx.x == 0) thr[row] = -__builtin_inff();
    return;
  }
  const float* s = a.scores + (int64_t)row * a.row_stride;
  const RadixResult r = radix_select_kth(s, L, a.k, hist, tmp, win);
  if (threadIdx.x == 0) thr[row] = key_to_score(r.key);
}

// Replace each fast score by +inf (certainly kept), -inf (certainly
// dropped) or its exact score (band).  One wave per 64 tokens; the band
// tokens of a wave are re-scored one at a time by the whole wave: lane h
// evaluates head h's dot product left to right, then one lane adds the
// group's weighted ReLU terms in head order.
__global__ __launch_bounds__(256) void refine_band_kernel(RefineArgs a) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const ScoreArgs& sa = a.score;
  const int row = blockIdx.y;
  const int b = row / sa.num_kv_heads, g = row % sa.num_kv_heads;
  const int cap = min(sa.max_kv_len, sa.max_pages * sa.page_size);
  const int L = clamp_len(sa.kv_lens[b], cap);
  const int t = (blockIdx.x * 4 + wid) * kWave + lane;
  if ((blockIdx.x * 4 + wid) * kWave >= L) return;
  const float* srow = sa.scores + (int64_t)row * sa.max_kv_len;
  float* rrow = a.refined + (int64_t)row * sa.max_kv_len;
  const bool live = t < L;
  float fast = live ? srow[t] : -__builtin_inff();
  if (L <= a.k) {  // every token is kept: the values do not matter
    if (live) rrow[t] = fast;
    return;
  }
  const double d2 = 2.0 * (double)a.row_bound[row];
  const double diff = (double)fast - (double)a.thr[row];
  float out;
  bool band = false;
  if (!live || fast == -__builtin_inff()) {
    out = -__builtin_inff();
  } else if (diff > d2) {
    out = __builtin_inff();
  } else if (diff < -d2) {
    out = -__builtin_inff();
  } else {
    band = true;
    out = 0.0f;
  }
  // exact re-score of the band tokens of this wave
  const int G = sa.q_heads / sa.num_kv_heads;
  uint64_t mask = __ballot(band);
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(sa.q) + ((int64_t)b * sa.q_heads + g * G) * 128;
  const float* wb = sa.head_weights + (int64_t)b * sa.q_heads + g * G;
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(sa.k) + (int64_t)g * sa.head_stride;
  const int32_t* bt = sa.block_table + (int64_t)b * sa.max_pages;
  while (mask) {
    const int src = __builtin_ctzll(mask);
    mask &= mask - 1;
    const int tt = (blockIdx.x * 4 + wid) * kWave + src;
    const int page = bt[tt / sa.page_size];
    const uint16_t* krow =
        kbase + (int64_t)page * sa.page_stride + (int64_t)(tt % sa.page_size) * sa.token_stride;
    float total = 0.0f;
    for (int h0 = 0; h0 < G; h0 += kWave) {
      const int h = h0 + lane;
      float term = 0.0f;
      if (h < G) {
        const uint16_t* qh = qb + (int64_t)h * 128;
        float acc = 0.0f;
        for (int d = 0; d < 128; d += 8) {
          const uint4 kv = *reinterpret_cast<const uint4*>(krow + d);
          const uint4 qv = *reinterpret_cast<const uint4*>(qh + d);
          acc = __builtin_fmaf(bf16_lo(qv.x), bf16_lo(kv.x), acc);
          acc = __builtin_fmaf(bf16_hi(qv.x), bf16_hi(kv.x), acc);
          acc = __builtin_fmaf(bf16_lo(qv.y), bf16_lo(kv.y), acc);
          acc = __builtin_fmaf(bf16_hi(qv.y), bf16_hi(kv.y), acc);
          acc = __builtin_fmaf(bf16_lo(qv.z), bf16_lo(kv.z), acc);
          acc = __builtin_fmaf(bf16_hi(qv.z), bf16_hi(kv.z), acc);
          acc = __builtin_fmaf(bf16_lo(qv.w), bf16_lo(kv.w), acc);
          acc = __builtin_fmaf(bf16_hi(qv.w), bf16_hi(kv.w), acc);
        }
        const float r = acc > 0.0f ? acc : 0.0f;
        term = __fmul_rn(wb[h], r);
      }
      const int n = min(kWave, G - h0);
      for (int j = 0; j < n; ++j) total = __fadd_rn(total, __shfl(term, j));
    }
    if (lane == src) out = total;
  }
  if (live) rrow[t] = out;
}

// ------------------------------------------------------------------ launch

hipError_t launch_topk(const TopkArgs& a, hipStream_t st) {
  const int rows = a.batch * a.groups;
  if (rows == 0) return hipSuccess;
  topk_row_kernel<<<rows, kTopkThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_topk_threshold(const TopkArgs& a, float* thr, hipStream_t st) {
  const int rows = a.batch * a.groups;
  if (rows == 0) return hipSuccess;
  topk_threshold_kernel<<<rows, kTopkThreads, 0, st>>>(a, thr);
  return hipGetLastError();
}

hipError_t launch_refine_band(const RefineArgs& a, hipStream_t st) {
  const ScoreArgs& s = a.score;
  if (s.batch == 0 || s.max_kv_len == 0) return hipSuccess;
  dim3 grid((s.max_kv_len + 255) / 256, s.batch * s.num_kv_heads);
  refine_band_kernel<<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sd
