// topk.hip -- per-row top-k selection with deterministic tie settlement.
//
// Selection keeps, per (request, KV head) row, the min(k, kv_len) positions
// that come first in (score descending, position ascending) order, and
// writes them in ascending position order padded with -1 ("Add TriAttention
// KV-cache compression method", Summary: TopK / tie settlement; Test Plan:
// deterministic heavy-tie settlement; the indices then feed core sparse
// attention as in "Overlap DSA heuristic prev_topk write-back on the aux
// stream", Description).
//
// One 512-thread block per row.  Thread `tid` owns the float4 groups
// t = sc*2048*NI + i*2048 + 4*tid + e (super-chunk sc, tile i, element e), so
// every load is a coalesced float4.  Rows up to 16 tiles (32768 tokens) stay
// in registers; longer rows are re-read from L2 in each pass that needs the
// values (up to 4 super-chunks of 65536).  Steps:
//   1. min / max / count of the finite scores;
//   2. a 2048-bin histogram that is linear in the score value over [min,max]
//      (value-linear bins keep LDS-atomic contention low where exponent bins
//      would put a whole row into a handful of bins), and the bin B* that
//      holds the k-th largest score;
//   3. every token is classed IN (certainly kept), OUT (certainly dropped) or
//      BAND (decided exactly below), and IN is counted;
//   4. a radix select (11+11+10 bits) over the order-preserving keys of the
//      BAND tokens only finds the key K* of the last kept token and how many
//      BAND tokens equal to K* are kept (the lowest positions);
//   5. ordered emission, one block scan per 2048-token tile.
//
// Exact scores: BAND = bin B*, IN = bins above, OUT = bins below.
// Fast scores s~ with |s~ - s| <= d on every token of the row (d from the
// scorer): with [lo*, hi*] the range of s~ inside bin B*, the k-th largest s~
// lies in [lo*, hi*], so the exact k-th score T lies in [lo* - d, hi* + d].
// A token with s~ > hi* + 2d has s > T (kept); one with s~ < lo* - 2d has
// s < T (dropped); the tokens in between are re-scored in the exact order
// (one wave per token: lane h evaluates head h's dot product left to right,
// then the head terms are added in head order) and selected on exact keys.
// The result is exactly the top-k of the exact scores.
#include <stdlib.h>

#include "common.h"
#include "kernels.h"
#include "wave_select.h"

namespace sd {

constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kBins = 2048;
constexpr int kTile = 4 * kSelThreads;  // tokens per tile (one float4 per thread)
constexpr int kMaxNI = 32;              // tiles held in registers: rows up to 65536
constexpr int kMaxChunks = 4;           // longer rows: up to 4 super-chunks, re-read per pass
enum : uint32_t { kOut = 0, kIn = 1, kBand = 2, kPad = 3 };

// Slot i of a row's output, and of its copy for the next step's hint when
// the caller asked for one (the write-back rides along with the output
// stores instead of a copy kernel after them).
__device__ __forceinline__ void put_index(const SelectArgs& a, int row, int i, int v) {
  a.indices[(int64_t)row * a.k + i] = v;
  if (a.writeback) a.writeback[(int64_t)row * a.wb_stride + i] = v;
}

constexpr int kRankMax = 512;  // band sizes the one-block path ranks directly
template <int NCLS>
struct SelSharedN {
  int hist[kBins];
  int tmp[kSelWaves];
  int win[2];
  float redf[2][kSelWaves];
  int redi[kSelWaves];
  uint8_t cls[NCLS];  // 4 x 2-bit classes per byte
  // a short band: (key << 32) | ~position per entry and whether it is kept
  uint64_t rkey[kRankMax];
  uint8_t rkeep[kRankMax];
  int rcount;
};
// the whole-row path at the longest rows; shorter rows need NI * kSelThreads bytes of classes
using SelShared = SelSharedN<kMaxChunks * kMaxNI * kSelThreads>;

template <typename SH>
__device__ __forceinline__ float block_min_f(float v, SH& sh) {
  v = fminf(v, __shfl_xor(v, 32)); v = fminf(v, __shfl_xor(v, 16)); v = fminf(v, __shfl_xor(v, 8));
  v = fminf(v, __shfl_xor(v, 4)); v = fminf(v, __shfl_xor(v, 2)); v = fminf(v, __shfl_xor(v, 1));
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) sh.redf[0][wid] = v;
  __syncthreads();
  float r = sh.redf[0][0];
  for (int w = 1; w < kSelWaves; ++w) r = fminf(r, sh.redf[0][w]);
  __syncthreads();
  return r;
}
template <typename SH>
__device__ __forceinline__ float block_max_f(float v, SH& sh) {
  v = fmaxf(v, __shfl_xor(v, 32)); v = fmaxf(v, __shfl_xor(v, 16)); v = fmaxf(v, __shfl_xor(v, 8));
  v = fmaxf(v, __shfl_xor(v, 4)); v = fmaxf(v, __shfl_xor(v, 2)); v = fmaxf(v, __shfl_xor(v, 1));
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) sh.redf[1][wid] = v;
  __syncthreads();
  float r = sh.redf[1][0];
  for (int w = 1; w < kSelWaves; ++w) r = fmaxf(r, sh.redf[1][w]);
  __syncthreads();
  return r;
}
template <typename SH>
__device__ __forceinline__ int block_sum_i(int v, SH& sh) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) sh.redi[wid] = v;
  __syncthreads();
  int r = 0;
  for (int w = 0; w < kSelWaves; ++w) r += sh.redi[w];
  __syncthreads();
  return r;
}

// min, max and sum over the block in one exchange (one pair of barriers)
template <typename SH>
__device__ __forceinline__ void block_min_max_sum(float& lo, float& hi, int& n, SH& sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o));
    hi = fmaxf(hi, __shfl_xor(hi, o));
    n += __shfl_xor(n, o);
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) {
    sh.redf[0][wid] = lo;
    sh.redf[1][wid] = hi;
    sh.redi[wid] = n;
  }
  __syncthreads();
  lo = sh.redf[0][0];
  hi = sh.redf[1][0];
  n = sh.redi[0];
  for (int w = 1; w < kSelWaves; ++w) {
    lo = fminf(lo, sh.redf[0][w]);
    hi = fmaxf(hi, sh.redf[1][w]);
    n += sh.redi[w];
  }
  __syncthreads();
}

// Neighbouring binary32 values (finite inputs).
__device__ __forceinline__ float next_up(float x) {
  const uint32_t u = __float_as_uint(x);
  if (x == 0.0f) return __uint_as_float(1u);
  return __uint_as_float((u & 0x80000000u) ? u - 1u : u + 1u);
}
__device__ __forceinline__ float next_down(float x) { return -next_up(-x); }

// LDS histogram increment; when every active lane of the wave hits the same
// bin (ties, constant rows) one lane adds the whole count.
__device__ __forceinline__ void hist_add(int* hist, int bin, bool active) {
  const uint64_t act = __ballot(active);
  if (!act) return;
  const int first = __shfl(bin, __builtin_ctzll(act));
  const uint64_t same = __ballot(active && bin == first);
  if (same == act) {
    if ((threadIdx.x & 63) == __builtin_ctzll(act)) atomicAdd(&hist[first], __popcll(act));
  } else if (active) {
    atomicAdd(&hist[bin], 1);
  }
}

// Find, over bins in descending order, the bin holding the `want`-th
// element (1-based); returns (bin, count strictly above it) via sh.win.
template <typename SH>
__device__ __forceinline__ void find_bin(SH& sh, int nb, int want) {
  constexpr int BPT = kBins / kSelThreads;  // bins per thread
  const int tid = threadIdx.x;
  int c[BPT];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int bin = nb - 1 - (tid * BPT + j);
    c[j] = bin >= 0 ? sh.hist[bin] : 0;
    sum += c[j];
  }
  int total;
  int excl = block_excl_scan<kSelThreads>(sum, sh.tmp, &total);
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int bin = nb - 1 - (tid * BPT + j);
    if (bin >= 0 && excl < want && want <= excl + c[j]) {
      sh.win[0] = bin;
      sh.win[1] = excl;
    }
    excl += c[j];
  }
  __syncthreads();
}

// find_bin for any block size NT, on a plain histogram array
template <int NT>
__device__ __forceinline__ void find_bin_n(const int* hist, int* tmp, int* win, int nb, int want) {
  constexpr int BPT = kBins / NT;
  const int tid = threadIdx.x;
  int c[BPT];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int bin = nb - 1 - (tid * BPT + j);
    c[j] = bin >= 0 ? hist[bin] : 0;
    sum += c[j];
  }
  int total;
  int excl = block_excl_scan<NT>(sum, tmp, &total);
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int bin = nb - 1 - (tid * BPT + j);
    if (bin >= 0 && excl < want && want <= excl + c[j]) {
      win[0] = bin;
      win[1] = excl;
    }
    excl += c[j];
  }
  __syncthreads();
}

// acc + q * k over eight (bf16 q, binary32 k) pairs in order, each product
// and each sum rounded once (k is a dequantized fp8 element).
__device__ __forceinline__ float dot8_f32k(float acc, uint4 qv, const float* k) {
  acc = __fadd_rn(acc, __fmul_rn(bf16_lo(qv.x), k[0]));
  acc = __fadd_rn(acc, __fmul_rn(bf16_hi(qv.x), k[1]));
  acc = __fadd_rn(acc, __fmul_rn(bf16_lo(qv.y), k[2]));
  acc = __fadd_rn(acc, __fmul_rn(bf16_hi(qv.y), k[3]));
  acc = __fadd_rn(acc, __fmul_rn(bf16_lo(qv.z), k[4]));
  acc = __fadd_rn(acc, __fmul_rn(bf16_hi(qv.z), k[5]));
  acc = __fadd_rn(acc, __fmul_rn(bf16_lo(qv.w), k[6]));
  acc = __fadd_rn(acc, __fmul_rn(bf16_hi(qv.w), k[7]));
  return acc;
}
// acc + q * k over eight bf16 pairs in order (the products are exact, so a
// fused multiply-add per step rounds only the sum, as the exact order asks).
__device__ __forceinline__ float dot8_bf16(float acc, uint4 qv, uint4 kv) {
  acc = __builtin_fmaf(bf16_lo(qv.x), bf16_lo(kv.x), acc);
  acc = __builtin_fmaf(bf16_hi(qv.x), bf16_hi(kv.x), acc);
  acc = __builtin_fmaf(bf16_lo(qv.y), bf16_lo(kv.y), acc);
  acc = __builtin_fmaf(bf16_hi(qv.y), bf16_hi(kv.y), acc);
  acc = __builtin_fmaf(bf16_lo(qv.z), bf16_lo(kv.z), acc);
  acc = __builtin_fmaf(bf16_hi(qv.z), bf16_hi(kv.z), acc);
  acc = __builtin_fmaf(bf16_lo(qv.w), bf16_lo(kv.w), acc);
  acc = __builtin_fmaf(bf16_hi(qv.w), bf16_hi(kv.w), acc);
  return acc;
}

// Exact score of one token, evaluated by a whole wave in the library's exact
// order (DSA mode, bf16 or fp8 K, head_dim 128): lane h forms dot_h left to
// right, then the terms w_h * relu(dot_h) are added in head order.
__device__ float exact_dsa_score(const ScoreArgs& sa, int b, int g, int t, float* lds_terms) {
  const int lane = threadIdx.x & 63;
  const int G = sa.q_heads / sa.num_kv_heads;
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(sa.q) + ((int64_t)b * sa.q_heads + g * G) * 128;
  const float* wb = sa.head_weights + (int64_t)b * sa.q_heads + g * G;
  const int page = sa.block_table[(int64_t)b * sa.max_pages + t / sa.page_size];
  const int slot = t % sa.page_size;
  const int64_t koff = (int64_t)page * sa.page_stride + (int64_t)g * sa.head_stride + (int64_t)slot * sa.token_stride;
  const bool fp8 = sa.dtype == 2;
  float total = 0.0f;
  for (int h0 = 0; h0 < G; h0 += kWave) {
    const int h = h0 + lane;
    float term = 0.0f;
    if (h < G) {
      const uint16_t* qh = qb + (int64_t)h * 128;
      const float ksc = fp8 ? sa.k_scale[fp8_scale_index(page, g, slot, sa.num_kv_heads, sa.page_size)] : 1.0f;
      // two halves of the row (dims 0..63, 64..127), each with its loads in
      // flight at once, then the ordered dot product
      float acc = 0.0f;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        uint4 kr[8], qr[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) qr[i] = *reinterpret_cast<const uint4*>(qh + 64 * half + 8 * i);
        if (fp8) {
          const uint8_t* krow = reinterpret_cast<const uint8_t*>(sa.k) + koff + 64 * half;
#pragma unroll
          for (int i = 0; i < 4; ++i) kr[i] = *reinterpret_cast<const uint4*>(krow + 16 * i);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float kd[16];
            fp8x4_dequant(kr[i].x, ksc, kd);
            fp8x4_dequant(kr[i].y, ksc, kd + 4);
            fp8x4_dequant(kr[i].z, ksc, kd + 8);
            fp8x4_dequant(kr[i].w, ksc, kd + 12);
            acc = dot8_f32k(acc, qr[2 * i], kd);
            acc = dot8_f32k(acc, qr[2 * i + 1], kd + 8);
          }
        } else {
          const uint16_t* krow = reinterpret_cast<const uint16_t*>(sa.k) + koff + 64 * half;
#pragma unroll
          for (int i = 0; i < 8; ++i) kr[i] = *reinterpret_cast<const uint4*>(krow + 8 * i);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc = dot8_bf16(acc, qr[i], kr[i]);
        }
      }
      const float r = acc > 0.0f ? acc : 0.0f;
      term = __fmul_rn(wb[h], r);
    }
    lds_terms[lane] = term;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int n = min(kWave, G - h0);
    // 16 terms at a time into registers, then the ordered sum
    for (int j0 = 0; j0 < n; j0 += 16) {
      float tv[16];
#pragma unroll
      for (int j = 0; j < 16; j += 4) {
        const float4 q4 = *reinterpret_cast<const float4*>(lds_terms + j0 + j);
        tv[j] = q4.x; tv[j + 1] = q4.y; tv[j + 2] = q4.z; tv[j + 3] = q4.w;
      }
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (j0 + j < n) total = __fadd_rn(total, tv[j]);
    }
    __builtin_amdgcn_wave_barrier();
  }
  return total;
}

// The whole selection of one row by one 512-thread block.  Used as the
// fallback of the multi-block path when a row's band does not fit the band
// list (e.g. long runs of equal scores).
template <int NI, bool RESIDENT, bool FAST, typename SH>
__device__ __forceinline__ void select_row_block(const SelectArgs& a, int row, SH& sh,
                                 float (*s_terms)[kWave]) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int b = row / a.groups;
  const int L = clamp_len(a.kv_lens[b], a.row_stride);
  const int k = a.k;
  if (L <= k) {  // every token is kept
    for (int i = tid; i < k; i += kSelThreads) put_index(a, row, i, i < L ? i : -1);
    if (a.counts && tid == 0) a.counts[row] = L;
    return;
  }
  const float* s = a.scores + (int64_t)row * a.row_stride;
  uint32_t* keys = reinterpret_cast<uint32_t*>(a.keys) + (int64_t)row * a.row_stride;
  constexpr int PER = kTile * NI;
  // loops over the tiles: unrolled in full when the tiles are held in
  // registers, by two when they are re-read (the rare overflow fallback)
  constexpr int kU = RESIDENT ? NI : 2;
  const int nsc = RESIDENT ? 1 : (L + PER - 1) / PER;
  const bool vec = ((reinterpret_cast<uintptr_t>(s) & 15) == 0);
  const float kNan = __builtin_nanf("");

  auto load4 = [&](int t0) -> float4 {
    if (vec && t0 + 3 < L) return *reinterpret_cast<const float4*>(s + t0);
    float4 r;
    r.x = t0 < L ? s[t0] : kNan;
    r.y = t0 + 1 < L ? s[t0 + 1] : kNan;
    r.z = t0 + 2 < L ? s[t0 + 2] : kNan;
    r.w = t0 + 3 < L ? s[t0 + 3] : kNan;
    return r;
  };
  auto tok = [&](int sc, int i) {
    int t4 = 4 * tid;
    asm volatile("" : "+v"(t4));  // recomputed at each use: no per-tile offsets held live
    return sc * PER + i * kTile + t4;
  };

  float4 v[NI];
  auto get = [&](int sc, int i) -> float4 {
    if constexpr (RESIDENT) return v[i];
    return load4(tok(sc, i));
  };
  if constexpr (RESIDENT) {
#pragma unroll
    for (int i = 0; i < NI; ++i) v[i] = load4(tok(0, i));
  }

  // ---- 1. min / max / count of finite scores
  float lo = __builtin_inff(), hi = -__builtin_inff();
  int nfin = 0;
  for (int sc = 0; sc < nsc; ++sc) {
#pragma unroll kU
    for (int i = 0; i < NI; ++i) {
      const float4 x = get(sc, i);
      const float e4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (__builtin_isfinite(e4[e])) {
          lo = fminf(lo, e4[e]);
          hi = fmaxf(hi, e4[e]);
          ++nfin;
        }
    }
  }
  block_min_max_sum(lo, hi, nfin, sh);

  // ---- 2. histogram and the bin of the k-th largest
  // value-linear bins; float arithmetic is monotone in x, which is all the
  // classification needs (NaN only if the range overflows: top bin)
  const float fscale = hi > lo ? (float)((double)kBins / ((double)hi - (double)lo)) : 0.0f;
  auto bin_of = [&](float x) -> int {
    const float f = (x - lo) * fscale;
    return (f >= (float)(kBins - 1) || f != f) ? kBins - 1 : (int)f;
  };
  int bstar = -1;
  if (nfin >= k) {
    for (int i = tid; i < kBins; i += kSelThreads) sh.hist[i] = 0;
    __syncthreads();
    for (int sc = 0; sc < nsc; ++sc) {
#pragma unroll kU
      for (int i = 0; i < NI; ++i) {
        const float4 x = get(sc, i);
        const float e4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool fin = __builtin_isfinite(e4[e]);
          hist_add(sh.hist, fin ? bin_of(e4[e]) : 0, fin);
        }
      }
    }
    __syncthreads();
    find_bin(sh, kBins, k);
    bstar = sh.win[0];
    __syncthreads();
  }

  // ---- 3. classes
  // bstar < 0: fewer than k finite scores -> every finite one is kept and the
  // -inf (absent) tokens compete, lowest position first.
  float band_lo = 0.0f, band_hi = 0.0f;  // outward-rounded band edges
  if constexpr (FAST) {
    if (bstar >= 0) {
      float mlo = __builtin_inff(), mhi = -__builtin_inff();
      for (int sc = 0; sc < nsc; ++sc) {
#pragma unroll kU
        for (int i = 0; i < NI; ++i) {
          const float4 x = get(sc, i);
          const float e4[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (__builtin_isfinite(e4[e]) && bin_of(e4[e]) == bstar) {
              mlo = fminf(mlo, e4[e]);
              mhi = fmaxf(mhi, e4[e]);
            }
        }
      }
      mlo = block_min_f(mlo, sh);
      mhi = block_max_f(mhi, sh);
      const double d2 = 2.0 * (double)a.row_bound[row];
      const double blo = (double)mlo - d2, bhi = (double)mhi + d2;
      band_lo = (float)blo;
      band_hi = (float)bhi;
      if ((double)band_lo > blo) band_lo = next_down(band_lo);
      if ((double)band_hi < bhi) band_hi = next_up(band_hi);
    }
  }
  int n_in = 0, n_band = 0;
  for (int sc = 0; sc < nsc; ++sc) {
#pragma unroll kU
    for (int i = 0; i < NI; ++i) {
      const float4 x = get(sc, i);
      const float e4[4] = {x.x, x.y, x.z, x.w};
      uint32_t byte = 0;
      const int t0 = tok(sc, i);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float val = e4[e];
        uint32_t c;
        if (t0 + e >= L) {
          c = kPad;
        } else if (bstar < 0) {
          c = __builtin_isfinite(val) ? kIn : kBand;
        } else if (!__builtin_isfinite(val)) {
          c = kOut;
        } else if constexpr (FAST) {
          c = val > band_hi ? kIn : (val < band_lo ? kOut : kBand);
        } else {
          const int bn = bin_of(val);
          c = bn > bstar ? kIn : (bn < bstar ? kOut : kBand);
        }
        n_in += c == kIn;
        n_band += c == kBand;
        // band keys: exact scores are re-derived from the scores themselves
        // below (no memory round trip); fast rows store the -inf fillers'
        if (c == kBand && FAST && bstar < 0) keys[t0 + e] = score_key(val);
        byte |= c << (2 * e);
      }
      sh.cls[(sc * NI + i) * kSelThreads + tid] = (uint8_t)byte;
    }
  }
  if constexpr (RESIDENT && NI * kTile < 65536) {
    // both counts in one sum (each at most the row length, below 2^16)
    const int packed = block_sum_i(n_in | (n_band << 16), sh);  // (has __syncthreads: classes visible)
    n_in = packed & 0xFFFF;
    n_band = packed >> 16;
  } else {
    n_in = block_sum_i(n_in, sh);  // (has __syncthreads: classes visible)
    n_band = block_sum_i(n_band, sh);
  }

  // ---- FAST: exact scores of the band tokens (each wave re-scores the band
  // tokens among its own 64 threads' positions)
  if constexpr (FAST) {
    if (bstar >= 0) {
      const int g = row % a.groups;
      for (int sc = 0; sc < nsc; ++sc)
        for (int i = 0; i < NI; ++i) {
          const uint32_t byte = sh.cls[(sc * NI + i) * kSelThreads + tid];
          for (int e = 0; e < 4; ++e) {
            uint64_t m = __ballot(((byte >> (2 * e)) & 3u) == kBand);
            while (m) {
              const int src = __builtin_ctzll(m);
              m &= m - 1;
              const int t = sc * PER + i * kTile + 4 * (wid * 64 + src) + e;
              const float ex = exact_dsa_score(a.score, b, g, t, s_terms[wid]);
              if (lane == 0) keys[t] = score_key(ex);
            }
          }
        }
      __threadfence_block();
      __syncthreads();
    }
  }

  // Keys of this thread's band tokens in tile (sc, i): exact scores give
  // them from the scores (registers when the row is resident); re-scored
  // fast rows read them back from the key array.
  auto band_keys = [&](int sc, int i, uint32_t byte, uint32_t (&k4)[4]) {
    if constexpr (FAST) {
      const int t0 = tok(sc, i);
#pragma unroll
      for (int e = 0; e < 4; ++e) k4[e] = ((byte >> (2 * e)) & 3u) == kBand ? keys[t0 + e] : 0u;
    } else {
      const float4 x = get(sc, i);
      k4[0] = score_key(x.x);
      k4[1] = score_key(x.y);
      k4[2] = score_key(x.z);
      k4[3] = score_key(x.w);
    }
  };

  int remaining = k - n_in;  // band tokens to keep (>= 1)

  // ---- 4'. a short band of a resident row: each entry is ranked against the
  // others in (key desc, position asc) order and kept when fewer than
  // `remaining` entries come before it; then the ordered emission
  if constexpr (RESIDENT) {
    if (n_band <= kRankMax) {
      if (tid == 0) sh.rcount = 0;
      __syncthreads();
      int bidx[NI][4];
#pragma unroll kU
      for (int i = 0; i < NI; ++i) {
        const uint32_t byte = sh.cls[i * kSelThreads + tid];
        const int t0 = tok(0, i);
        uint32_t k4[4];
        band_keys(0, i, byte, k4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bidx[i][e] = -1;
          if (((byte >> (2 * e)) & 3u) == kBand) {
            const int j = atomicAdd(&sh.rcount, 1);
            sh.rkey[j] = ((uint64_t)k4[e] << 32) | (uint32_t)~(uint32_t)(t0 + e);
            bidx[i][e] = j;
          }
        }
      }
      __syncthreads();
      for (int j = tid; j < n_band; j += kSelThreads) {
        const uint64_t x = sh.rkey[j];
        int rank = 0;
        for (int m = 0; m < n_band; ++m) rank += sh.rkey[m] > x;
        sh.rkeep[j] = rank < remaining;
      }
      __syncthreads();
      uint32_t keepm[NI];
      int kept[NI];
#pragma unroll kU
      for (int i = 0; i < NI; ++i) {
        const uint32_t byte = sh.cls[i * kSelThreads + tid];
        keepm[i] = 0;
        kept[i] = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t c = (byte >> (2 * e)) & 3u;
          const bool kp = c == kIn || (c == kBand && sh.rkeep[bidx[i][e]]);
          keepm[i] |= (uint32_t)kp << e;
          kept[i] += kp;
        }
      }
      auto emit_tile = [&](int i, int pos) {
        const int t0 = tok(0, i);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((keepm[i] >> e) & 1u) {
            if (pos < k) put_index(a, row, pos, t0 + e);
            ++pos;
          }
      };
      if constexpr (NI <= 2) {  // both tiles' counts (below 2^16 each) in one scan
        int total;
        const int packed = block_excl_scan<kSelThreads>(kept[0] | (NI > 1 ? kept[NI - 1] << 16 : 0), sh.tmp, &total);
        emit_tile(0, packed & 0xFFFF);
        if constexpr (NI > 1) emit_tile(1, (total & 0xFFFF) + (packed >> 16));
      } else {
        int base = 0;
#pragma unroll kU
        for (int i = 0; i < NI; ++i) {
          int total;
          emit_tile(i, base + block_excl_scan<kSelThreads>(kept[i], sh.tmp, &total));
          base += total;
        }
      }
      if (a.counts && tid == 0) a.counts[row] = k;
      return;
    }
  }

  // ---- 4. radix select over the band keys
  uint32_t prefix = 0, pmask = 0;
  {
    const int shifts[3] = {21, 10, 0};
    const int nbits[3] = {11, 11, 10};
#pragma unroll 1
    for (int p = 0; p < 3; ++p) {
      const int nb = 1 << nbits[p];
      for (int i = tid; i < kBins; i += kSelThreads) sh.hist[i] = 0;
      __syncthreads();
      for (int sc = 0; sc < nsc; ++sc)
        for (int i = 0; i < NI; ++i) {
          const uint32_t byte = sh.cls[(sc * NI + i) * kSelThreads + tid];
          uint32_t k4[4];
          band_keys(sc, i, byte, k4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bool act = ((byte >> (2 * e)) & 3u) == kBand;
            const uint32_t key = act ? k4[e] : 0u;
            act = act && (key & pmask) == prefix;
            hist_add(sh.hist, (int)((key >> shifts[p]) & (uint32_t)(nb - 1)), act);
          }
        }
      __syncthreads();
      find_bin(sh, nb, remaining);
      remaining -= sh.win[1];
      prefix |= (uint32_t)sh.win[0] << shifts[p];
      pmask |= (uint32_t)(nb - 1) << shifts[p];
      __syncthreads();
    }
  }
  const uint32_t kth = prefix;
  int need = remaining;  // band tokens equal to kth that are kept, lowest positions first

  // ---- 5. ordered emission, tile by tile
  int base = 0;
  for (int sc = 0; sc < nsc; ++sc)
    for (int i = 0; i < NI; ++i) {
      const uint32_t byte = sh.cls[(sc * NI + i) * kSelThreads + tid];
      const int t0 = tok(sc, i);
      int gt = 0, eq = 0;
      uint32_t flags = 0;  // bit e: strictly kept, bit 4+e: tie
      uint32_t k4[4];
      band_keys(sc, i, byte, k4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t c = (byte >> (2 * e)) & 3u;
        if (c == kIn) {
          flags |= 1u << e;
          ++gt;
        } else if (c == kBand) {
          const uint32_t key = k4[e];
          if (key > kth) {
            flags |= 1u << e;
            ++gt;
          } else if (key == kth) {
            flags |= 16u << e;
            ++eq;
          }
        }
      }
      int total;
      const int packed = block_excl_scan<kSelThreads>((eq << 16) | gt, sh.tmp, &total);
      const int gt_before = packed & 0xFFFF, eq_before = packed >> 16;
      const int tot_gt = total & 0xFFFF, tot_eq = total >> 16;
      const int take_before = min(max(need, 0), eq_before);
      int take = max(0, min(eq, need - eq_before));
      int pos = base + gt_before + take_before;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool keep = (flags & (1u << e)) || ((flags & (16u << e)) && take > 0);
        if (!(flags & (1u << e)) && keep) --take;
        if (keep && pos < k) put_index(a, row, pos, t0 + e);
        pos += keep;
      }
      const int took = min(max(need, 0), tot_eq);
      base += tot_gt + took;
      need -= took;
    }
  if (a.counts && tid == 0) a.counts[row] = k;
}

// ------------------------------------------------------------------ multi-block path
//
// The rows are long and few (16 rows of 65536 tokens for the DSA decode), so
// every pass over the scores is spread over all CUs, 4096 tokens per block:
//   init     per-row statistics zeroed (before the scorer, which adds the
//            min / max keys of the finite scores with one atomic per wave);
//   hist     value-linear 2048-bin histogram of every row;
//   classify the bin of the k-th largest score, every token classed IN /
//            OUT / BAND (as in the one-block path), IN counted per chunk,
//            BAND tokens (re-scored exactly for fast scores) appended to the
//            row's band list;
//   emit     the band list sorted by (key desc, position asc); its first
//            k - |IN| entries are kept; every block writes its chunk's kept
//            positions at the offset given by the per-chunk counts.
// A row whose band overflows the list is finished by one block with
// select_row_block (exact, slower).

constexpr int kChunkThreads = 512;
constexpr int kStageRows = kChunkThreads / 16;  // band K rows staged per pass
constexpr int kPerThread = kSelChunk / kChunkThreads;  // 8 contiguous tokens

struct RowView {
  int L;
  bool any_finite;
  float lo, hi, fscale;
};

// The row's histogram range [lo, hi]: the min / max finite score, with lo
// raised to the floor a hint certified (no token below it can be selected).
__device__ __forceinline__ RowView view_of_keys(const SelectArgs& a, int row, uint32_t kmin, uint32_t kmax,
                                                float floor) {
  const int b = row / a.groups;
  RowView v;
  v.L = clamp_len(a.kv_lens[b], a.row_stride);
  v.any_finite = kmin <= kmax;
  v.lo = v.any_finite ? key_to_score(kmin) : 0.0f;
  v.hi = v.any_finite ? key_to_score(kmax) : 0.0f;
  if (v.any_finite && floor > v.lo) v.lo = fminf(floor, v.hi);
  // identical to the one-block path when there is no floor: same bins, same classes
  v.fscale = v.hi > v.lo ? (float)((double)kBins / ((double)v.hi - (double)v.lo)) : 0.0f;
  return v;
}
__device__ __forceinline__ RowView make_view(const SelectArgs& a, int row, float floor) {
  const int32_t* st = a.stats + (int64_t)row * kStatStride;
  return view_of_keys(a, row, (uint32_t)st[0], (uint32_t)st[1], floor);
}
__device__ __forceinline__ RowView row_view(const SelectArgs& a, int row) {
  return make_view(a, row, __int_as_float(a.stats[(int64_t)row * kStatStride + 7]));
}

__device__ __forceinline__ int bin_of_v(const RowView& v, float x) {
  const float f = (x - v.lo) * v.fscale;
  return (f >= (float)(kBins - 1) || f != f) ? kBins - 1 : (int)f;
}

// The passes below issue every load that does not depend on the row's
// statistics first (scores, histogram, ...), so a block waits on memory once
// rather than once per dependent step: load8_raw reads this thread's 8
// tokens within the row's stride before kv_len is known, mask8 then marks
// those past kv_len NaN.
__device__ __forceinline__ void load8_raw(const float* s, int t0, int n, float (&x)[kPerThread]) {
  if (t0 + kPerThread <= n && ((reinterpret_cast<uintptr_t>(s + t0) & 15) == 0)) {
    const float4 p = *reinterpret_cast<const float4*>(s + t0);
    const float4 q = *reinterpret_cast<const float4*>(s + t0 + 4);
    x[0] = p.x; x[1] = p.y; x[2] = p.z; x[3] = p.w;
    x[4] = q.x; x[5] = q.y; x[6] = q.z; x[7] = q.w;
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) x[e] = t0 + e < n ? s[t0 + e] : __builtin_nanf("");
  }
}
__device__ __forceinline__ void mask8(int t0, int L, float (&x)[kPerThread]) {
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    if (t0 + e >= L) x[e] = __builtin_nanf("");
}

// this thread's 8 contiguous tokens of chunk c (NaN past kv_len)
__device__ __forceinline__ void load8(const float* s, int t0, int L, float (&x)[kPerThread]) {
  if (t0 + kPerThread <= L && ((reinterpret_cast<uintptr_t>(s + t0) & 15) == 0)) {
    const float4 p = *reinterpret_cast<const float4*>(s + t0);
    const float4 q = *reinterpret_cast<const float4*>(s + t0 + 4);
    x[0] = p.x; x[1] = p.y; x[2] = p.z; x[3] = p.w;
    x[4] = q.x; x[5] = q.y; x[6] = q.z; x[7] = q.w;
  } else {
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) x[e] = t0 + e < L ? s[t0 + e] : __builtin_nanf("");
  }
}

struct ChunkShared {
  int hist[kBins];
  int tmp[kSelWaves];
  int win[2];
  int redi[kSelWaves];
  float redf[2][kSelWaves];
};

__device__ __forceinline__ int chunk_sum_i(int v, int* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  int r = 0;
  for (int w = 0; w < kSelWaves; ++w) r += red[w];
  __syncthreads();
  return r;
}

// Decision data of a row, identical in every block: the bin of the k-th
// largest finite score (or -1 when fewer than k scores are finite) and, for
// fast scores, the band edges.
struct RowCut {
  int bstar;
  int nfin;
  float band_lo, band_hi;
};

constexpr int kBinsPerThread = kBins / kChunkThreads;
static_assert(kBins % kChunkThreads == 0, "histogram bins per thread");

// hb: this thread's bins tid + j * kChunkThreads of the row's histogram
__device__ RowCut row_cut(const SelectArgs& a, int row, const RowView& v, ChunkShared& sh, bool fast,
                          const int (&hb)[kBinsPerThread]) {
  int part = 0;
#pragma unroll
  for (int j = 0; j < kBinsPerThread; ++j) {
    const int h = v.any_finite ? hb[j] : 0;
    sh.hist[threadIdx.x + j * kChunkThreads] = h;
    part += h;
  }
  RowCut c;
  c.nfin = chunk_sum_i(part, sh.redi);  // (barriers: hist visible)
  c.bstar = -1;
  c.band_lo = c.band_hi = 0.0f;
  if (c.nfin >= a.k) {
    find_bin_n<kChunkThreads>(sh.hist, sh.tmp, sh.win, kBins, a.k);
    c.bstar = sh.win[0];
    __syncthreads();
    if (fast) {
      // values in bin B* lie in [e_lo, e_hi]: the bin edges widened by the
      // rounding of the bin arithmetic (three binary32 roundings)
      const double dlo = v.lo, dhi = v.hi;
      const double w = v.fscale > 0.0f ? 1.0 / (double)v.fscale : 0.0;
      const double eps = 8.0 * 5.9604644775390625e-8 * (dhi - dlo) + 1e-30;
      double e_lo = dlo + c.bstar * w - eps, e_hi = dlo + (c.bstar + 1) * w + eps;
      if (c.bstar == 0 || e_lo < dlo) e_lo = dlo;
      if (c.bstar == kBins - 1 || e_hi > dhi) e_hi = dhi;
      const double d2 = 2.0 * (double)a.row_bound[row];
      const double blo = e_lo - d2, bhi = e_hi + d2;
      c.band_lo = (float)blo;
      c.band_hi = (float)bhi;
      if ((double)c.band_lo > blo) c.band_lo = next_down(c.band_lo);
      if ((double)c.band_hi < bhi) c.band_hi = next_up(c.band_hi);
    }
  }
  return c;
}

// The cut as the classify pass published it (stat slots 3..6).
__device__ __forceinline__ RowCut stored_cut(const SelectArgs& a, int row) {
  const int32_t* st = a.stats + (int64_t)row * kStatStride;
  RowCut c;
  c.bstar = st[3];
  c.nfin = st[4];
  c.band_lo = __int_as_float(st[5]);
  c.band_hi = __int_as_float(st[6]);
  return c;
}

// IN / OUT / BAND of one token (NaN = past kv_len -> kPad)
__device__ __forceinline__ uint32_t classify(const RowView& v, const RowCut& c, float x, bool fast) {
  if (x != x) return kPad;
  if (c.bstar < 0) return __builtin_isfinite(x) ? kIn : kBand;  // -inf tokens fill the quota
  if (!__builtin_isfinite(x) || x < v.lo) return kOut;  // below the hint's floor: never selected
  if (fast) return x > c.band_hi ? kIn : (x < c.band_lo ? kOut : kBand);
  const int bn = bin_of_v(v, x);
  return bn > c.bstar ? kIn : (bn < c.bstar ? kOut : kBand);
}

__global__ __launch_bounds__(256) void select_init_kernel(SelectArgs a) {
  const int row = blockIdx.x;
  int32_t* st = a.stats + (int64_t)row * kStatStride;
  for (int i = threadIdx.x; i < kStatStride; i += 256) st[i] = 0;
  if (threadIdx.x == 0) st[0] = (int32_t)0xFFFFFFFFu;  // kmin starts at the largest key
  if (threadIdx.x == 0) st[7] = (int32_t)0xFF800000u;  // no floor (-inf)
  // the fast scorer max-accumulates its error bound into row_bound
  if (threadIdx.x == 0 && a.row_bound) a.row_bound[row] = 0.0f;
}

// min / max keys of the finite scores (standalone selection; the scorers do
// this themselves in the fused path)
__global__ __launch_bounds__(kChunkThreads) void select_stats_kernel(SelectArgs a) {
  const int row = blockIdx.y, c = blockIdx.x;
  const int L = clamp_len(a.kv_lens[row / a.groups], a.row_stride);
  const int t0 = c * kSelChunk + kPerThread * threadIdx.x;
  if (L <= a.k || c * kSelChunk >= L) return;
  float x[kPerThread];
  load8(a.scores + (int64_t)row * a.row_stride, t0, L, x);
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    if (__builtin_isfinite(x[e])) {
      const uint32_t key = score_key(x[e]);
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  if ((threadIdx.x & 63) == 0 && kmin <= kmax) {
    int32_t* st = a.stats + (int64_t)row * kStatStride;
    atomicMin(reinterpret_cast<unsigned int*>(st), kmin);
    atomicMax(reinterpret_cast<unsigned int*>(st + 1), kmax);
  }
}

// Exclusive max over the threads of a chunk block (-1 for thread 0); `red`
// needs kSelWaves ints.  Contains __syncthreads.
__device__ __forceinline__ int chunk_excl_max(int v, int* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int w = __shfl_up(inc, o);
    if (lane >= o) inc = max(inc, w);
  }
  if (lane == 63) red[wid] = inc;
  __syncthreads();
  int before = -1;
  for (int w = 0; w < wid; ++w) before = max(before, red[w]);
  const int excl = max(before, __shfl_up(inc, 1));
  __syncthreads();
  return lane == 0 ? before : excl;
}

// Floor certified by a hint: when the hint names at least k distinct
// positions below L, the k-th largest score is at least the smallest of
// their scores (exact scores), or that minus the row bound d (fast scores,
// whose exact values differ by at most d); a token whose score is below
// min - 2d (fast) or min (exact) is then below the k-th largest exact score
// and is never selected.  -inf when the hint certifies nothing.  Distinct
// positions are counted without a set: an entry counts when it is valid and
// larger than every valid entry before it, so an ascending hint (what the
// write-back produces) counts in full and any other hint counts a subset of
// distinct positions.  Every block of the row computes the same value.
__device__ float hint_floor(const SelectArgs& a, int row, int L, float bound, int* red) {
  const int tid = threadIdx.x;
  const int n = a.hint_len;
  const int per = (n + kChunkThreads - 1) / kChunkThreads;  // a contiguous run per thread
  const int i0 = min(n, tid * per), i1 = min(n, i0 + per);
  const int32_t* h = a.hint + (int64_t)row * a.hint_stride;
  const float* s = a.scores + (int64_t)row * a.row_stride;
  int lmax = -1;
  for (int i = i0; i < i1; ++i) {
    const int p = h[i];
    if (p >= 0 && p < L) lmax = max(lmax, p);
  }
  int run = chunk_excl_max(lmax, red);
  int distinct = 0;
  float vmin = __builtin_inff();
  for (int i = i0; i < i1; ++i) {
    const int p = h[i];
    if (p >= 0 && p < L && p > run) {
      run = p;
      ++distinct;
      vmin = fminf(vmin, s[p]);
    }
  }
  distinct = chunk_sum_i(distinct, red);
  vmin = fminf(vmin, __shfl_xor(vmin, 32)); vmin = fminf(vmin, __shfl_xor(vmin, 16));
  vmin = fminf(vmin, __shfl_xor(vmin, 8)); vmin = fminf(vmin, __shfl_xor(vmin, 4));
  vmin = fminf(vmin, __shfl_xor(vmin, 2)); vmin = fminf(vmin, __shfl_xor(vmin, 1));
  if ((tid & 63) == 0) red[tid >> 6] = __float_as_int(vmin);
  __syncthreads();
  float m = __int_as_float(red[0]);
  for (int w = 1; w < kSelWaves; ++w) m = fminf(m, __int_as_float(red[w]));
  __syncthreads();
  if (distinct < a.k || !__builtin_isfinite(m)) return -__builtin_inff();
  if (!a.row_bound) return m;
  const double f = (double)m - 2.0 * (double)bound;
  float fl = (float)f;
  if ((double)fl > f) fl = next_down(fl);
  return fl;
}

// The fused path's fast scorer leaves per-block slots instead of the row's
// min / max keys and bound: every block reduces them (a few dozen at most)
// and block 0 publishes the result for the later passes.
struct RowKeys {
  uint32_t kmin, kmax;
  float bound;
};
__device__ RowKeys reduce_span_slots(const SelectArgs& a, int row, uint32_t (*red)[kSelWaves]) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u, bd = 0u;  // bound bits: non-negative floats order as integers
  const int32_t* sl = a.span_slots + (int64_t)row * a.nspans * 4;
  for (int i = tid; i < a.nspans; i += kChunkThreads) {
    const int4 e = *reinterpret_cast<const int4*>(sl + 4 * i);
    kmin = min(kmin, (uint32_t)e.x);
    kmax = max(kmax, (uint32_t)e.y);
    bd = max(bd, (uint32_t)e.z);
  }
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  bd = wave_max_u32(bd);
  if (lane == 0) {
    red[0][wid] = kmin;
    red[1][wid] = kmax;
    red[2][wid] = bd;
  }
  __syncthreads();
  RowKeys r{red[0][0], red[1][0], 0.0f};
  bd = red[2][0];
  for (int w = 1; w < kSelWaves; ++w) {
    r.kmin = min(r.kmin, red[0][w]);
    r.kmax = max(r.kmax, red[1][w]);
    bd = max(bd, red[2][w]);
  }
  r.bound = __uint_as_float(bd);
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kChunkThreads) void select_hist_kernel(SelectArgs a) {
  __shared__ int hist[kBins];
  __shared__ int red[kSelWaves];
  __shared__ uint32_t red3[3][kSelWaves];
  const int row = blockIdx.y, c = blockIdx.x;
  int32_t* st = a.stats + (int64_t)row * kStatStride;
  float x[kPerThread];
  const int t0 = c * kSelChunk + kPerThread * threadIdx.x;
  load8_raw(a.scores + (int64_t)row * a.row_stride, t0, a.row_stride, x);
  RowKeys r;
  if (a.span_slots) {
    r = reduce_span_slots(a, row, red3);
    if (c == 0 && threadIdx.x == 0) {
      st[0] = (int32_t)r.kmin;
      st[1] = (int32_t)r.kmax;
      a.row_bound[row] = r.bound;
    }
  } else {
    r = RowKeys{(uint32_t)st[0], (uint32_t)st[1], a.row_bound ? a.row_bound[row] : 0.0f};
  }
  RowView v = view_of_keys(a, row, r.kmin, r.kmax, __int_as_float(st[7]));
  if (v.L <= a.k || c * kSelChunk >= v.L || !v.any_finite) return;
  if (a.hint) {
    const float floor = hint_floor(a, row, v.L, r.bound, red);
    v = view_of_keys(a, row, r.kmin, r.kmax, floor);
    if (c == 0 && threadIdx.x == 0) a.stats[(int64_t)row * kStatStride + 7] = __float_as_int(floor);
  }
  for (int i = threadIdx.x; i < kBins; i += kChunkThreads) hist[i] = 0;
  __syncthreads();
  mask8(t0, v.L, x);
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const bool fin = __builtin_isfinite(x[e]) && x[e] >= v.lo;
    hist_add(hist, fin ? bin_of_v(v, x[e]) : 0, fin);
  }
  __syncthreads();
  int32_t* gh = a.stats + (int64_t)row * kStatStride + 8;
  for (int i = threadIdx.x; i < kBins; i += kChunkThreads)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// Shared memory of the classify pass (the re-score buffers only with fast scores).
template <bool FAST>
struct ClassifySmem {
  ChunkShared sh;
  uint16_t s_bpos[kSelChunk];  // band tokens of the chunk (offsets in it)
  int s_nband, s_base;
  // K rows of band tokens being re-scored: bf16 rows as they are (256 bytes),
  // fp8 rows dequantized to binary32 (512 bytes)
  __attribute__((aligned(16))) float s_krow[kStageRows][128];
  int s_tpage[FAST ? kChunkThreads : 1];  // page of each thread's eight tokens (fast scores)
  // query rows of the band re-score, one per head, 17 units apart (the
  // per-lane reads of one unit then hit distinct banks)
  __attribute__((aligned(16))) uint4 s_q[FAST ? 64 * 17 : 1];
};

// This thread's page of its eight tokens (fast scores; one page: the fast
// path's page size is a multiple of 16), or -1.
__device__ __forceinline__ int thread_page(const SelectArgs& a, int b, int t0) {
  const ScoreArgs& sa = a.score;
  const int pi = t0 / sa.page_size;
  return (t0 < a.row_stride && pi < sa.max_pages) ? sa.block_table[(int64_t)b * sa.max_pages + pi] : -1;
}

// Classify pass of chunk c of a row of more than k tokens, on the row's view
// v, this thread's eight scores x (NaN past kv_len) and its bins hb of the
// row's histogram: the cut, the chunk's (kept-for-sure, -inf) counts, and
// its band entries (exact keys; re-scored with fast scores).  Returns the cut.
template <bool FAST>
__device__ RowCut classify_chunk(const SelectArgs& a, int row, int c, const RowView& v, const float (&x)[kPerThread],
                                 const int (&hb)[kBinsPerThread], int tpage, ClassifySmem<FAST>& S,
                                 float (*s_terms)[kWave]) {
  constexpr int kQStride = 17;
  ChunkShared& sh = S.sh;
  uint16_t* s_bpos = S.s_bpos;
  int& s_nband = S.s_nband;
  int& s_base = S.s_base;
  float (*s_krow)[128] = S.s_krow;
  int* s_tpage = S.s_tpage;
  uint4* s_q = S.s_q;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int g = row % a.groups, b = row / a.groups;
  const ScoreArgs& sa = a.score;
  const int G = FAST ? sa.q_heads / sa.num_kv_heads : 0;  // <= 64 on the fast path
  const int t0 = c * kSelChunk + kPerThread * tid;
  const RowCut cut = row_cut(a, row, v, sh, FAST, hb);

  if (tid == 0) s_nband = 0;
  __syncthreads();
  int n_in = 0, n_neg = 0;
  uint32_t* keys = reinterpret_cast<uint32_t*>(a.keys) + (int64_t)row * a.row_stride;
  int32_t* st = a.stats + (int64_t)row * kStatStride;
  uint64_t* band = a.band + (int64_t)row * kBandCap;
  const int cstart = c * kSelChunk;
  // band tokens go to the chunk's list; this thread remembers their list
  // slots (-1: not in the band)
  int bslot[kPerThread];
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const uint32_t cl = classify(v, cut, x[e], FAST);
    n_in += cl == kIn;
    n_neg += (x[e] == -__builtin_inff());
    bslot[e] = -1;
    if (cl == kBand) {
      bslot[e] = atomicAdd(&s_nband, 1);
      s_bpos[bslot[e]] = (uint16_t)(t0 + e - cstart);
    }
  }
  if constexpr (FAST) s_tpage[tid] = tpage;
  n_in = chunk_sum_i(n_in, sh.redi);
  n_neg = chunk_sum_i(n_neg, sh.redi);  // (barrier: the band list complete)
  if (tid == 0) {
    int32_t* cc = a.chunk_counts + ((int64_t)row * a.nchunks + c) * 2;
    st_coherent(reinterpret_cast<uint64_t*>(cc), (uint64_t)(uint32_t)n_in | ((uint64_t)(uint32_t)n_neg << 32));
  }
  const int nb = s_nband;  // (visible: the barriers above)
  if (nb == 0) return cut;
  // The chunk's entries of the row's band list: one reservation per block.
  // Re-scored bands publish the reservation with the staging barrier below,
  // so that its round trip overlaps the staging loads.
  int reserved = 0;
  if (tid == 0) reserved = atomicAdd(&st[2], nb);
  // band entry of token t with key `key`, list slot i of the chunk
  auto put_band = [&](int i, int t, uint32_t key) {
    const int slot = s_base + i;
    keys[t] = key;
    if (slot < kBandCap) st_coherent(band + slot, ((uint64_t)key << 32) | (uint32_t)~(uint32_t)t);
  };
  if (!FAST || cut.bstar < 0) {
    if (tid == 0) s_base = reserved;
    __syncthreads();
    // the scores are the keys: each thread writes its own band tokens
#pragma unroll
    for (int e = 0; e < kPerThread; ++e)
      if (bslot[e] >= 0) put_band(bslot[e], t0 + e, score_key(x[e]));
    return cut;
  }
  {
    // Exact re-score of the band: the group's query rows and the K rows of
    // up to kStageRows tokens at a time are staged in LDS (one round trip),
    // and a wave scores one token in the library's exact order (lane h:
    // dot_h left to right; then the head terms in head order),
    // bit-identical to the exact scorer.
    const bool hact = lane < G;
    const float wh = hact ? sa.head_weights[(int64_t)b * sa.q_heads + g * G + lane] : 0.0f;
    for (int u = tid; u < G * 16; u += kChunkThreads) {
      const int h = u >> 4, part = u & 15;
      s_q[h * kQStride + part] = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(sa.q) +
                                                                ((int64_t)b * sa.q_heads + g * G + h) * 128 + 8 * part);
    }
    const uint4* qrow = s_q + lane * kQStride;
    const bool fp8 = sa.dtype == 2;
    for (int p0 = 0; p0 < nb; p0 += kStageRows) {
      const int np = min(kStageRows, nb - p0);
      {
        const int i = tid >> 4, part = tid & 15;  // 16 threads per row
        if (i < np) {
          const int off = s_bpos[p0 + i];
          const int t = cstart + off;
          const int page = s_tpage[off / kPerThread];
          const int slot = t % sa.page_size;
          const int64_t koff = (int64_t)page * sa.page_stride + (int64_t)g * sa.head_stride +
                               (int64_t)slot * sa.token_stride;
          if (fp8) {  // 8 codes per thread, dequantized once here
            const uint2 c = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(sa.k) + koff + 8 * part);
            const float ksc = sa.k_scale[fp8_scale_index(page, g, slot, sa.num_kv_heads, sa.page_size)];
            float kd[8];
            fp8x4_dequant(c.x, ksc, kd);
            fp8x4_dequant(c.y, ksc, kd + 4);
            *reinterpret_cast<float4*>(&s_krow[i][8 * part]) = make_float4(kd[0], kd[1], kd[2], kd[3]);
            *reinterpret_cast<float4*>(&s_krow[i][8 * part + 4]) = make_float4(kd[4], kd[5], kd[6], kd[7]);
          } else {
            reinterpret_cast<uint4*>(s_krow[i])[part] =
                *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(sa.k) + koff + 8 * part);
          }
        }
      }
      if (p0 == 0 && tid == 0) s_base = reserved;
      __syncthreads();
      for (int i = wid; i < np; i += kSelWaves) {
        float term = 0.0f;
        if (hact) {
          float acc = 0.0f;
          if (fp8) {
#pragma unroll
            for (int c8 = 0; c8 < 16; ++c8) {
              float kd[8];
              const float4 lo = *reinterpret_cast<const float4*>(&s_krow[i][8 * c8]);
              const float4 hi = *reinterpret_cast<const float4*>(&s_krow[i][8 * c8 + 4]);
              kd[0] = lo.x; kd[1] = lo.y; kd[2] = lo.z; kd[3] = lo.w;
              kd[4] = hi.x; kd[5] = hi.y; kd[6] = hi.z; kd[7] = hi.w;
              acc = dot8_f32k(acc, qrow[c8], kd);
              // K reads in groups of four units: fewer registers live at once
              if ((c8 & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
          } else {
#pragma unroll
            for (int c8 = 0; c8 < 16; ++c8) {
              acc = dot8_bf16(acc, qrow[c8], reinterpret_cast<const uint4*>(s_krow[i])[c8]);
              if ((c8 & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
          }
          term = __fmul_rn(wh, acc > 0.0f ? acc : 0.0f);
        }
        s_terms[wid][lane] = term;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float total = 0.0f;
        for (int j0 = 0; j0 < G; j0 += 16) {
          float tv[16];
#pragma unroll
          for (int j = 0; j < 16; j += 4) {
            const float4 q4 = *reinterpret_cast<const float4*>(&s_terms[wid][j0 + j]);
            tv[j] = q4.x; tv[j + 1] = q4.y; tv[j + 2] = q4.z; tv[j + 3] = q4.w;
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) total = __fadd_rn(total, tv[j]);
        }
        if (lane == 0) put_band(p0 + i, cstart + s_bpos[p0 + i], score_key(total));
        __builtin_amdgcn_wave_barrier();
      }
      __syncthreads();  // the staging rows may be reused
    }
  }
  return cut;
}

template <bool FAST>
__global__ __launch_bounds__(kChunkThreads) void select_classify_kernel(SelectArgs a) {
  __shared__ ClassifySmem<FAST> S;
  __shared__ __attribute__((aligned(16))) float s_terms[kSelWaves][kWave];
  const int tid = threadIdx.x;
  const int row = blockIdx.x, c = blockIdx.y;  // chunk-major grid
  const int b = row / a.groups;
  // loads that do not depend on the cut, all in flight together
  float x[kPerThread];
  const int t0 = c * kSelChunk + kPerThread * tid;
  load8_raw(a.scores + (int64_t)row * a.row_stride, t0, a.row_stride, x);
  int hb[kBinsPerThread];
  {
    const int32_t* gh = a.stats + (int64_t)row * kStatStride + 8;
#pragma unroll
    for (int j = 0; j < kBinsPerThread; ++j) hb[j] = gh[tid + j * kChunkThreads];
  }
  const int tpage = FAST ? thread_page(a, b, t0) : -1;
  const RowView v = row_view(a, row);
  if (v.L <= a.k || c * kSelChunk >= v.L) return;
  mask8(t0, v.L, x);
  const RowCut cut = classify_chunk<FAST>(a, row, c, v, x, hb, tpage, S, s_terms);
  if (c == 0 && tid == 0) {  // for the emit kernel (identical in every block)
    int32_t* stc = a.stats + (int64_t)row * kStatStride;
    stc[3] = cut.bstar;
    stc[4] = cut.nfin;
    stc[5] = __float_as_int(cut.band_lo);
    stc[6] = __float_as_int(cut.band_hi);
  }
}

struct EmitShared {
  ChunkShared cs;
  uint64_t band[kBandCap];
  uint32_t chosen[kSelChunk / 32];  // chunk-local bitmap of kept band tokens
  int red2[4];
};

union EmitSmem {
  EmitShared e;
  SelShared one;  // fallback: one block finishes the row
};

// Emit pass of chunk c of a row of more than k tokens: the kept band entries
// (the first k - |IN| in (key desc, position asc) order), then this chunk's
// kept positions written at the offset the per-chunk counts give.  x holds
// this thread's eight scores as loaded (masked here), ccv wave 0's chunk
// counts (chunks tid and tid + 64).
template <bool FAST>
__device__ void emit_chunk(const SelectArgs& a, int row, int c, const RowView& v, const RowCut& cut, int nband,
                           float (&x)[kPerThread], const int2 (&ccv)[2], EmitShared& ue) {
  const int tid = threadIdx.x;
  const int cstart = c * kSelChunk;
  const int t0 = cstart + kPerThread * tid;
  const int k = a.k;
  const int32_t* cc = a.chunk_counts + (int64_t)row * a.nchunks * 2;
  // per-chunk counts (kept-for-sure, -inf) before this chunk and in total:
  // wave 0 reduces them, LDS hands them to the block
  const int nch = (v.L + kSelChunk - 1) / kSelChunk;
  if (tid < kWave) {
    int in_total = 0, in_before = 0, neg_before = 0;
    auto add = [&](int i, int2 e) {
      in_total += e.x;
      if (i < c) {
        in_before += e.x;
        neg_before += e.y;
      }
    };
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (tid + kWave * j < nch) add(tid + kWave * j, ccv[j]);
    for (int i = tid + 2 * kWave; i < nch; i += kWave) add(i, ld_coherent2(cc + 2 * i));
    in_total = wave_sum(in_total);
    in_before = wave_sum(in_before);
    neg_before = wave_sum(neg_before);
    if (tid == 0) {
      ue.red2[0] = in_total;
      ue.red2[1] = in_before;
      ue.red2[2] = neg_before;
    }
  }
  for (int i = tid; i < nband; i += kChunkThreads) ue.band[i] = ld_coherent(a.band + (int64_t)row * kBandCap + i);
  for (int i = tid; i < kSelChunk / 32; i += kChunkThreads) ue.chosen[i] = 0u;
  __syncthreads();
  const int in_total = ue.red2[0], in_before = ue.red2[1], neg_before = ue.red2[2];
  const int need = k - in_total;  // BAND tokens to keep (>= 1)

  // Band entry i is kept iff fewer than `need` entries come before it in
  // (key desc, position asc) order, i.e. have a larger composite
  // (key << 32) | ~position.  Counting them is a pass over the list per
  // entry (the list is short: tokens within a few error bounds of the
  // threshold); long lists are sorted instead.
  int chosen_before = 0;
  if (cut.bstar >= 0) {
    if (nband <= 2 * kChunkThreads) {
      for (int i = tid; i < nband; i += kChunkThreads) {
        const uint64_t x = ue.band[i];
        int rank = 0;
        for (int j = 0; j < nband; ++j) rank += ue.band[j] > x;
        if (rank < need) {
          const int t = (int)~(uint32_t)(x & 0xFFFFFFFFull);
          if (t < cstart) ++chosen_before;
          else if (t < cstart + kSelChunk) atomicOr(&ue.chosen[(t - cstart) >> 5], 1u << ((t - cstart) & 31));
        }
      }
    } else {
      // sort (key desc, position asc) = descending 64-bit composite
      int nb_pow = 1;
      while (nb_pow < nband) nb_pow <<= 1;
      for (int i = nband + tid; i < nb_pow; i += kChunkThreads) ue.band[i] = 0ull;
      __syncthreads();
      for (int size = 2; size <= nb_pow; size <<= 1)
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          for (int i = tid; i < nb_pow / 2; i += kChunkThreads) {
            const int lo = 2 * i - (i & (stride - 1));
            const int hi = lo + stride;
            const bool desc = (lo & size) == 0;
            const uint64_t x0 = ue.band[lo], x1 = ue.band[hi];
            if ((x0 < x1) == desc) {
              ue.band[lo] = x1;
              ue.band[hi] = x0;
            }
          }
          __syncthreads();
        }
      for (int i = tid; i < need && i < nband; i += kChunkThreads) {
        const int t = (int)~(uint32_t)(ue.band[i] & 0xFFFFFFFFull);
        if (t < cstart) ++chosen_before;
        else if (t < cstart + kSelChunk) atomicOr(&ue.chosen[(t - cstart) >> 5], 1u << ((t - cstart) & 31));
      }
    }
  }
  chosen_before = chunk_sum_i(chosen_before, ue.cs.redi);  // (barrier: bitmap complete)

  mask8(t0, v.L, x);
  uint32_t keep = 0;
  int nkeep = 0, nneg = 0;
#pragma unroll
  for (int e = 0; e < kPerThread; ++e) {
    const uint32_t cl = classify(v, cut, x[e], FAST);
    bool kp = cl == kIn;
    if (cl == kBand) {
      if (cut.bstar >= 0) {
        const int r = t0 + e - cstart;
        kp = (ue.chosen[r >> 5] >> (r & 31)) & 1u;
      } else {
        ++nneg;  // -inf filler: decided by rank below
      }
    }
    keep |= (uint32_t)kp << e;
    nkeep += kp;
  }
  int total;
  int offset;
  if (cut.bstar >= 0) {
    offset = in_before + chosen_before + block_excl_scan<kChunkThreads>(nkeep, ue.cs.tmp, &total);
  } else {
    // fewer finite scores than k: all finite kept, then -inf ones by position
    const int need_neg = k - in_total;
    const int neg_rank = neg_before + block_excl_scan<kChunkThreads>(nneg, ue.cs.tmp, &total);
    int taken_before = min(max(need_neg, 0), neg_before);
    // kept so far in earlier chunks: their finite ones plus their taken -inf
    offset = in_before + taken_before;
    // this thread: finite kept before it in the chunk + -inf taken before it
    int fin_prefix = block_excl_scan<kChunkThreads>(nkeep, ue.cs.tmp, &total);
    const int take_before_me = min(max(need_neg, 0), neg_rank) - taken_before;
    offset += fin_prefix + take_before_me;
    int r = neg_rank;
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      if (x[e] == -__builtin_inff()) {
        if (r < need_neg) keep |= 1u << e;
        ++r;
      }
    }
  }
#pragma unroll
  for (int e = 0; e < kPerThread; ++e)
    if ((keep >> e) & 1u) {
      if (offset < k) put_index(a, row, offset, t0 + e);
      ++offset;
    }
  if (a.counts && c == 0 && tid == 0) a.counts[row] = k;
}

// Rows of at most k tokens: every token kept, in order (chunk c's share),
// then the -1 padding and the count (chunk 0).
__device__ __forceinline__ void emit_all(const SelectArgs& a, int row, int c, int L) {
  const int tid = threadIdx.x, cstart = c * kSelChunk, k = a.k;
  for (int t = cstart + tid; t < min(L, cstart + kSelChunk); t += kChunkThreads) put_index(a, row, t, t);
  if (c == 0) {
    for (int i = L + tid; i < k; i += kChunkThreads) put_index(a, row, i, -1);
    if (a.counts && tid == 0) a.counts[row] = L;
  }
}

// Wave 0's per-chunk counts of a row (chunks tid and tid + 64).
__device__ __forceinline__ void load_chunk_counts(const SelectArgs& a, int row, int2 (&ccv)[2]) {
  const int tid = threadIdx.x;
  const int32_t* cc = a.chunk_counts + (int64_t)row * a.nchunks * 2;
  ccv[0] = ccv[1] = int2{0, 0};
  if (tid < kWave) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      if (tid + kWave * j < a.nchunks) ccv[j] = ld_coherent2(cc + 2 * (tid + kWave * j));
  }
}

template <bool FAST>
__global__ __launch_bounds__(kChunkThreads) void select_emit_kernel(SelectArgs a) {
  __shared__ EmitSmem u;
  __shared__ __attribute__((aligned(16))) float s_terms[kSelWaves][kWave];
  const int tid = threadIdx.x;
  const int row = blockIdx.x, c = blockIdx.y;  // chunk-major grid
  const int cstart = c * kSelChunk;
  // loads that do not depend on the row's statistics, in flight together
  float x[kPerThread];
  const int t0 = cstart + kPerThread * tid;
  load8_raw(a.scores + (int64_t)row * a.row_stride, t0, a.row_stride, x);
  int2 ccv[2];
  load_chunk_counts(a, row, ccv);
  const RowView v = row_view(a, row);
  if (v.L <= a.k) {  // every token kept (dense-equivalent)
    emit_all(a, row, c, v.L);
    return;
  }
  if (cstart >= v.L) return;
  const int32_t* st = a.stats + (int64_t)row * kStatStride;
  const int nband = st[2];
  if (nband > kBandCap) {
    if (c == 0) select_row_block<kMaxNI, false, FAST>(a, row, u.one, s_terms);
    return;
  }
  emit_chunk<FAST>(a, row, c, v, stored_cut(a, row), nband, x, ccv, u.e);
}

// ------------------------------------------------------------------ one launch

// The three passes above in one launch, for grids whose blocks are all
// resident at once: the blocks of a row meet at two row barriers (after the
// histogram, after the classification) instead of kernel boundaries, and
// keep their scores, view and cut in registers across them.
//
// A row barrier is an arrival counter in the row's statistics (cleared by
// the fast scorer or select_init): each block publishes its writes, adds
// one, and waits until every participating block has arrived.  The wait is
// bounded: a block that has waited spin_ticks (it can only happen when other
// work holds the CUs its partners need) finishes the whole row by itself
// with select_row_block, which is exact on its own, and the row's other
// blocks, which then never see it at the next barrier, do the same; every
// block that writes the row's outputs writes the same values.
constexpr int64_t kDefaultSpinTicks = 200000;  // 2 ms at the 100 MHz wall clock

__device__ __forceinline__ bool row_barrier(int32_t* counter, int target, int64_t ticks, int* s_flag) {
  wait_stores();  // this thread's coherent stores and atomics have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ok = 1;
    const uint64_t t_start = wall_clock64();
    while (ld_coherent(counter) < target) {
      if ((int64_t)(wall_clock64() - t_start) > ticks) {
        ok = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    *s_flag = ok;
  }
  __syncthreads();
  const bool ok = *s_flag != 0;
  __syncthreads();  // s_flag may be reused
  return ok;
}

template <bool FAST>
__global__ __launch_bounds__(kChunkThreads) void select_fused_kernel(SelectArgs a) {
  __shared__ union {
    struct {
      int hist[kBins];
      int red[kSelWaves];
      uint32_t red3[3][kSelWaves];
    } h;
    ClassifySmem<FAST> cl;
    EmitSmem em;
  } u;
  __shared__ __attribute__((aligned(16))) float s_terms[kSelWaves][kWave];
  __shared__ int s_flag;
  const int tid = threadIdx.x;
  const int row = blockIdx.x, c = blockIdx.y;  // chunk-major grid
  const int b = row / a.groups;
  int32_t* st = a.stats + (int64_t)row * kStatStride;
  const int64_t ticks = a.spin_ticks > 0 ? a.spin_ticks : kDefaultSpinTicks;
  // loads that do not depend on the row's statistics
  float x[kPerThread];
  const int t0 = c * kSelChunk + kPerThread * tid;
  load8_raw(a.scores + (int64_t)row * a.row_stride, t0, a.row_stride, x);
  const int tpage = FAST ? thread_page(a, b, t0) : -1;
  RowKeys r;
  if (a.span_slots) {
    r = reduce_span_slots(a, row, u.h.red3);
    // every block publishes the (identical) row keys and bound: a block that
    // finishes the row alone reads them back
    if (tid == 0) {
      st[0] = (int32_t)r.kmin;
      st[1] = (int32_t)r.kmax;
      a.row_bound[row] = r.bound;
    }
  } else {
    r = RowKeys{(uint32_t)st[0], (uint32_t)st[1], a.row_bound ? a.row_bound[row] : 0.0f};
  }
  RowView v = view_of_keys(a, row, r.kmin, r.kmax, -__builtin_inff());
  if (v.L <= a.k) {  // every token kept (dense-equivalent): no barriers
    emit_all(a, row, c, v.L);
    return;
  }
  const int nch = (v.L + kSelChunk - 1) / kSelChunk;  // the row's participating blocks
  if (c >= nch) return;
  // A top-k hint is not used here: its floor costs every block a scan of the
  // hint and of the scores it names, and can only narrow the histogram's
  // range, while this pass's band is already a few dozen tokens per row
  // (the hint never changes the result; its write-back is the emission's).
  __syncthreads();  // stats written above, before a fallback reads them back

  // ---- histogram (select_hist_kernel's pass)
  mask8(t0, v.L, x);
  if (v.any_finite) {
    for (int i = tid; i < kBins; i += kChunkThreads) u.h.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kPerThread; ++e) {
      const bool fin = __builtin_isfinite(x[e]) && x[e] >= v.lo;
      hist_add(u.h.hist, fin ? bin_of_v(v, x[e]) : 0, fin);
    }
    __syncthreads();
    int32_t* gh = st + 8;
    for (int i = tid; i < kBins; i += kChunkThreads)
      if (u.h.hist[i]) atomicAdd(&gh[i], u.h.hist[i]);
  }
  // the block finishes the row alone after a barrier it waited too long
  // at, and block 0 does when the band overflows its list (one call site)
  bool solo = !row_barrier(st + kStatBarrier, nch, ticks, &s_flag);
  if (!solo) {
    // ---- classification (select_classify_kernel's pass)
    int hb[kBinsPerThread];
#pragma unroll
    for (int j = 0; j < kBinsPerThread; ++j) hb[j] = ld_coherent(st + 8 + tid + j * kChunkThreads);
    const RowCut cut = classify_chunk<FAST>(a, row, c, v, x, hb, tpage, u.cl, s_terms);
    solo = !row_barrier(st + kStatBarrier + 1, nch, ticks, &s_flag);
    if (!solo) {
      // ---- emission (select_emit_kernel's pass)
      const int nband = ld_coherent(st + 2);
      if (nband <= kBandCap) {
        int2 ccv[2];
        load_chunk_counts(a, row, ccv);
        emit_chunk<FAST>(a, row, c, v, cut, nband, x, ccv, u.em.e);  // (masking x again changes nothing)
        return;
      }
      if (c != 0) return;
    }
  }
  select_row_block<kMaxNI, false, FAST>(a, row, u.em.one, s_terms);
}

// ------------------------------------------------------------------ launch

int select_max_row() { return kMaxChunks * kMaxNI * kTile; }

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

size_t select_workspace_bytes(int rows, int row_stride) {
  const int nch = (row_stride + kSelChunk - 1) / kSelChunk;
  return align256((size_t)rows * row_stride * 4) + align256((size_t)rows * kStatStride * 4) +
         align256((size_t)rows * nch * 2 * 4) + align256((size_t)rows * kBandCap * 8);
}

void select_bind_workspace(SelectArgs* a, void* ws) {
  const int rows = a->batch * a->groups;
  a->nchunks = (a->row_stride + kSelChunk - 1) / kSelChunk;
  char* p = static_cast<char*>(ws);
  a->keys = reinterpret_cast<float*>(p);
  p += align256((size_t)rows * a->row_stride * 4);
  a->stats = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * kStatStride * 4);
  a->chunk_counts = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)rows * a->nchunks * 2 * 4);
  a->band = reinterpret_cast<uint64_t*>(p);
}

// Rows of at most NI * kTile tokens with exact scores: one block per row
// holds the row in registers and does the whole selection (no statistics,
// histogram or band passes between launches).
template <int NI>
__global__ __launch_bounds__(kSelThreads) void select_rows_kernel(SelectArgs a) {
  __shared__ SelSharedN<NI * kSelThreads> sh;
  __shared__ __attribute__((aligned(16))) float s_terms[kSelWaves][kWave];
  select_row_block<NI, true, false>(a, blockIdx.x, sh, s_terms);
}

// Rows of at most 256 NI tokens with exact scores, when there are many rows:
// one wave per row holds the row's keys in registers and selects alone
// (wave_select.h), with no block barrier.
template <int NI>
__global__ __launch_bounds__(64) void select_wave_rows_kernel(SelectArgs a) {
  __shared__ WaveSelectSmem<NI> sh;
  const int row = blockIdx.x, lane = threadIdx.x;
  const int L = clamp_len(a.kv_lens[row / a.groups], a.row_stride);
  const int k = a.k;
  int32_t* const out = a.indices + (int64_t)row * k;
  int32_t* const wb = a.writeback ? a.writeback + (int64_t)row * a.wb_stride : nullptr;
  if (L <= k) {  // every token is kept
    for (int i = lane; i < k; i += 64) {
      out[i] = i < L ? i : -1;
      if (wb) wb[i] = i < L ? i : -1;
    }
    if (a.counts && lane == 0) a.counts[row] = L;
    return;
  }
  const float* s = a.scores + (int64_t)row * a.row_stride;
  const bool vec = (a.row_stride % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0;
  // keys of the tokens below L; 0 past it
  uint32_t key[NI][4];
  uint32_t kmin1 = 0xFFFFFFFFu, kmax = 0u;  // kmin1: smallest live key - 1 (key 0 wraps)
  const bool full = vec && L >= 256 * NI;  // every element present: no per-token checks
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int t0 = 4 * (lane + 64 * i);
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if (full) {
      const float4 q = *reinterpret_cast<const float4*>(s + t0);
      x[0] = q.x; x[1] = q.y; x[2] = q.z; x[3] = q.w;
    } else if (vec) {
      if (t0 < L) {  // t0 + 3 < row_stride
        const float4 q = *reinterpret_cast<const float4*>(s + t0);
        x[0] = q.x; x[1] = q.y; x[2] = q.z; x[3] = q.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t0 + e < L) x[e] = s[t0 + e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t kk = max(wave_key(x[e]), 1u);
      if (!full) kk = t0 + e < L ? kk : 0u;
      asm volatile("" : "+v"(kk));  // the scores are not kept beside their keys
      key[i][e] = kk;
      kmin1 = min(kmin1, kk - 1u);
      kmax = max(kmax, kk);
    }
  }
  const uint32_t kmin = uniform_u32(wave_min_u32(kmin1)) + 1u;
  kmax = uniform_u32(wave_max_u32(kmax));
  wave_select<NI>(key, kmin, kmax, k, out, wb, sh);
  if (a.counts && lane == 0) a.counts[row] = k;
}

// rows for which the one-wave selection pays (many short rows)
constexpr int kWaveRowsMin = 2048;

constexpr int kShortRow = 8 * kTile;  // 16384 tokens

bool select_short_path(const SelectArgs& a) { return !a.row_bound && a.row_stride <= kShortRow; }

hipError_t launch_select_short(const SelectArgs& a, hipStream_t st) {
  const int rows = a.batch * a.groups;
  if (rows == 0) return hipSuccess;
  {
    // SD_SELECT_WAVE_ROWS (tests): 1 takes the one-wave path for any row
    // count, 0 never
    const char* env = getenv("SD_SELECT_WAVE_ROWS");
    const bool force = env && env[0] == '1', never = env && env[0] == '0';
    if (!never && (force || rows >= kWaveRowsMin) && a.row_stride <= 4096) {
      if (a.row_stride <= 1024) select_wave_rows_kernel<4><<<rows, 64, 0, st>>>(a);
      else if (a.row_stride <= 2048) select_wave_rows_kernel<8><<<rows, 64, 0, st>>>(a);
      else select_wave_rows_kernel<16><<<rows, 64, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  if (a.row_stride <= kTile) select_rows_kernel<1><<<rows, kSelThreads, 0, st>>>(a);
  else if (a.row_stride <= 2 * kTile) select_rows_kernel<2><<<rows, kSelThreads, 0, st>>>(a);
  else if (a.row_stride <= 4 * kTile) select_rows_kernel<4><<<rows, kSelThreads, 0, st>>>(a);
  else select_rows_kernel<8><<<rows, kSelThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_select_init(const SelectArgs& a, hipStream_t st) {
  const int rows = a.batch * a.groups;
  if (rows == 0) return hipSuccess;
  select_init_kernel<<<rows, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_select_stats(const SelectArgs& a, hipStream_t st) {
  const int rows = a.batch * a.groups;
  if (rows == 0 || a.nchunks == 0) return hipSuccess;
  select_stats_kernel<<<dim3(a.nchunks, rows), kChunkThreads, 0, st>>>(a);
  return hipGetLastError();
}

// Blocks of the one-launch selection that may be resident at once on this
// device (occupancy times compute units), looked up once per device.
static int fused_capacity(bool fast) {
  static int cap[2][64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int& c = cap[fast][dev];
  if (c == 0) {
    int per_cu = 0, cus = 0;
    const hipError_t e = fast ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, select_fused_kernel<true>, kChunkThreads, 0)
                              : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, select_fused_kernel<false>, kChunkThreads, 0);
    if (e != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      c = -1;
    else
      c = per_cu * cus;
  }
  return c;
}

hipError_t launch_select(const SelectArgs& a, hipStream_t st) {
  const int rows = a.batch * a.groups;
  if (rows == 0) return hipSuccess;
  if (a.row_stride > select_max_row()) return hipErrorInvalidValue;
  {
    // one launch when the whole grid fits in half of what the device holds
    // at once (so that a second call on another stream fits beside it)
    const int ny = max(max(a.nchunks, 1), (a.k + kSelChunk - 1) / kSelChunk);
    const int64_t blocks = (int64_t)rows * ny;
    const int cap = fused_capacity(a.row_bound != nullptr);
    // SD_SELECT_ONE_LAUNCH=0 (tests): always the three launches
    const char* one = getenv("SD_SELECT_ONE_LAUNCH");
    const bool allowed = !(one && one[0] == '0');
    if (allowed && cap > 0 && 2 * blocks <= cap) {
      const dim3 fgrid(rows, ny);
      SelectArgs f = a;
      // SD_SELECT_SPIN_TICKS (tests): a shorter wait at the row barriers, to
      // exercise the path where blocks finish their rows alone
      if (f.spin_ticks <= 0) {
        const char* env = getenv("SD_SELECT_SPIN_TICKS");
        if (env && *env) f.spin_ticks = strtoll(env, nullptr, 10);
      }
      if (a.row_bound) select_fused_kernel<true><<<fgrid, kChunkThreads, 0, st>>>(f);
      else select_fused_kernel<false><<<fgrid, kChunkThreads, 0, st>>>(f);
      return hipGetLastError();
    }
  }
  const dim3 grid(max(a.nchunks, 1), rows);
  // classify and emit run chunk-major (block x = row, y = chunk): blocks
  // handed out together belong to different rows, the row's blocks share an
  // XCD when the row count is a multiple of 8, and the blocks of chunks past
  // short rows' ends come last
  const dim3 cgrid(rows, max(a.nchunks, 1));
  if (a.nchunks > 0) {
    select_hist_kernel<<<grid, kChunkThreads, 0, st>>>(a);
    if (a.row_bound) select_classify_kernel<true><<<cgrid, kChunkThreads, 0, st>>>(a);
    else select_classify_kernel<false><<<cgrid, kChunkThreads, 0, st>>>(a);
  }
  // emit also covers the output of rows whose tokens are all kept
  const dim3 egrid(rows, max(a.nchunks, (a.k + kSelChunk - 1) / kSelChunk));
  if (a.row_bound) select_emit_kernel<true><<<egrid, kChunkThreads, 0, st>>>(a);
  else select_emit_kernel<false><<<egrid, kChunkThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sd
