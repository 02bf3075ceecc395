// score.hip -- paged-K token scoring for top-k sparse decode.
//
// Every cached token t < kv_len of request b is scored from the paged K pool
// through the block table, reading pages in place ("Add TriAttention KV-cache
// compression method", Key Design Decisions: direct paged-pool scoring with
// no gather or reformat; Summary: per-head scores reduced to one per KV head).
//
// Two kernels:
//  * score_exact_kernel: one lane per token; each lane evaluates the binary32
//    dot products left to right over the head dimension (one rounding per
//    product and per sum; for bf16 operands the product is exact, so a fused
//    multiply-add per step gives the same bits), then reduces over the group's
//    heads in head order.  Bit-identical to any other evaluation in that order.
//  * score_dsa_mfma_kernel: the DSA indexer score s_t = sum_h w_h relu(q_h.k_t)
//    ("Overlap DSA heuristic prev_topk write-back on the aux stream",
//    Description: the indexer scores every token before the top-k kernel) on
//    bf16 MFMA 16x16x32 tiles -- heads x tokens x head_dim is a real dense
//    contraction there (64 x tokens x 128).  It also produces a rigorous
//    per-row bound on |fast score - exact score| so that selection can still
//    be made exact (see topk.hip).
#include "common.h"
#include "kernels.h"

namespace sd {

// ------------------------------------------------------------------ exact

template <typename KT>
struct Elems;
template <>
struct Elems<float> {
  static constexpr int kPerUnit = 4;  // elements per 16-byte unit
};
template <>
struct Elems<uint16_t> {
  static constexpr int kPerUnit = 8;
};

__device__ __forceinline__ void unpack_unit(const uint4& u, float (&v)[4]) {
  v[0] = __uint_as_float(u.x);
  v[1] = __uint_as_float(u.y);
  v[2] = __uint_as_float(u.z);
  v[3] = __uint_as_float(u.w);
}
__device__ __forceinline__ void unpack_unit(const uint4& u, float (&v)[8]) {
  v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
  v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
  v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
  v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
}

// acc + q*k with the product rounded, then the sum rounded.  For bf16 q and
// k the product is exact in binary32, so the fused form is the same value.
template <typename KT>
__device__ __forceinline__ float dot_step(float acc, float q, float k);
template <>
__device__ __forceinline__ float dot_step<float>(float acc, float q, float k) {
  return __fadd_rn(acc, __fmul_rn(q, k));
}
template <>
__device__ __forceinline__ float dot_step<uint16_t>(float acc, float q, float k) {
  return __builtin_fmaf(q, k, acc);
}

// Fold a wave's finite scores into the row's min / max keys (selection
// statistics): one atomic pair per wave.
__device__ __forceinline__ void note_minmax(int32_t* stat, float s, bool finite) {
  uint32_t kmin = finite ? score_key(s) : 0xFFFFFFFFu;
  uint32_t kmax = finite ? score_key(s) : 0u;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o));
  }
  if ((threadIdx.x & 63) == 0 && kmin <= kmax) {
    atomicMin(reinterpret_cast<unsigned int*>(stat), kmin);
    atomicMax(reinterpret_cast<unsigned int*>(stat + 1), kmax);
  }
}

template <typename KT, int G>
__global__ __launch_bounds__(256) void score_exact_kernel(ScoreArgs a) {
  constexpr int EPU = Elems<KT>::kPerUnit;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.y / a.num_kv_heads, g = blockIdx.y % a.num_kv_heads;
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int t = (blockIdx.x * 4 + wid) * kWave + lane;
  float* row = a.scores + (int64_t)blockIdx.y * a.max_kv_len;
  if (a.row_bound && blockIdx.x == 0 && threadIdx.x == 0) a.row_bound[blockIdx.y] = 0.0f;
  const bool in_row = t < a.max_kv_len;
  bool ok = in_row && t < L;
  int64_t off = 0;
  if (ok) {
    const int page = a.block_table[(int64_t)b * a.max_pages + t / a.page_size];
    ok = page >= 0 && page < a.num_pages;
    off = (int64_t)page * a.page_stride + (int64_t)g * a.head_stride +
          (int64_t)(t % a.page_size) * a.token_stride;
  }
  float s = -__builtin_inff();
  if (ok) {
    const KT* krow = reinterpret_cast<const KT*>(a.k) + off;
    const KT* qbase = reinterpret_cast<const KT*>(a.q) + ((int64_t)b * a.q_heads + g * G) * a.head_dim;
    float acc[G];
#pragma unroll
    for (int j = 0; j < G; ++j) acc[j] = 0.0f;
    const int units = a.head_dim / EPU;
    for (int u = 0; u < units; ++u) {
      float kv[EPU];
      unpack_unit(*reinterpret_cast<const uint4*>(krow + u * EPU), kv);
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float qv[EPU];
        unpack_unit(*reinterpret_cast<const uint4*>(qbase + (int64_t)j * a.head_dim + u * EPU), qv);
#pragma unroll
        for (int e = 0; e < EPU; ++e) acc[j] = dot_step<KT>(acc[j], qv[e], kv[e]);
      }
    }
    s = 0.0f;
    if (a.mode == 0) {
#pragma unroll
      for (int j = 0; j < G; ++j) s = __fadd_rn(s, __fmul_rn(acc[j], a.head_scale));
    } else if (a.mode == 1) {
#pragma unroll
      for (int j = 0; j < G; ++j) s = __fadd_rn(s, acc[j]);
      s = __fmul_rn(s, a.inv_g);
    } else {
      const float* w = a.head_weights + (int64_t)b * a.q_heads + g * G;
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float r = acc[j] > 0.0f ? acc[j] : 0.0f;
        s = __fadd_rn(s, __fmul_rn(w[j], r));
      }
    }
  }
  if (in_row) row[t] = s;
  if (a.row_stats) note_minmax(a.row_stats + (int64_t)blockIdx.y * kStatStride, s, ok && __builtin_isfinite(s));
}

// ------------------------------------------------------------------ fast DSA

// u = 2^-24 for the round-to-nearest VALU arithmetic; the matrix-core sums
// are charged 2^-23 per addition, which also covers truncating adders.
__device__ __forceinline__ float gamma_n(float n, float u) { return n * u / (1.0f - n * u); }

// MT = query heads / 16.  Each wave handles 32 consecutive tokens per
// iteration as two 16-token N tiles: C[16 heads x 16 tokens] per (M tile, N
// tile), K = 128 split into four 32-wide steps.  MFMA operand layout for
// 16x16x32 bf16: lane l holds A[row l%16][8 k-values], B[8 k-values][col
// l%16], and C[rows 4*(l/16)+r][col l%16].  Which head dims a lane's 8
// k-values stand for is free as long as A and B agree; here k-step ks, lane
// group l/16 carries dims 32*ks + 8*(l/16) .. +8, so four lanes read 64
// contiguous bytes of a key row.
template <int MT>
__global__ __launch_bounds__(256) void score_dsa_mfma_kernel(ScoreArgs a, int iters) {
  constexpr int D = 128;
  constexpr int KS = D / 32;
  constexpr int G = 16 * MT;
  __shared__ float s_a[D];   // a_d = sum_h |w_h| |q_hd|
  __shared__ float s_part[2][D];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.y / a.num_kv_heads, g = blockIdx.y % a.num_kv_heads;
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int span = 4 * 32 * iters;
  const int tb0 = blockIdx.x * span;
  float* row = a.scores + (int64_t)blockIdx.y * a.max_kv_len;
  if (tb0 >= a.max_kv_len) return;
  if (tb0 >= L) {  // nothing to score: fill -inf
    const int end = min(tb0 + span, a.max_kv_len);
    for (int t = tb0 + threadIdx.x; t < end; t += 256) row[t] = -__builtin_inff();
    return;
  }

  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.q_heads + g * G) * D;
  const float* wb = a.head_weights + (int64_t)b * a.q_heads + g * G;

  // a_d for the bound: 256 threads, two halves of the heads per dim.
  {
    const int d = threadIdx.x & (D - 1), half = threadIdx.x >> 7;
    float acc = 0.0f;
    for (int h = half; h < G; h += 2) acc += fabsf(wb[h]) * fabsf(bf16_to_f32(qb[h * D + d]));
    s_part[half][d] = acc;
    __syncthreads();
    if (threadIdx.x < D) s_a[threadIdx.x] = s_part[0][threadIdx.x] + s_part[1][threadIdx.x];
    __syncthreads();
  }

  const int col = lane & 15, grp = lane >> 4;
  bf16x8 qf[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[mt][ks] = *reinterpret_cast<const bf16x8*>(qb + (16 * mt + col) * D + 32 * ks + 8 * grp);
  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = wb[16 * mt + 4 * grp + r];
  float av[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) av[ks][e] = s_a[32 * ks + 8 * grp + e];

  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + (int64_t)g * a.head_stride;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const float u24 = 5.9604644775390625e-8f, u23 = 1.1920928955078125e-7f;
  const float gD = gamma_n((float)D, u23), gH = gamma_n((float)(G + 1), u24);
  float dmax = 0.0f;
  float smin = __builtin_inff(), smax = -__builtin_inff();  // finite scores of this lane

  // One 32-token tile (two 16-token N tiles) per step; the next tile's key
  // fragments are loaded before the current one is computed, so two tiles'
  // worth of loads (16 KB per wave) are in flight.
  struct Tile {
    bf16x8 kf[2][KS];
    bool ok[2];
  };
  auto load_tile = [&](int t0, Tile& T) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int t = t0 + 16 * n + col;
      bool ok = t < L;
      int64_t off = 0;
      if (ok) {
        const int page = bt[t / a.page_size];
        ok = page >= 0 && page < a.num_pages;
        off = (int64_t)page * a.page_stride + (int64_t)(t % a.page_size) * a.token_stride;
      }
      T.ok[n] = ok;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        T.kf[n][ks] = ok ? *reinterpret_cast<const bf16x8*>(kbase + off + 32 * ks + 8 * grp) : bf16x8{};
    }
  };
  auto compute_tile = [&](int t0, const Tile& T) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      floatx4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[mt][ks], T.kf[n][ks], acc[mt], 0, 0, 0);
      }
      float s = 0.0f, m = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = acc[mt][r] > 0.0f ? acc[mt][r] : 0.0f;
          s += wv[mt][r] * x;
          m += fabsf(wv[mt][r]) * x;
        }
      float bsum = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kw = __builtin_bit_cast(u32x4, T.kf[n][ks]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bsum += av[ks][2 * e] * fabsf(bf16_lo(kw[e]));
          bsum += av[ks][2 * e + 1] * fabsf(bf16_hi(kw[e]));
        }
      }
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      m += __shfl_xor(m, 16);
      m += __shfl_xor(m, 32);
      bsum += __shfl_xor(bsum, 16);
      bsum += __shfl_xor(bsum, 32);
      const int t = t0 + 16 * n + col;
      if (T.ok[n]) {
        // |fast - exact| <= gH*(2M + 2gD*B) + 2gD*B   (see topk.hip / header)
        const float bterm = 2.0f * gD * bsum;
        const float d = gH * (2.0f * m + bterm) + bterm;
        dmax = fmaxf(dmax, d);
      }
      if (grp == 0 && t < a.max_kv_len) row[t] = T.ok[n] ? s : -__builtin_inff();
      if (T.ok[n]) {
        smin = fminf(smin, s);
        smax = fmaxf(smax, s);
      }
    }
  };
  auto tile_t0 = [&](int it) { return tb0 + (it * 4 + wid) * 32; };
  auto live = [&](int it) { return it < iters && tile_t0(it) < a.max_kv_len; };
  Tile A, B;
  if (live(0)) load_tile(tile_t0(0), A);
  for (int it = 0; live(it); it += 2) {
    const bool hasB = live(it + 1);
    if (hasB) load_tile(tile_t0(it + 1), B);
    compute_tile(tile_t0(it), A);
    if (!hasB) break;
    const bool hasA = live(it + 2);
    if (hasA) load_tile(tile_t0(it + 2), A);
    compute_tile(tile_t0(it + 1), B);
    if (!hasA) break;
  }
  if (a.row_stats) {
    int32_t* stat = a.row_stats + (int64_t)blockIdx.y * kStatStride;
    note_minmax(stat, smin, smin <= smax);
    note_minmax(stat, smax, smin <= smax);
  }
  if (a.row_bound) {
    dmax = wave_max(dmax);
    // 1e-3 relative slack covers the rounding of the bound's own evaluation,
    // the absolute term any flushed subnormal.
    dmax = dmax * 1.001f + 1e-30f;
    if (lane == 0) atomicMax(reinterpret_cast<unsigned int*>(a.row_bound + blockIdx.y), __float_as_uint(dmax));
  }
}

// ------------------------------------------------------------------ launch

template <typename KT>
static hipError_t launch_exact_t(const ScoreArgs& a, hipStream_t st) {
  const int G = a.q_heads / a.num_kv_heads;
  dim3 grid((a.max_kv_len + 255) / 256, a.batch * a.num_kv_heads);
  switch (G) {
    case 1: score_exact_kernel<KT, 1><<<grid, 256, 0, st>>>(a); break;
    case 2: score_exact_kernel<KT, 2><<<grid, 256, 0, st>>>(a); break;
    case 4: score_exact_kernel<KT, 4><<<grid, 256, 0, st>>>(a); break;
    case 8: score_exact_kernel<KT, 8><<<grid, 256, 0, st>>>(a); break;
    case 16: score_exact_kernel<KT, 16><<<grid, 256, 0, st>>>(a); break;
    case 32: score_exact_kernel<KT, 32><<<grid, 256, 0, st>>>(a); break;
    case 64: score_exact_kernel<KT, 64><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool score_exact_supported(int G) {
  return G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64;
}

hipError_t launch_score_exact(const ScoreArgs& a, hipStream_t st) {
  if (a.batch == 0 || a.max_kv_len == 0) return hipSuccess;
  return a.dtype == 0 ? launch_exact_t<float>(a, st) : launch_exact_t<uint16_t>(a, st);
}

bool score_fast_supported(const ScoreArgs& a) {
  const int G = a.q_heads / a.num_kv_heads;
  return a.dtype == 1 && a.mode == 2 && a.head_dim == 128 && (G % 16) == 0 && G <= 64 &&
         (a.page_size % 16) == 0 && (a.token_stride % 8) == 0 && (a.page_stride % 8) == 0 &&
         (a.head_stride % 8) == 0;
}

hipError_t launch_score_fast(const ScoreArgs& a, hipStream_t st) {
  if (a.batch == 0 || a.max_kv_len == 0) return hipSuccess;
  const int G = a.q_heads / a.num_kv_heads;
  const int iters = 16;
  dim3 grid((a.max_kv_len + 4 * 32 * iters - 1) / (4 * 32 * iters), a.batch * a.num_kv_heads);
  switch (G / 16) {
    case 1: score_dsa_mfma_kernel<1><<<grid, 256, 0, st>>>(a, iters); break;
    case 2: score_dsa_mfma_kernel<2><<<grid, 256, 0, st>>>(a, iters); break;
    case 3: score_dsa_mfma_kernel<3><<<grid, 256, 0, st>>>(a, iters); break;
    case 4: score_dsa_mfma_kernel<4><<<grid, 256, 0, st>>>(a, iters); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sd
