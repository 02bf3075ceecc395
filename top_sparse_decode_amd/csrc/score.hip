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

constexpr int kScoreIters = 16;                    // 32-token tiles per wave
constexpr int kScoreSpan = 4 * 32 * kScoreIters;   // tokens per block

// MT = query heads / 16.  Each wave handles 32 consecutive tokens per
// iteration as two 16-token N tiles: C[16 heads x 16 tokens] per (M tile, N
// tile), K = 128 split into four 32-wide steps.  MFMA operand layout for
// 16x16x32 bf16: lane l holds A[row l%16][8 k-values], B[8 k-values][col
// l%16], and C[rows 4*(l/16)+r][col l%16].  Which head dims a lane's 8
// k-values stand for is free as long as A and B agree; here k-step ks, lane
// group l/16 carries dims 32*ks + 8*(l/16) .. +8, so four lanes read 64
// contiguous bytes of a key row.
template <int MT>
__global__ __launch_bounds__(256) void score_dsa_mfma_kernel(ScoreArgs a) {
  constexpr int D = 128;
  constexpr int KS = D / 32;
  constexpr int G = 16 * MT;
  __shared__ float s_a[D];   // a_d = sum_h |w_h| |q_hd|
  __shared__ float s_part[2][D];
  __shared__ int s_page[kScoreSpan / 16 + 2];  // page ids of the block's tokens (-1: absent)
  // the group's query heads, rows padded by 16 bytes so a fragment's 16 rows
  // fall on different banks
  __shared__ __attribute__((aligned(16))) uint16_t s_q[G][D + 8];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.y / a.num_kv_heads, g = blockIdx.y % a.num_kv_heads;
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  constexpr int iters = kScoreIters;
  constexpr int span = kScoreSpan;
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

  // page ids of the span: logical page p of the block -> physical page
  {
    const int p0 = tb0 / a.page_size;
    const int np = (tb0 + span - 1) / a.page_size - p0 + 1;
    for (int i = threadIdx.x; i < np; i += 256) {
      const int lp = p0 + i;
      int page = -1;
      if (lp < a.max_pages && lp * a.page_size < L) {
        page = a.block_table[(int64_t)b * a.max_pages + lp];
        if (page < 0 || page >= a.num_pages) page = -1;
      }
      s_page[i] = page;
    }
  }
  __syncthreads();  // s_page visible
  const int col = lane & 15, grp = lane >> 4;
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.k) + (int64_t)g * a.head_stride;
  // One 32-token tile (two 16-token N tiles) per step.
  struct Tile {
    bf16x8 kf[2][KS];
    bool ok[2];
  };
  // Page ids of the block's span come from LDS (staged below), so a tile's
  // loads never wait on a global load issued after the previous tile's; an
  // absent token loads row 0 of the pool (always mapped) and is masked.
  auto load_tile = [&](int t0, Tile& T) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int t = t0 + 16 * n + col;
      const int page = t < L ? s_page[t / a.page_size - tb0 / a.page_size] : -1;
      const bool ok = page >= 0;
      const int64_t off = ok ? (int64_t)page * a.page_stride + (int64_t)(t % a.page_size) * a.token_stride : 0;
      T.ok[n] = ok;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        T.kf[n][ks] = *reinterpret_cast<const bf16x8*>(kbase + off + 32 * ks + 8 * grp);
    }
  };
  auto tile_t0 = [&](int it) { return tb0 + (it * 4 + wid) * 32; };
  // The first two tiles' loads go out before the per-block set-up below.
  Tile T[3];
  load_tile(tile_t0(0), T[0]);
  load_tile(tile_t0(1), T[1]);

  // the group's query rows into LDS (visible after the barriers below)
  for (int i = threadIdx.x; i < G * D / 8; i += 256) {
    const int h = i / (D / 8), c = i % (D / 8);
    *reinterpret_cast<uint4*>(&s_q[h][8 * c]) = *reinterpret_cast<const uint4*>(qb + h * D + 8 * c);
  }
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

  float wv[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = wb[16 * mt + 4 * grp + r];
  // The bound's sum_d a_d |k_d| runs on the matrix cores as one more M tile
  // whose row 0 holds a_d rounded up to bf16 (an upper bound of a_d) and
  // whose B operand is |K|.
  bf16x8 af[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    u32x4 w4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = col == 0 ? bf16_round_up(s_a[32 * ks + 8 * grp + 2 * e]) : 0u;
      const uint32_t hi = col == 0 ? bf16_round_up(s_a[32 * ks + 8 * grp + 2 * e + 1]) : 0u;
      w4[e] = lo | (hi << 16);
    }
    af[ks] = __builtin_bit_cast(bf16x8, w4);
  }
  const float u24 = 5.9604644775390625e-8f, u23 = 1.1920928955078125e-7f;
  const float gD = gamma_n((float)D, u23), gH = gamma_n((float)(G + 1), u24);
  const float bcoef = 2.0f * gH * (1.0f + gD) + 2.0f * gD;
  float dmax = 0.0f;
  float smin = __builtin_inff(), smax = -__builtin_inff();  // finite scores of this lane

  auto compute_tile = [&](int t0, Tile& T) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      if (!T.ok[n]) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) T.kf[n][ks] = bf16x8{};
      }
      floatx4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *reinterpret_cast<const bf16x8*>(&s_q[16 * mt + col][32 * ks + 8 * grp]), T.kf[n][ks], acc[mt], 0, 0, 0);
      }
      floatx4 accb = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 kw = __builtin_bit_cast(u32x4, T.kf[n][ks]);
        const u32x4 ka = kw & 0x7FFF7FFFu;  // |K|
        accb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], __builtin_bit_cast(bf16x8, ka), accb, 0, 0, 0);
      }
      // s~ = sum_h w_h relu(dot_h): this lane's 4*MT heads, then the 4 lane groups
      float s = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s = __builtin_fmaf(wv[mt][r], fmaxf(acc[mt][r], 0.0f), s);
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      const int t = t0 + 16 * n + col;
      if (grp == 0 && T.ok[n]) {
        // B_t = sum_d a_d |k_td| (row 0 of the extra tile, lanes 0..15) bounds both
        // sum_h |w_h| relu(.) terms, so |s~ - s| <= B_t * (2 gH (1 + gD) + 2 gD)
        dmax = fmaxf(dmax, accb[0] * bcoef);
      }
      if (grp == 0 && t < a.max_kv_len) row[t] = T.ok[n] ? s : -__builtin_inff();
      if (T.ok[n]) {
        smin = fminf(smin, s);
        smax = fmaxf(smax, s);
      }
    }
  };
  // Fully unrolled, with every look-ahead load unconditional (a tile past
  // the row reads pool row 0 and is masked), so the compiler's wait counts
  // are exact: tiles it+1 and it+2 are in flight while tile it is computed.
#pragma unroll
  for (int it = 0; it < iters; ++it) {
    if (it + 2 < iters) load_tile(tile_t0(it + 2), T[(it + 2) % 3]);
    if (tile_t0(it) < a.max_kv_len) compute_tile(tile_t0(it), T[it % 3]);
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
  dim3 grid((a.max_kv_len + kScoreSpan - 1) / kScoreSpan, a.batch * a.num_kv_heads);
  switch (G / 16) {
    case 1: score_dsa_mfma_kernel<1><<<grid, 256, 0, st>>>(a); break;
    case 2: score_dsa_mfma_kernel<2><<<grid, 256, 0, st>>>(a); break;
    case 3: score_dsa_mfma_kernel<3><<<grid, 256, 0, st>>>(a); break;
    case 4: score_dsa_mfma_kernel<4><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace sd
