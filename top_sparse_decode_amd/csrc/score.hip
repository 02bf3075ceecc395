// score.hip -- paged-K token scoring for top-k sparse decode.
//
// Every cached token t < kv_len of request b is scored from the paged K pool
// through the block table, reading pages in place ("Add TriAttention KV-cache
// compression method", Key Design Decisions: direct paged-pool scoring with
// no gather or reformat; Summary: per-head scores reduced to one per KV head).
//
// Kernels:
//  * score_exact_staged_kernel / score_exact_kernel: one lane per token; each
//    lane evaluates the binary32 dot products left to right over the head
//    dimension (one rounding per product and per sum; for bf16 operands the
//    product is exact, so a fused multiply-add per step gives the same bits),
//    then reduces over the group's heads in head order.  Bit-identical to any
//    other evaluation in that order.  The staged kernel brings K rows and the
//    query through LDS with whole-row loads; the other reads rows directly.
//  * score_dsa_kernel: the DSA indexer score s_t = sum_h w_h relu(q_h.k_t)
//    ("Overlap DSA heuristic prev_topk write-back on the aux stream",
//    Description: the indexer scores every token before the top-k kernel) on
//    bf16 MFMA 16x16x32 tiles -- heads x tokens x head_dim is a real dense
//    contraction there (64 x tokens x 128).  It also produces a rigorous
//    per-row bound on |fast score - exact score| so that selection can still
//    be made exact (see topk.hip).
//  * score_dsa_fp8_kernel: the same score over an FP8 E4M3 indexer cache with
//    one binary32 scale per row (codes widened exactly to bf16 for the matrix
//    cores, the bound on the fp8 matrix cores).
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

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
template <>
struct Elems<uint8_t> {  // fp8 codes; the query stays bf16
  static constexpr int kPerUnit = 16;
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

// One 16-byte unit of a K row as binary32 values; an fp8 unit is dequantized
// with its row scale.
template <typename KT>
__device__ __forceinline__ void cvt_k_unit(const uint4& u, float scale, float (&v)[Elems<KT>::kPerUnit]) {
  unpack_unit(u, v);
}
template <>
__device__ __forceinline__ void cvt_k_unit<uint8_t>(const uint4& u, float scale, float (&v)[16]) {
  fp8x4_dequant(u.x, scale, v);
  fp8x4_dequant(u.y, scale, v + 4);
  fp8x4_dequant(u.z, scale, v + 8);
  fp8x4_dequant(u.w, scale, v + 12);
}
template <typename KT>
__device__ __forceinline__ void load_k_unit(const KT* p, float scale, float (&v)[Elems<KT>::kPerUnit]) {
  cvt_k_unit<KT>(*reinterpret_cast<const uint4*>(p), scale, v);
}
// The query elements that meet one K unit (bf16 for an fp8 pool).
template <typename KT>
__device__ __forceinline__ void load_q_unit(const void* p, float (&v)[Elems<KT>::kPerUnit]) {
  unpack_unit(*reinterpret_cast<const uint4*>(p), v);
}
template <>
__device__ __forceinline__ void load_q_unit<uint8_t>(const void* p, float (&v)[16]) {
  const uint4* u = reinterpret_cast<const uint4*>(p);
  float lo[8], hi[8];
  unpack_unit(u[0], lo);
  unpack_unit(u[1], hi);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = lo[e];
    v[8 + e] = hi[e];
  }
}
template <typename KT>
struct QElem {
  typedef KT type;
};
template <>
struct QElem<uint8_t> {
  typedef uint16_t type;
};

// acc + q*k with the product rounded, then the sum rounded.  For bf16 q and
// k the product is exact in binary32, so the fused form is the same value.
template <typename KT>
__device__ __forceinline__ float dot_step(float acc, float q, float k) {
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

// The score of one token from its K row, in the exact order: the G dot
// products left to right over the head dimension, then the group reduction
// in head order.  kunit(u, v) yields K unit u and qunit(j, u, v) the query
// elements of head j that meet it, as binary32 values; UNITS > 0 fixes the
// number of units at compile time (else head_dim / units per element).
// The group reduction of the G dot products, in head order.
template <int G>
__device__ __forceinline__ float group_score(const ScoreArgs& a, int b, int g, const float (&acc)[G]) {
  float s = 0.0f;
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
  return s;
}

template <typename KT, int G, int UNITS, typename KUnit, typename QUnit>
__device__ __forceinline__ float exact_token_score(const ScoreArgs& a, int b, int g, KUnit&& kunit, QUnit&& qunit) {
  constexpr int EPU = Elems<KT>::kPerUnit;
  float acc[G];
#pragma unroll
  for (int j = 0; j < G; ++j) acc[j] = 0.0f;
  auto step = [&](int u) {
    float kv[EPU];
    kunit(u, kv);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float qv[EPU];
      qunit(j, u, qv);
#pragma unroll
      for (int e = 0; e < EPU; ++e) acc[j] = dot_step<KT>(acc[j], qv[e], kv[e]);
    }
  };
  if constexpr (UNITS > 0) {
#pragma unroll
    for (int u = 0; u < UNITS; ++u) step(u);
  } else {
    const int units = a.head_dim / EPU;
    for (int u = 0; u < units; ++u) step(u);
  }
  return group_score<G>(a, b, g, acc);
}

// Each lane reads its own K row from memory (any layout).
template <typename KT, int G>
__global__ __launch_bounds__(256) void score_exact_kernel(ScoreArgs a) {
  constexpr int EPU = Elems<KT>::kPerUnit;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.y / a.num_kv_heads, g = blockIdx.y % a.num_kv_heads;
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int t = (blockIdx.x * 4 + wid) * kWave + lane;
  float* row = a.scores + (int64_t)blockIdx.y * a.max_kv_len;
  const bool in_row = t < a.max_kv_len;
  bool ok = in_row && t < L;
  int64_t off = 0, scale_idx = 0;
  if (ok) {
    const int page = a.block_table[(int64_t)b * a.max_pages + t / a.page_size];
    ok = page >= 0 && page < a.num_pages;
    off = (int64_t)page * a.page_stride + (int64_t)g * a.head_stride +
          (int64_t)(t % a.page_size) * a.token_stride;
    scale_idx = fp8_scale_index(page, g, t % a.page_size, a.num_kv_heads, a.page_size);
  }
  float s = -__builtin_inff();
  if (ok) {
    typedef typename QElem<KT>::type QT;
    const KT* krow = reinterpret_cast<const KT*>(a.k) + off;
    const float ksc = std::is_same<KT, uint8_t>::value ? a.k_scale[scale_idx] : 1.0f;
    const QT* qbase = reinterpret_cast<const QT*>(a.q) + ((int64_t)b * a.q_heads + g * G) * a.head_dim;
    s = exact_token_score<KT, G, 0>(
        a, b, g, [&](int u, float (&kv)[EPU]) { load_k_unit<KT>(krow + u * EPU, ksc, kv); },
        [&](int j, int u, float (&qv)[EPU]) { load_q_unit<KT>(qbase + (int64_t)j * a.head_dim + u * EPU, qv); });
  }
  if (in_row) row[t] = s;
  if (a.row_stats) note_minmax(a.row_stats + (int64_t)blockIdx.y * kStatStride, s, ok && __builtin_isfinite(s));
}

// The same scores with the K rows staged through LDS.  A lane reading its
// own row straight from memory touches a different 128-byte line in every
// lane of every load; here a wave's 64 rows arrive with whole-row loads
// (each instruction covers UPR * 16 / ... one kilobyte: 64 / UPR complete
// rows) and each lane then reads its row from LDS.  Rows of UPR 16-byte
// units; unit p of row r sits at position p ^ ((r / (16 / UPR)) & (UPR - 1)),
// so the 16 lanes of each read phase hit 64 different banks (rows of 256 bytes
// lie 64 banks apart, rows of 128 bytes 32).
template <typename KT, int G, int UPR>
__global__ __launch_bounds__(256) void score_exact_staged_kernel(ScoreArgs a) {
  constexpr int EPU = Elems<KT>::kPerUnit;
  typedef typename QElem<KT>::type QT;
  // the group's G query rows: UPR units of K meet UPR * EPU query elements each
  constexpr int kQUnits = G * UPR * EPU * (int)sizeof(QT) / 16;
  __shared__ uint4 s_rows[4][64 * UPR];
  __shared__ uint4 s_q[kQUnits];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.y / a.num_kv_heads, g = blockIdx.y % a.num_kv_heads;
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int t = (blockIdx.x * 4 + wid) * kWave + lane;
  float* row = a.scores + (int64_t)blockIdx.y * a.max_kv_len;
  const bool in_row = t < a.max_kv_len;
  bool ok = in_row && t < L;
  int64_t off = 0, scale_idx = 0;
  if (ok) {
    const int page = a.block_table[(int64_t)b * a.max_pages + t / a.page_size];
    ok = page >= 0 && page < a.num_pages;
    off = (int64_t)page * a.page_stride + (int64_t)g * a.head_stride +
          (int64_t)(t % a.page_size) * a.token_stride;
    scale_idx = fp8_scale_index(page, g, t % a.page_size, a.num_kv_heads, a.page_size);
  }
  // the query rows (contiguous: heads g*G .. g*G+G-1 of request b), loaded
  // with the K rows below and written to LDS after them
  constexpr int kQPerThread = (kQUnits + 255) / 256;
  uint4 qreg[kQPerThread];
  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(reinterpret_cast<const QT*>(a.q) +
                                                       ((int64_t)b * a.q_heads + g * G) * a.head_dim);
#pragma unroll
    for (int k = 0; k < kQPerThread; ++k) qreg[k] = qsrc[min((int)threadIdx.x + 256 * k, kQUnits - 1)];
  }
  // byte offset of this lane's row, -1 when it is not read
  const int64_t rb = ok ? off * (int64_t)sizeof(KT) : -1;
  const uint32_t rb_lo = (uint32_t)(uint64_t)rb, rb_hi = (uint32_t)((uint64_t)rb >> 32);
  const char* kb = reinterpret_cast<const char*>(a.k);
  constexpr int kRowsPerRead = 64 / UPR;
  auto swz = [](int r) { return (r / (16 / UPR)) & (UPR - 1); };
  uint4 v[UPR];
#pragma unroll
  for (int c = 0; c < UPR; ++c) {
    const int r = c * kRowsPerRead + lane / UPR, p = lane % UPR;
    const uint32_t lo = (uint32_t)__shfl((int)rb_lo, r), hi = (uint32_t)__shfl((int)rb_hi, r);
    const int64_t src = (int64_t)(((uint64_t)hi << 32) | lo);
    // rows not read load the pool's first unit instead (branch-free, so all
    // UPR loads are in flight together); their values are never used
    v[c] = *reinterpret_cast<const uint4*>(kb + (src >= 0 ? src + 16 * p : 0));
  }
#pragma unroll
  for (int c = 0; c < UPR; ++c) {
    const int r = c * kRowsPerRead + lane / UPR, p = lane % UPR;
    s_rows[wid][r * UPR + (p ^ swz(r))] = v[c];
  }
  // (threads past the last unit all write the last one, the same value)
#pragma unroll
  for (int k = 0; k < kQPerThread; ++k) s_q[min((int)threadIdx.x + 256 * k, kQUnits - 1)] = qreg[k];
  __syncthreads();
  float s = -__builtin_inff();
  if (ok) {
    const float ksc = std::is_same<KT, uint8_t>::value ? a.k_scale[scale_idx] : 1.0f;
    const uint4* mine = &s_rows[wid][lane * UPR];
    const int sw = swz(lane);
    // query units: QT elements u*EPU .. of head j (one 16-byte unit for bf16 or
    // f32 K, two for fp8 K), the same address in every lane
    constexpr int kQPerK = EPU * (int)sizeof(QT) / 16;
    s = exact_token_score<KT, G, UPR>(
        a, b, g, [&](int u, float (&kv)[EPU]) { cvt_k_unit<KT>(mine[u ^ sw], ksc, kv); },
        [&](int j, int u, float (&qv)[EPU]) { load_q_unit<KT>(&s_q[(j * UPR + u) * kQPerK], qv); });
  }
  if (in_row) row[t] = s;
  if (a.row_stats) note_minmax(a.row_stats + (int64_t)blockIdx.y * kStatStride, s, ok && __builtin_isfinite(s));
}

// Four heads' dot products over one 8-element unit: acc_j + q_j,e k_e for
// e = 0..7 in order, each a fused multiply-add (one rounding, as fmaf), the
// four chains interleaved so that no product waits on the one before it.
// q_j,e comes from lane L_j of this lane's 16-lane row by a DPP row
// broadcast, so every lane of the row uses the same query unit.  One asm
// block: two wait states first, for a query register written by the vector
// unit just before (the block writes none of its broadcast sources).
template <int L0, int L1, int L2, int L3>
__device__ __forceinline__ void fmac8x4_row_bcast(float (&acc)[4], const float (&q0)[8], const float (&q1)[8],
                                                  const float (&q2)[8], const float (&q3)[8], const float (&k)[8]) {
  asm volatile(
      "s_nop 1\n\t"
      "v_fmac_f32_dpp %0, %4, %36 row_newbcast:%44 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %12, %36 row_newbcast:%45 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %20, %36 row_newbcast:%46 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %28, %36 row_newbcast:%47 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %5, %37 row_newbcast:%44 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %13, %37 row_newbcast:%45 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %21, %37 row_newbcast:%46 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %29, %37 row_newbcast:%47 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %6, %38 row_newbcast:%44 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %14, %38 row_newbcast:%45 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %22, %38 row_newbcast:%46 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %30, %38 row_newbcast:%47 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %7, %39 row_newbcast:%44 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %15, %39 row_newbcast:%45 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %23, %39 row_newbcast:%46 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %31, %39 row_newbcast:%47 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %8, %40 row_newbcast:%44 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %16, %40 row_newbcast:%45 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %24, %40 row_newbcast:%46 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %32, %40 row_newbcast:%47 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %9, %41 row_newbcast:%44 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %17, %41 row_newbcast:%45 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %25, %41 row_newbcast:%46 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %33, %41 row_newbcast:%47 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %10, %42 row_newbcast:%44 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %18, %42 row_newbcast:%45 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %26, %42 row_newbcast:%46 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %34, %42 row_newbcast:%47 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %0, %11, %43 row_newbcast:%44 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %1, %19, %43 row_newbcast:%45 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %2, %27, %43 row_newbcast:%46 row_mask:0xf bank_mask:0xf\n\t"
      "v_fmac_f32_dpp %3, %35, %43 row_newbcast:%47 row_mask:0xf bank_mask:0xf\n\t"
      : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3])
      : "v"(q0[0]), "v"(q0[1]), "v"(q0[2]), "v"(q0[3]), "v"(q0[4]), "v"(q0[5]), "v"(q0[6]), "v"(q0[7]), "v"(q1[0]), "v"(q1[1]), "v"(q1[2]), "v"(q1[3]), "v"(q1[4]), "v"(q1[5]), "v"(q1[6]), "v"(q1[7]), "v"(q2[0]), "v"(q2[1]), "v"(q2[2]), "v"(q2[3]), "v"(q2[4]), "v"(q2[5]), "v"(q2[6]), "v"(q2[7]), "v"(q3[0]), "v"(q3[1]), "v"(q3[2]), "v"(q3[3]), "v"(q3[4]), "v"(q3[5]), "v"(q3[6]), "v"(q3[7]),
        "v"(k[0]), "v"(k[1]), "v"(k[2]), "v"(k[3]), "v"(k[4]), "v"(k[5]), "v"(k[6]), "v"(k[7]), "i"(L0), "i"(L1), "i"(L2), "i"(L3));
}

// The exact scores of bf16 K rows (128 or 256 bytes, staged through LDS as in
// score_exact_staged_kernel) with the query in registers: the group's G x
// UPR query units, widened to binary32 once, sit one unit per lane of every
// 16-lane row (unit F = 16 n + i in lane i, registers qv[n]), and each
// product takes its query element from the row by a DPP broadcast.  The
// per-token work is then the K widening and one fused multiply-add per
// product: no per-lane query reads or widening, no LDS traffic for the query.
// The order is exact_token_score's (each head's dot left to right, then the
// group reduction).  Every lane runs the products (a broadcast must not read
// an inactive lane); tokens that are not usable are dropped afterwards.
template <int G, int UPR>
__global__ __launch_bounds__(256) void score_exact_bcast_kernel(ScoreArgs a) {
  constexpr int NG = G * UPR / 16;  // query registers groups of eight values
  static_assert((G * UPR) % 16 == 0 && NG >= 1 && NG <= 8, "query units must fill whole 16-lane rows");
  __shared__ uint4 s_rows[4][64 * UPR];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int b = blockIdx.y / a.num_kv_heads, g = blockIdx.y % a.num_kv_heads;
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int t = (blockIdx.x * 4 + wid) * kWave + lane;
  float* row = a.scores + (int64_t)blockIdx.y * a.max_kv_len;
  const bool in_row = t < a.max_kv_len;
  bool ok = in_row && t < L;
  int64_t off = 0;
  if (ok) {
    const int page = a.block_table[(int64_t)b * a.max_pages + t / a.page_size];
    ok = page >= 0 && page < a.num_pages;
    off = (int64_t)page * a.page_stride + (int64_t)g * a.head_stride + (int64_t)(t % a.page_size) * a.token_stride;
  }
  // query unit F of the group (head F / UPR, unit F % UPR) for F = 16 n + lane % 16
  uint4 qraw[NG];
  {
    const uint4* qsrc = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) +
                                                       ((int64_t)b * a.q_heads + g * G) * a.head_dim);
#pragma unroll
    for (int n = 0; n < NG; ++n) qraw[n] = qsrc[16 * n + (lane & 15)];
  }
  const int64_t rb = ok ? off * 2 : -1;
  const uint32_t rb_lo = (uint32_t)(uint64_t)rb, rb_hi = (uint32_t)((uint64_t)rb >> 32);
  const char* kb = reinterpret_cast<const char*>(a.k);
  constexpr int kRowsPerRead = 64 / UPR;
  auto swz = [](int r) { return (r / (16 / UPR)) & (UPR - 1); };
  uint4 v[UPR];
#pragma unroll
  for (int c = 0; c < UPR; ++c) {
    const int r = c * kRowsPerRead + lane / UPR, p = lane % UPR;
    const uint32_t lo = (uint32_t)__shfl((int)rb_lo, r), hi = (uint32_t)__shfl((int)rb_hi, r);
    const int64_t src = (int64_t)(((uint64_t)hi << 32) | lo);
    v[c] = *reinterpret_cast<const uint4*>(kb + (src >= 0 ? src + 16 * p : 0));
  }
#pragma unroll
  for (int c = 0; c < UPR; ++c) {
    const int r = c * kRowsPerRead + lane / UPR, p = lane % UPR;
    s_rows[wid][r * UPR + (p ^ swz(r))] = v[c];
  }
  float qv[NG][8];
#pragma unroll
  for (int n = 0; n < NG; ++n) unpack_unit(qraw[n], qv[n]);
  // a wave reads only the rows it staged: a wave-level barrier suffices
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint4* mine = &s_rows[wid][lane * UPR];
  const int sw = swz(lane);
  float acc[G];
  // heads in fours
  static_assert(G % 4 == 0, "the products run four heads at a time");
  constexpr int GQ = G / 4;
  float acc4[GQ][4];
#pragma unroll
  for (int c = 0; c < GQ; ++c)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc4[c][j] = 0.0f;
  static_for<0, UPR>([&](auto uc) {
    constexpr int u = decltype(uc)::value;
    float kv[8];
    unpack_unit(mine[u ^ sw], kv);
    static_for<0, GQ>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      constexpr int j0 = 4 * c, j1 = j0 + 1, j2 = j0 + 2, j3 = j0 + 3;
      constexpr int F0 = j0 * UPR + u, F1 = j1 * UPR + u, F2 = j2 * UPR + u, F3 = j3 * UPR + u;
      fmac8x4_row_bcast<F0 % 16, F1 % 16, F2 % 16, F3 % 16>(acc4[c], qv[F0 / 16], qv[F1 / 16], qv[F2 / 16],
                                                           qv[F3 / 16], kv);
    });
  });
#pragma unroll
  for (int j = 0; j < G; ++j) acc[j] = acc4[j / 4][j % 4];
  const float s = ok ? group_score<G>(a, b, g, acc) : -__builtin_inff();
  if (in_row) row[t] = s;
  if (a.row_stats) note_minmax(a.row_stats + (int64_t)blockIdx.y * kStatStride, s, ok && __builtin_isfinite(s));
}

// ------------------------------------------------------------------ fast DSA

// u = 2^-24 for the round-to-nearest VALU arithmetic; the matrix-core sums
// are charged 2^-23 per addition, which also covers truncating adders.
__device__ __forceinline__ float gamma_n(float n, float u) { return n * u / (1.0f - n * u); }

typedef __attribute__((address_space(3))) void* lds_ptr;

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

constexpr int kTileTok = 32;                // tokens per wave per step
constexpr int kTileBytes = kTileTok * 256;  // their bf16 K rows (D = 128)

// relu on the bit pattern: negative floats (and -0) are negative integers.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// Sum over the 16 lanes of a DPP row (the 16 rows of one MFMA column group).
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false));  // row_ror 4
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror 8
  return v;
}

// The K ring is filled by DMA (global_load_lds), which the compiler tracks
// as one LDS write per instruction in flight: an ordinary LDS load would make
// it drain every DMA before the read.  Fragment reads are therefore one asm
// block that waits for its own results (so no output register is live while
// its load is in flight).  Eight 16-byte reads: four k-steps of the two
// 16-token halves of a tile, the halves 4096 bytes apart.
template <int OFF>
__device__ __forceinline__ void ring_read8(u32x4 (&f)[8], const uint32_t (&addr)[4]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%12\n\t"
      "ds_read_b128 %1, %9 offset:%12\n\t"
      "ds_read_b128 %2, %10 offset:%12\n\t"
      "ds_read_b128 %3, %11 offset:%12\n\t"
      "ds_read_b128 %4, %8 offset:%13\n\t"
      "ds_read_b128 %5, %9 offset:%13\n\t"
      "ds_read_b128 %6, %10 offset:%13\n\t"
      "ds_read_b128 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]), "=&v"(f[6]),
        "=&v"(f[7])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "i"(OFF), "i"(OFF + 4096)
      : "memory");
}
// A score into the LDS staging row (same reason: no compiler-visible LDS access).
__device__ __forceinline__ void lds_store_f32(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "i"(N) : "memory");
}

// Fused-path bookkeeping of a fast-scorer block: its slot (min / max finite
// score keys, bound) and its share of the row's selection statistics,
// cleared (slot 7, the hint floor, to -inf).  Nothing else touches those
// statistics until the histogram pass, a later launch.
__device__ __forceinline__ void span_bookkeeping(const ScoreArgs& a, int nthreads, uint32_t kmin, uint32_t kmax,
                                                 float bound, bool leader) {
  int32_t* st = a.row_stats + (int64_t)blockIdx.y * kStatStride;
  const int nx = gridDim.x;
  const int per = (kStatStride + nx - 1) / nx;
  const int i0 = blockIdx.x * per, i1 = min(kStatStride, i0 + per);
  for (int i = i0 + threadIdx.x; i < i1; i += nthreads) st[i] = i == 7 ? (int32_t)0xFF800000u : 0;
  if (leader) {
    int32_t* sl = a.span_slots + ((int64_t)blockIdx.y * nx + blockIdx.x) * 4;
    sl[0] = (int32_t)kmin;
    sl[1] = (int32_t)kmax;
    sl[2] = __float_as_int(bound);
    sl[3] = 0;
  }
}

// End of a fast-scorer block: the block's min / max finite score keys and
// its bound (one atomic each, or the block's slot on the fused path), then
// the span's scores from the LDS staging row (every token below L lies in a
// scored tile; the rest is -inf).
template <int NW>
__device__ __forceinline__ void finish_span(const ScoreArgs& a, uint32_t (*s_red)[3], const float* s_out,
                                            float* row, int tb0, int tend, int L, float smin, float smax,
                                            float dmax) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t kmin = smin <= smax ? score_key(smin) : 0xFFFFFFFFu;
  uint32_t kmax = smin <= smax ? score_key(smax) : 0u;
  kmin = wave_min_u32(kmin);
  kmax = wave_max_u32(kmax);
  dmax = wave_max(dmax);
  if (lane == 0) {
    s_red[wid][0] = kmin;
    s_red[wid][1] = kmax;
    s_red[wid][2] = __float_as_uint(dmax);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t bmin = s_red[0][0], bmax = s_red[0][1];
    float bd = __uint_as_float(s_red[0][2]);
#pragma unroll
    for (int w = 1; w < NW; ++w) {
      bmin = min(bmin, s_red[w][0]);
      bmax = max(bmax, s_red[w][1]);
      bd = fmaxf(bd, __uint_as_float(s_red[w][2]));
    }
    // 1e-3 relative slack covers the rounding of the bound's own evaluation,
    // the absolute term any flushed subnormal.
    bd = bd * 1.001f + 1e-30f;
    if (!a.span_slots && a.row_stats && bmin <= bmax) {
      int32_t* stat = a.row_stats + (int64_t)blockIdx.y * kStatStride;
      atomicMin(reinterpret_cast<unsigned int*>(stat), bmin);
      atomicMax(reinterpret_cast<unsigned int*>(stat + 1), bmax);
    }
    if (a.row_bound) atomicMax(reinterpret_cast<unsigned int*>(a.row_bound + blockIdx.y), __float_as_uint(bd));
    s_red[0][0] = bmin;
    s_red[0][1] = bmax;
    s_red[0][2] = __float_as_uint(bd);
  }
  if (a.span_slots) {
    __syncthreads();
    span_bookkeeping(a, NW * 64, s_red[0][0], s_red[0][1], __uint_as_float(s_red[0][2]), threadIdx.x == 0);
  }
  for (int t = tb0 + threadIdx.x; t < tend; t += NW * 64) row[t] = t < L ? s_out[t - tb0] : -__builtin_inff();
}

// MT = query heads / 16, NW waves per block, S ring stages per wave.
//
// Each wave scores 32-token tiles; tile it of wave w starts at token
// tb0 + (it * NW + w) * 32.  A tile's K rows (32 x 256 bytes) reach the
// wave's LDS ring by DMA, eight 1 KB instructions of four whole rows each
// (64 lanes x 16 bytes, fully coalesced), S - 1 tiles ahead of the one being
// computed.  Within a row the 16-byte units are stored XOR-swizzled
// (position = unit ^ (row & 15)) so that the fragment reads below hit 16
// different bank groups.
//
// MFMA 16x16x32 bf16, C[16 heads x 16 tokens] per (M tile, token half),
// K = 128 in four 32-wide steps.  Operand layout: lane l holds A[row l%16]
// [8 k-values], B[8 k-values][col l%16], C[rows 4*(l/16)+r][col l%16].  The
// head dims a lane's 8 k-values stand for are free as long as A and B agree:
// k-step ks, lane group l/16 carries dims 32*ks + 8*(l/16) .. +8.
template <int MT, int NW, int S, int MAXIT>
__global__ __launch_bounds__(NW * 64) void score_dsa_kernel(ScoreArgs a, int iters) {
  constexpr int D = 128;
  constexpr int KS = D / 32;
  constexpr int G = 16 * MT;
  __shared__ __attribute__((aligned(1024))) uint4 s_ring[NW * S * kTileBytes / 16];
  __shared__ float s_out[NW * kTileTok * MAXIT];
  __shared__ uint32_t s_red[NW][3];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int b = blockIdx.y / a.num_kv_heads, g = blockIdx.y % a.num_kv_heads;
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int span = NW * kTileTok * iters;
  const int tb0 = blockIdx.x * span;
  float* row = a.scores + (int64_t)blockIdx.y * a.max_kv_len;
  const int tend = min(tb0 + span, a.max_kv_len);
  if (tb0 >= L) {  // nothing to score: fill -inf
    for (int t = tb0 + threadIdx.x; t < tend; t += NW * 64) row[t] = -__builtin_inff();
    if (a.span_slots) span_bookkeeping(a, NW * 64, 0xFFFFFFFFu, 0u, 0.0f, threadIdx.x == 0);
    return;
  }
  const int ps = a.page_size;
  const int p0 = tb0 / ps;
  // tiles of this wave that hold a token below L
  const int n_it = min(iters, max(0, (L - tb0 - wid * kTileTok + NW * kTileTok - 1) / (NW * kTileTok)));

  // page ids of the span's logical pages, lane i <- page p0 + i (-1: absent)
  // (loaded from a clamped slot, checked once the loads below are out)
  const int lp = p0 + lane;
  const int pg_raw = a.block_table[(int64_t)b * a.max_pages + min(lp, a.max_pages - 1)];
  // this wave's query fragments and weights
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.q_heads + g * G) * D;
  const float* wb = a.head_weights + (int64_t)b * a.q_heads + g * G;
  bf16x8 qf[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[mt][ks] = *reinterpret_cast<const bf16x8*>(qb + (16 * mt + col) * D + 32 * ks + 8 * grp);
  float wv[MT][4], wa[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = wb[16 * mt + 4 * grp + r];
    wa[mt] = fabsf(wb[16 * mt + col]);
  }

  // Every ordinary load completes before the first DMA: the compiler counts
  // DMA and ordinary loads as different kinds of memory event and, with both
  // outstanding, can only wait for zero.  These empty asm uses make it wait
  // here, once, for all of them.
  asm volatile("" : : "v"(pg_raw));
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : : "v"(qf[mt][ks]));
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" : : "v"(wv[mt][r]));
    asm volatile("" : : "v"(wa[mt]));
  }
  const int mypage = (lp < a.max_pages && lp * ps < L && pg_raw >= 0 && pg_raw < a.num_pages) ? pg_raw : -1;

  // DMA lane layout: lane (r = l/16, p = l%16) of chunk c' moves row 4c'+r,
  // 16-byte unit p ^ (4c'+r) of a 16-row half tile.
  const int64_t ts2 = a.token_stride * 2;
  uint32_t vofs[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) vofs[c] = (uint32_t)((4 * c + grp) * ts2 + 16 * (col ^ (4 * c + grp)));
  const char* kbase = reinterpret_cast<const char*>(a.k) + (int64_t)g * a.head_stride * 2;
  const uint32_t ring0 = (uint32_t)(uintptr_t)(lds_ptr)s_ring + (uint32_t)(wid * S * kTileBytes);
  auto tile_t0 = [&](int it) { return tb0 + (it * NW + wid) * kTileTok; };
  auto half_page = [&](int t) { return __builtin_amdgcn_readlane(mypage, min(t / ps - p0, 63)); };
  auto issue = [&](int it, int stage) {
    const int t0 = tile_t0(it);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = t0 + 16 * h;
      const int pg = max(half_page(t), 0);  // an absent page reads page 0 (masked)
      const char* hb = kbase + ((int64_t)pg * a.page_stride + (int64_t)(t % ps) * a.token_stride) * 2;
      const uint32_t dst = ring0 + (uint32_t)(stage * kTileBytes + h * 4096);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        __builtin_amdgcn_global_load_lds(hb + vofs[c], (lds_ptr)(uintptr_t)(dst + c * 1024), 16, 0, kLoadStream);
    }
  };
  // The first S - 1 tiles go out before the per-wave set-up below, whether
  // or not the wave has that many (a tile past L reads pages it holds, or
  // page 0, and is never used), so that the compiler sees straight-line
  // code and keeps its waits for the loads above exact.
  static_for<0, S - 1>([&](auto j) { issue(decltype(j)::value, decltype(j)::value); });

  // a_d = sum_h |w_h| |q_hd| for the bound: this lane's 4*MT heads per dim,
  // then the 16 lanes of each column group.  The bound's sum_d a_d |k_d|
  // runs on the matrix cores as one more M tile whose row 0 holds a_d
  // rounded up to bf16 (an upper bound of a_d) and whose B operand is |K|.
  bf16x8 af[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    float part[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) part[j] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 w4 = __builtin_bit_cast(u32x4, qf[mt][ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part[2 * e] += wa[mt] * fabsf(bf16_lo(w4[e]));
        part[2 * e + 1] += wa[mt] * fabsf(bf16_hi(w4[e]));
      }
    }
    u32x4 p4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = row16_sum(part[2 * e]), hi = row16_sum(part[2 * e + 1]);
      p4[e] = col == 0 ? (bf16_round_up(lo) | (bf16_round_up(hi) << 16)) : 0u;
    }
    af[ks] = __builtin_bit_cast(bf16x8, p4);
  }
  const float u24 = 5.9604644775390625e-8f, u23 = 1.1920928955078125e-7f;
  const float gD = gamma_n((float)D, u23), gH = gamma_n((float)(G + 1), u24);
  const float bcoef = 2.0f * gH * (1.0f + gD) + 2.0f * gD;
  float dmax = 0.0f;
  float smin = __builtin_inff(), smax = -__builtin_inff();  // finite scores of this lane

  // fragment read addresses: token row col, unit 4*ks + grp (swizzled)
  uint32_t raddr[4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) raddr[ks] = ring0 + col * 256 + 16 * ((4 * ks + grp) ^ col);
  const uint32_t out0 = (uint32_t)(uintptr_t)(lds_ptr)s_out;

  auto compute = [&](int it, auto sc) {
    constexpr int s = decltype(sc)::value;
    u32x4 kb[8];
    ring_read8<s * kTileBytes>(kb, raddr);
    const int t0 = tile_t0(it);
    float sv[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      floatx4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[mt][ks], __builtin_bit_cast(bf16x8, kb[4 * n + ks]),
                                                            acc[mt], 0, 0, 0);
      }
      floatx4 accb = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        accb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[ks], __builtin_bit_cast(bf16x8, kb[4 * n + ks] & 0x7FFF7FFFu),
                                                       accb, 0, 0, 0);
      // s~ = sum_h w_h relu(dot_h): this lane's 4*MT heads, then the 4 lane groups
      float sum = 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sum = __builtin_fmaf(wv[mt][r], relu_bits(acc[mt][r]), sum);
      sum = rows4_sum(sum);
      const int t = t0 + 16 * n + col;
      const bool ok = t < L && half_page(t0 + 16 * n) >= 0;
      if (ok) {
        // B_t = sum_d a_d |k_td| (row 0 of the extra tile, lanes 0..15) bounds both
        // sum_h |w_h| relu(.) terms, so |s~ - s| <= B_t * (2 gH (1 + gD) + 2 gD)
        if (grp == 0) dmax = fmaxf(dmax, accb[0] * bcoef);
        smin = fminf(smin, sum);
        smax = fmaxf(smax, sum);
      }
      sv[n] = ok ? sum : -__builtin_inff();
    }
    // lanes 0..15 hold tokens t0 + col, lanes 16..31 the second half's
    if (lane < 32) lds_store_f32(out0 + 4 * (t0 - tb0 + lane), lane < 16 ? sv[0] : sv[1]);
  };

  for (int it0 = 0; it0 < n_it; it0 += S) {
    static_for<0, S>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const int it = it0 + s;
      if (it < n_it) {
        const int ahead = min(n_it - 1 - it, S - 1);  // tiles in flight after tile it
        if (ahead == S - 1) {
          issue(it + S - 1, (s + S - 1) % S);
          wait_vmcnt<8 * (S - 1)>();
        } else {
          static_for<0, S - 1>([&](auto j) {
            if (ahead == decltype(j)::value) wait_vmcnt<8 * decltype(j)::value>();
          });
        }
        compute(it, sc);
      }
    });
  }
  // no DMA may still be writing the ring when the wave leaves (a wave with
  // fewer than S - 1 tiles has prologue tiles in flight), and the staged
  // scores are written
  wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  finish_span<NW>(a, s_red, s_out, row, tb0, tend, L, smin, smax, dmax);
}

// ------------------------------------------------------------------ fast DSA, fp8 K

// The same score over an FP8 E4M3 indexer cache with one binary32 scale per
// row ("Overlap DSA heuristic prev_topk write-back on the aux stream", Test
// Coverage: the block-scaled FP8 indexer cache).  Each code widens exactly to
// bf16 (3 mantissa bits, exponents 2^-9 .. 2^8), so the matrix cores form
// t~_h = sum_d q_hd code_d, and the head's dot product is sigma_t * t~_h.
constexpr int kTileBytes8 = kTileTok * 128;      // a tile's fp8 K rows (D = 128)
constexpr int kStageBytes8 = kTileBytes8 + 256;  // + its 32 row scales (one 256-byte DMA)

// Eight E4M3 codes (two words) -> bf16, exact.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A tile's fragment reads as one asm block (see ring_read8): two 16-byte
// units (64 head dims each) of each 16-token half, the halves 2048 bytes
// apart, and the scales of this lane's two tokens.
template <int OFF>
__device__ __forceinline__ void ring_read_fp8(u32x4 (&f)[4], float (&sc)[2], const uint32_t (&addr)[2],
                                              uint32_t saddr) {
  asm volatile(
      "ds_read_b128 %0, %6 offset:%8\n\t"
      "ds_read_b128 %1, %7 offset:%8\n\t"
      "ds_read_b128 %2, %6 offset:%9\n\t"
      "ds_read_b128 %3, %7 offset:%9\n\t"
      "ds_read_b32 %4, %10 offset:%11\n\t"
      "ds_read_b32 %5, %10 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(sc[0]), "=&v"(sc[1])
      : "v"(addr[0]), "v"(addr[1]), "i"(OFF), "i"(OFF + 2048), "v"(saddr), "i"(OFF + kTileBytes8),
        "i"(OFF + kTileBytes8 + 64)
      : "memory");
}

// Tiles, waves and the MFMA layout as in score_dsa_kernel; what differs:
//  * a tile is 32 x 128 bytes, four 1 KB DMA instructions of eight rows
//    each, plus one 4-byte-per-lane DMA of the 32 row scales (lanes 32..63
//    repeat lanes 0..31);
//  * 16-byte units are swizzled as unit ^ ((row >> 1) & 7): two 128-byte rows
//    share one 256-byte bank line, and 16 rows read at one unit then hit 16
//    different bank groups;
//  * the 8 k-values of lane group l/16 at k-step ks are head dims
//    64 (ks/2) + 16 (l/16) + 8 (ks%2) .. +8, so one 16-byte read serves two
//    k-steps;
//  * the scale is applied once per token: for sigma >= 0,
//    sum_h w_h relu(sigma t~_h) = sigma sum_h w_h relu(t~_h) (a tile with a
//    negative scale takes the per-head form).
// Error bound: the exact score dequantizes (one rounding), rounds every
// product and every sum, so each head's dot differs from sigma sum_d q_d c_d
// by at most gamma_{D+1} |sigma| sum_d |q_d c_d|; the matrix-core value
// sigma t~ by at most gamma_D times the same (its final scaling counts with
// the head sum's roundings).  Both are below gamma_{D+2} (unit 2^-23), so the
// bf16 form holds with B_t = |sigma_t| sum_d a_d |c_td|.  B_t comes from one
// fp8 MFMA per 16 tokens: a_d scaled by a power of two and rounded up to
// E4M3 against the codes' magnitudes (products of two E4M3 values are exact
// in binary32).
template <int MT, int NW, int S, int MAXIT>
__global__ __launch_bounds__(NW * 64) void score_dsa_fp8_kernel(ScoreArgs a, int iters) {
  constexpr int D = 128;
  constexpr int KS = D / 32;
  constexpr int G = 16 * MT;
  __shared__ __attribute__((aligned(1024))) uint4 s_ring[NW * S * kStageBytes8 / 16];
  __shared__ float s_out[NW * kTileTok * MAXIT];
  __shared__ uint32_t s_red[NW][3];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int b = blockIdx.y / a.num_kv_heads, g = blockIdx.y % a.num_kv_heads;
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int span = NW * kTileTok * iters;
  const int tb0 = blockIdx.x * span;
  float* row = a.scores + (int64_t)blockIdx.y * a.max_kv_len;
  const int tend = min(tb0 + span, a.max_kv_len);
  if (tb0 >= L) {
    for (int t = tb0 + threadIdx.x; t < tend; t += NW * 64) row[t] = -__builtin_inff();
    if (a.span_slots) span_bookkeeping(a, NW * 64, 0xFFFFFFFFu, 0u, 0.0f, threadIdx.x == 0);
    return;
  }
  const int ps = a.page_size;
  const int p0 = tb0 / ps;
  const int n_it = min(iters, max(0, (L - tb0 - wid * kTileTok + NW * kTileTok - 1) / (NW * kTileTok)));

  const int lp = p0 + lane;
  const int pg_raw = a.block_table[(int64_t)b * a.max_pages + min(lp, a.max_pages - 1)];
  const uint16_t* qb = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.q_heads + g * G) * D;
  const float* wb = a.head_weights + (int64_t)b * a.q_heads + g * G;
  bf16x8 qf[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[mt][ks] = *reinterpret_cast<const bf16x8*>(qb + (16 * mt + col) * D + 64 * (ks >> 1) + 16 * grp +
                                                    8 * (ks & 1));
  float wv[MT][4], wa[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = wb[16 * mt + 4 * grp + r];
    wa[mt] = fabsf(wb[16 * mt + col]);
  }
  // ordinary loads complete before the first DMA (see score_dsa_kernel)
  asm volatile("" : : "v"(pg_raw));
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : : "v"(qf[mt][ks]));
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" : : "v"(wv[mt][r]));
    asm volatile("" : : "v"(wa[mt]));
  }
  const int mypage = (lp < a.max_pages && lp * ps < L && pg_raw >= 0 && pg_raw < a.num_pages) ? pg_raw : -1;

  // K DMA lane layout: chunk c of a 16-token half moves rows 8c + l/8, unit
  // (l%8) ^ swz(row); the scale DMA gives lane l the scale of token l%16 of
  // half (l/16)%2.
  const int64_t ts = a.token_stride;  // fp8: elements are bytes
  uint32_t vofs[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = 8 * c + (lane >> 3);
    vofs[c] = (uint32_t)(r * ts + 16 * ((lane & 7) ^ ((r >> 1) & 7)));
  }
  const int shalf = (lane >> 4) & 1;
  const char* kbase = reinterpret_cast<const char*>(a.k) + (int64_t)g * a.head_stride;
  const uint32_t ring0 = (uint32_t)(uintptr_t)(lds_ptr)s_ring + (uint32_t)(wid * S * kStageBytes8);
  auto tile_t0 = [&](int it) { return tb0 + (it * NW + wid) * kTileTok; };
  auto half_page = [&](int t) { return __builtin_amdgcn_readlane(mypage, min(t / ps - p0, 63)); };
  auto issue = [&](int it, int stage) {
    const int t0 = tile_t0(it);
    const uint32_t dst = ring0 + (uint32_t)(stage * kStageBytes8);
    int pgh[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = t0 + 16 * h;
      pgh[h] = max(half_page(t), 0);  // an absent page reads page 0 (masked)
      const char* hb = kbase + (int64_t)pgh[h] * a.page_stride + (int64_t)(t % ps) * ts;
#pragma unroll
      for (int c = 0; c < 2; ++c)
        __builtin_amdgcn_global_load_lds(hb + vofs[c], (lds_ptr)(uintptr_t)(dst + h * 2048 + c * 1024), 16, 0,
                                         kLoadStream);
    }
    const int spg = shalf ? pgh[1] : pgh[0];
    const float* sp = a.k_scale + fp8_scale_index(spg, g, (t0 + 16 * shalf) % ps + col, a.num_kv_heads, ps);
    __builtin_amdgcn_global_load_lds(sp, (lds_ptr)(uintptr_t)(dst + kTileBytes8), 4, 0, kLoadStream);
  };
  static_for<0, S - 1>([&](auto j) { issue(decltype(j)::value, decltype(j)::value); });

  // a_d = sum_h |w_h| |q_hd| for the bound, on this lane's 32 dims (those of
  // its B fragment: k-steps 0..3 = dims 16 grp + [0, 16), 64 + 16 grp +
  // [0, 16)), summed over its MT heads and then the 16 lanes of its column
  // group.  Row 0 of the bound tile (lanes with col 0) holds a_d * 2^-e
  // rounded up to E4M3, with 2^e a power of two that keeps max_d a_d * 2^-e
  // in [128, 256); the other rows are zero.
  float ad[KS][8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
    for (int j = 0; j < 8; ++j) ad[ks][j] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x4 w4 = __builtin_bit_cast(u32x4, qf[mt][ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ad[ks][2 * e] += wa[mt] * fabsf(bf16_lo(w4[e]));
        ad[ks][2 * e + 1] += wa[mt] * fabsf(bf16_hi(w4[e]));
      }
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ad[ks][j] = row16_sum(ad[ks][j]);
      amax = fmaxf(amax, ad[ks][j]);
    }
  amax = wave_max(amax);
  // 2^-e with max_d a_d * 2^-e in [128, 256) (e = 0 for an all-zero tile)
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  const int e2 = amax > 0.0f ? ebits - 127 - 7 : 0;
  const float down = __uint_as_float((uint32_t)(127 - e2) << 23), up = __uint_as_float((uint32_t)(127 + e2) << 23);
  intx8 af8;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) word |= fp8_round_up(ad[2 * (w >> 2) + ((w >> 1) & 1)][4 * (w & 1) + j] * down) << (8 * j);
    af8[w] = col == 0 ? (int)word : 0;
  }
  const float u24 = 5.9604644775390625e-8f, u23 = 1.1920928955078125e-7f;
  const float gD = gamma_n((float)(D + 2), u23), gH = gamma_n((float)(G + 1), u24);
  const float bcoef = (2.0f * gH * (1.0f + gD) + 2.0f * gD) * up;
  float dmax = 0.0f;
  float smin = __builtin_inff(), smax = -__builtin_inff();

  uint32_t raddr[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) raddr[j] = ring0 + col * 128 + 16 * ((4 * j + grp) ^ ((col >> 1) & 7));
  const uint32_t saddr = ring0 + 4 * col;
  const uint32_t out0 = (uint32_t)(uintptr_t)(lds_ptr)s_out;

  auto compute = [&](int it, auto sc) {
    constexpr int s = decltype(sc)::value;
    u32x4 kr[4];
    float sig[2];
    ring_read_fp8<s * kStageBytes8>(kr, sig, raddr, saddr);
    const int t0 = tile_t0(it);
    // one uniform test per tile: any negative scale (sign bit) among its tokens
    const bool neg = __builtin_amdgcn_ballot_w64((__float_as_uint(sig[0]) | __float_as_uint(sig[1])) >> 31) != 0;
    float sv[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      bf16x8 kb[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 w = kr[2 * n + (ks >> 1)];
        kb[ks] = fp8x8_to_bf16(w[2 * (ks & 1)], w[2 * (ks & 1) + 1]);
      }
      floatx4 acc[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acc[mt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[mt][ks], kb[ks], acc[mt], 0, 0, 0);
      }
      // the bound tile: sum_d (a_d 2^-e)^ |c_d| on the fp8 matrix cores, |c| by
      // clearing the code sign bits (E4M3 A and B, unit block scales)
      const u32x4 c0 = kr[2 * n], c1 = kr[2 * n + 1];
      const intx8 cabs = intx8{(int)(c0[0] & 0x7F7F7F7Fu), (int)(c0[1] & 0x7F7F7F7Fu), (int)(c0[2] & 0x7F7F7F7Fu),
                               (int)(c0[3] & 0x7F7F7F7Fu), (int)(c1[0] & 0x7F7F7F7Fu), (int)(c1[1] & 0x7F7F7F7Fu),
                               (int)(c1[2] & 0x7F7F7F7Fu), (int)(c1[3] & 0x7F7F7F7Fu)};
      const floatx4 accb = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
          af8, cabs, floatx4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0, 127, 0, 127);
      float sum = 0.0f;
      if (!neg) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sum = __builtin_fmaf(wv[mt][r], relu_bits(acc[mt][r]), sum);
        sum = rows4_sum(sum);
        sum = __fmul_rn(sig[n], sum);
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sum = __builtin_fmaf(wv[mt][r], relu_bits(__fmul_rn(sig[n], acc[mt][r])), sum);
        sum = rows4_sum(sum);
      }
      const int t = t0 + 16 * n + col;
      const bool ok = t < L && half_page(t0 + 16 * n) >= 0;
      // selects, not a branch: the bound MFMA stays in straight-line code
      const float bt = fabsf(sig[n]) * accb[0];
      dmax = (ok && grp == 0) ? fmaxf(dmax, bt) : dmax;
      smin = ok ? fminf(smin, sum) : smin;
      smax = ok ? fmaxf(smax, sum) : smax;
      sv[n] = ok ? sum : -__builtin_inff();
    }
    if (lane < 32) lds_store_f32(out0 + 4 * (t0 - tb0 + lane), lane < 16 ? sv[0] : sv[1]);
  };

  constexpr int kPerTile = 5;  // DMA instructions per tile
  for (int it0 = 0; it0 < n_it; it0 += S) {
    static_for<0, S>([&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const int it = it0 + s;
      if (it < n_it) {
        const int ahead = min(n_it - 1 - it, S - 1);
        if (ahead == S - 1) {
          issue(it + S - 1, (s + S - 1) % S);
          wait_vmcnt<kPerTile * (S - 1)>();
        } else {
          static_for<0, S - 1>([&](auto j) {
            if (ahead == decltype(j)::value) wait_vmcnt<kPerTile * decltype(j)::value>();
          });
        }
        compute(it, sc);
      }
    });
  }
  wait_vmcnt<0>();
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  finish_span<NW>(a, s_red, s_out, row, tb0, tend, L, smin, smax, dmax * bcoef);
}

// ------------------------------------------------------------------ launch

template <typename KT, int UPR>
static hipError_t launch_exact_g(const ScoreArgs& a, dim3 grid, hipStream_t st) {
  switch (a.q_heads / a.num_kv_heads) {
    case 1: score_exact_staged_kernel<KT, 1, UPR><<<grid, 256, 0, st>>>(a); break;
    case 2: score_exact_staged_kernel<KT, 2, UPR><<<grid, 256, 0, st>>>(a); break;
    case 4: score_exact_staged_kernel<KT, 4, UPR><<<grid, 256, 0, st>>>(a); break;
    case 8: score_exact_staged_kernel<KT, 8, UPR><<<grid, 256, 0, st>>>(a); break;
    case 16: score_exact_staged_kernel<KT, 16, UPR><<<grid, 256, 0, st>>>(a); break;
    case 32: score_exact_staged_kernel<KT, 32, UPR><<<grid, 256, 0, st>>>(a); break;
    case 64: score_exact_staged_kernel<KT, 64, UPR><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename KT>
static hipError_t launch_exact_t(const ScoreArgs& a, hipStream_t st) {
  const int G = a.q_heads / a.num_kv_heads;
  dim3 grid((a.max_kv_len + 255) / 256, a.batch * a.num_kv_heads);
  // rows of 128 or 256 bytes starting on 16-byte boundaries are staged through LDS
  const int64_t es = (int64_t)sizeof(KT), rbytes = (int64_t)a.head_dim * es;
  const bool aligned = (reinterpret_cast<uintptr_t>(a.k) & 15) == 0 && (a.token_stride * es) % 16 == 0 &&
                       (a.page_stride * es) % 16 == 0 && (a.head_stride * es) % 16 == 0;
  if constexpr (std::is_same<KT, uint16_t>::value) {
    static const bool bcast = [] {
      const char* e = getenv("SD_EXACT_BCAST");
      return !(e && e[0] == '0');
    }();
    if (bcast && aligned && a.num_pages > 0 && (rbytes == 256 || rbytes == 128)) {
      hipError_t e = hipErrorInvalidValue;
      if (rbytes == 256) {
        switch (G) {
          case 4: score_exact_bcast_kernel<4, 16><<<grid, 256, 0, st>>>(a); e = hipSuccess; break;
          case 8: score_exact_bcast_kernel<8, 16><<<grid, 256, 0, st>>>(a); e = hipSuccess; break;
          default: break;
        }
      } else {
        switch (G) {
          case 4: score_exact_bcast_kernel<4, 8><<<grid, 256, 0, st>>>(a); e = hipSuccess; break;
          case 8: score_exact_bcast_kernel<8, 8><<<grid, 256, 0, st>>>(a); e = hipSuccess; break;
          case 16: score_exact_bcast_kernel<16, 8><<<grid, 256, 0, st>>>(a); e = hipSuccess; break;
          default: break;
        }
      }
      if (e == hipSuccess) return hipGetLastError();
    }
  }
  if (aligned && a.num_pages > 0 && rbytes == 256) return launch_exact_g<KT, 16>(a, grid, st);
  if (aligned && a.num_pages > 0 && rbytes == 128) return launch_exact_g<KT, 8>(a, grid, st);
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
  if (a.dtype == 0) return launch_exact_t<float>(a, st);
  if (a.dtype == 1) return launch_exact_t<uint16_t>(a, st);
  return launch_exact_t<uint8_t>(a, st);
}

bool score_fast_supported(const ScoreArgs& a) {
  const int G = a.q_heads / a.num_kv_heads;
  const int es = a.dtype == 1 ? 2 : 1;  // bytes per K element (bf16, fp8)
  return (a.dtype == 1 || (a.dtype == 2 && a.k_scale)) && a.mode == 2 && a.head_dim == 128 &&
         (G == 16 || G == 32 || G == 64) && (a.page_size % 16) == 0 && (a.token_stride * es) % 16 == 0 &&
         (a.page_stride * es) % 16 == 0 && (a.head_stride * es) % 16 == 0;
}

namespace {
// waves per block, ring stages, tiles per wave at most, blocks per CU
constexpr int kScoreNW = 4, kScoreStages = 4, kScoreMaxIt = 32, kScoreBlocksPerCU = 1;      // bf16 K
// bf16 K when the grid needs several rounds of blocks: two smaller blocks per
// CU, so that one block's start and drain overlap the other's stream, and
// shorter spans (rows of different lengths balance better)
constexpr int kScoreMNW = 4, kScoreMStages = 2, kScoreMMaxIt = 16, kScoreMBlocksPerCU = 2;
constexpr int kScore8NW = 8, kScore8Stages = 3, kScore8MaxIt = 16, kScore8BlocksPerCU = 1;  // fp8 K

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

// Tiles per wave: enough blocks to fill the chip once, and a span that
// overlaps at most 64 logical pages (their ids ride in one register per
// lane): span / page_size pages when the span is a whole number of pages,
// else up to two more.
int score_iters(const ScoreArgs& a, int nw, int maxit, int bpc) {
  const int cus = device_cus();
  const int64_t rows = (int64_t)a.batch * a.num_kv_heads;
  const int64_t tiles = rows * ((a.max_kv_len + kTileTok - 1) / kTileTok);
  const int64_t per_block = (tiles + (int64_t)cus * bpc - 1) / ((int64_t)cus * bpc);
  int iters = (int)std::min<int64_t>((per_block + nw - 1) / nw, maxit);
  auto pages_spanned = [&](int it) {
    const int span = nw * kTileTok * it;
    return span % a.page_size == 0 ? span / a.page_size : (span - 1) / a.page_size + 2;
  };
  while (iters > 1 && pages_spanned(iters) > 64) --iters;
  return std::max(iters, 1);
}

// Launch shape of the fast scorer: 0 = one round of large bf16 blocks,
// 1 = several rounds (two blocks per CU), 2 = fp8.
struct FastShape {
  int kind, nw, iters;
};
FastShape fast_shape(const ScoreArgs& a) {
  if (a.dtype == 2) return {2, kScore8NW, score_iters(a, kScore8NW, kScore8MaxIt, kScore8BlocksPerCU)};
  const int64_t rows = (int64_t)a.batch * a.num_kv_heads;
  const int64_t tiles = rows * ((a.max_kv_len + kTileTok - 1) / kTileTok);
  if (tiles <= (int64_t)device_cus() * kScoreBlocksPerCU * kScoreNW * kScoreMaxIt)
    return {0, kScoreNW, score_iters(a, kScoreNW, kScoreMaxIt, kScoreBlocksPerCU)};
  return {1, kScoreMNW, score_iters(a, kScoreMNW, kScoreMMaxIt, kScoreMBlocksPerCU)};
}

}  // namespace

int score_fast_spans(const ScoreArgs& a) {
  const FastShape f = fast_shape(a);
  const int span = f.nw * kTileTok * f.iters;
  return (a.max_kv_len + span - 1) / span;
}

int score_fast_max_spans(int max_kv_len) {  // one tile per wave, the smallest block
  const int span = std::min(std::min(kScoreNW, kScoreMNW), kScore8NW) * kTileTok;
  return (max_kv_len + span - 1) / span;
}

namespace {
template <int MT>
hipError_t launch_dsa(const ScoreArgs& a, hipStream_t st) {
  const FastShape f = fast_shape(a);
  const unsigned rows = (unsigned)(a.batch * a.num_kv_heads);
  const int span = f.nw * kTileTok * f.iters;
  const dim3 grid((a.max_kv_len + span - 1) / span, rows);
  if (f.kind == 2)
    score_dsa_fp8_kernel<MT, kScore8NW, kScore8Stages, kScore8MaxIt><<<grid, kScore8NW * 64, 0, st>>>(a, f.iters);
  else if (f.kind == 1)
    score_dsa_kernel<MT, kScoreMNW, kScoreMStages, kScoreMMaxIt><<<grid, kScoreMNW * 64, 0, st>>>(a, f.iters);
  else
    score_dsa_kernel<MT, kScoreNW, kScoreStages, kScoreMaxIt><<<grid, kScoreNW * 64, 0, st>>>(a, f.iters);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_score_fast(const ScoreArgs& a, hipStream_t st) {
  if (a.batch == 0 || a.max_kv_len == 0) return hipSuccess;
  switch (a.q_heads / a.num_kv_heads / 16) {
    case 1: return launch_dsa<1>(a, st);
    case 2: return launch_dsa<2>(a, st);
    case 4: return launch_dsa<4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sd
