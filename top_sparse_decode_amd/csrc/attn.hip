// attn.hip -- gather of the selected K/V rows through the block table and
// split-K online-softmax attention over them, then a combine pass.
//
// Selected-token attention as in "Add DSA Vanilla sparse attention"
// (Walkthrough: selected-token attention over request-local selections, MLA
// latent rows read from the paged cache), consuming the predicted indices as
// "Unify sparse attention framework with clean backend interfaces"
// (Description) describes.  Index -> pool slot goes through the block table
// with the invalidation rules of its Dev Engineer Review (negative position,
// page outside the pool).
//
// Partials live in the log2 domain: x = (scale*log2 e) * q.k, a split keeps
// (m = max x, l = sum 2^(x-m), o = sum 2^(x-m) v); combine merges the splits.
#include "common.h"
#include "kernels.h"

namespace sd {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int kPer = 4;
  __device__ static void unpack(const uint4& u, float (&v)[4]) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
};
template <>
struct Vec<uint16_t> {
  static constexpr int kPer = 8;
  __device__ static void unpack(const uint4& u, float (&v)[8]) {
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
  }
};

// Sum of x over each aligned group of N lanes (N = 8, 16 or 32), in every
// lane of the group.  Groups of 16 use DPP rotations within a 16-lane row
// (VALU operands, no LDS permutes); other sizes use lane shuffles.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N == 16) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x124, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x122, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x121, 0xF, 0xF, false));
  } else {
#pragma unroll
    for (int off = N / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
  }
  return x;
}

__device__ __forceinline__ void merge_ml(float& m, float& l, float mo, float lo, float& a_self, float& a_other) {
  const float M = fmaxf(m, mo);
  if (M == -__builtin_inff()) {
    a_self = 0.0f;
    a_other = 0.0f;
    return;
  }
  a_self = exp2f(m - M);
  a_other = exp2f(mo - M);
  l = l * a_self + lo * a_other;
  m = M;
}

// Returns the element offset of token t's row, or -1 if t is not usable.
__device__ __forceinline__ int64_t sel_row(const AttnArgs& a, const int32_t* bt, int L, int t,
                                           int g, int64_t page_stride, int64_t head_stride,
                                           int64_t token_stride, int num_pages) {
  if (t < 0 || t >= L) return -1;
  const int page = bt[t / a.page_size];
  if (page < 0 || page >= num_pages) return -1;
  return (int64_t)page * page_stride + (int64_t)g * head_stride + (int64_t)(t % a.page_size) * token_stride;
}

// ------------------------------------------------------------------ vector path

// One block per (split, request*KV head); four waves.  A row of D elements is
// spread over LPR lanes (16 bytes each), so a wave works on 64/LPR rows at
// a time (RPW row slots), each slot with its own running (m, l, o); slots
// and waves are merged at the end.
template <typename T, int D, int G>
__global__ __launch_bounds__(256) void attn_vec_kernel(AttnArgs a) {
  constexpr int EPL = Vec<T>::kPer;
  constexpr int LPR = D / EPL;
  constexpr int RPW = kWave / LPR;
  __shared__ float s_ml[4][G][2];
  __shared__ float s_o[4][G][D];

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int sub = lane % LPR, slot = lane / LPR;
  const int b = blockIdx.y / a.num_kv_heads, g = blockIdx.y % a.num_kv_heads;
  const int split = blockIdx.x;
  const int r0 = split * a.chunk, r1 = min(a.k_sel, r0 + a.chunk);
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int32_t* sel = a.indices + ((int64_t)b * a.num_kv_heads + g) * a.k_sel;
  const float c = a.scale * kLog2e;

  float qf[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    const T* qp = reinterpret_cast<const T*>(a.q) + ((int64_t)b * a.q_heads + g * G + j) * D + sub * EPL;
    Vec<T>::unpack(*reinterpret_cast<const uint4*>(qp), qf[j]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[j][e] *= c;
  }
  float m[G], l[G], o[G][EPL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    m[j] = -__builtin_inff();
    l[j] = 0.0f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[j][e] = 0.0f;
  }
  const T* kb = reinterpret_cast<const T*>(a.k);
  const T* vb = reinterpret_cast<const T*>(a.v);
  // Batches of 64 selected rows per wave, four batches resolved at once:
  // lane l looks up row base + l of each (position, then its page: two
  // rounds of independent loads for 256 rows), then the rows go through the
  // wave RPW at a time with kPF groups' K and V loads in flight together.
  // Rows that are not usable load the pool's first row instead (branch-free)
  // and are skipped.
  constexpr int kPF = LPR < 8 ? LPR : 8;
  constexpr int kSB = 4;
  // (an empty pool has no first row: nothing is usable then)
  const int r_end = a.k_num_pages > 0 && a.v_num_pages > 0 ? r1 : r0;
  for (int sbase = r0 + wid * kWave * kSB; sbase < r_end; sbase += 4 * kWave * kSB) {
    int tsel[kSB], pg[kSB];
#pragma unroll
    for (int bi = 0; bi < kSB; ++bi) {
      const int row = sbase + bi * kWave + lane;
      tsel[bi] = row < r1 ? sel[row] : -1;
    }
#pragma unroll
    for (int bi = 0; bi < kSB; ++bi) {
      const bool in = tsel[bi] >= 0 && tsel[bi] < L;
      const int p = bt[in ? tsel[bi] / a.page_size : 0];
      pg[bi] = in ? p : -1;
    }
    uint32_t k_lo[kSB], k_hi[kSB], v_lo[kSB], v_hi[kSB];
#pragma unroll
    for (int bi = 0; bi < kSB; ++bi) {
      const int t = tsel[bi], p = pg[bi];
      const bool ok = p >= 0 && p < a.k_num_pages && p < a.v_num_pages;
      const int slot_t = ok ? t % a.page_size : 0;
      const int64_t ko = ok ? (int64_t)p * a.k_page_stride + (int64_t)g * a.k_head_stride + (int64_t)slot_t * a.k_token_stride : -1;
      const int64_t vo = ok ? (int64_t)p * a.v_page_stride + (int64_t)g * a.v_head_stride + (int64_t)slot_t * a.v_token_stride : -1;
      k_lo[bi] = (uint32_t)(uint64_t)ko;
      k_hi[bi] = (uint32_t)((uint64_t)ko >> 32);
      v_lo[bi] = (uint32_t)(uint64_t)vo;
      v_hi[bi] = (uint32_t)((uint64_t)vo >> 32);
    }
#pragma unroll
    for (int bi = 0; bi < kSB; ++bi) {
      const int base = sbase + bi * kWave;
      if (base >= r1) break;
      const int ngrp = min(LPR, (r1 - base + RPW - 1) / RPW);  // groups holding a row below r1
      for (int q0 = 0; q0 < ngrp; q0 += kPF) {
        uint4 kbuf[kPF], vbuf[kPF];
        bool okb[kPF];
#pragma unroll
        for (int q = 0; q < kPF; ++q) {
          const int src = ((q0 + q) * RPW + slot) & 63;  // the lane that resolved this row
          const int64_t k_o = (int64_t)(((uint64_t)(uint32_t)__shfl((int)k_hi[bi], src) << 32) | (uint32_t)__shfl((int)k_lo[bi], src));
          const int64_t v_o = (int64_t)(((uint64_t)(uint32_t)__shfl((int)v_hi[bi], src) << 32) | (uint32_t)__shfl((int)v_lo[bi], src));
          okb[q] = q0 + q < ngrp && k_o >= 0;
          kbuf[q] = *reinterpret_cast<const uint4*>(kb + (okb[q] ? k_o : 0) + sub * EPL);
          vbuf[q] = *reinterpret_cast<const uint4*>(vb + (okb[q] ? v_o : 0) + sub * EPL);
        }
        // the group's logits first, then one rescale per head for the kPF
        // rows (against their joint maximum) and their weighted V rows
        float x[kPF][G];
#pragma unroll
        for (int q = 0; q < kPF; ++q) {
          float kv[EPL];
          Vec<T>::unpack(kbuf[q], kv);
#pragma unroll
          for (int j = 0; j < G; ++j) {
            float d = 0.0f;
#pragma unroll
            for (int e = 0; e < EPL; ++e) d = __builtin_fmaf(qf[j][e], kv[e], d);
            x[q][j] = group_sum<LPR>(d);
          }
        }
        float mn[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
          mn[j] = m[j];
#pragma unroll
          for (int q = 0; q < kPF; ++q)
            if (okb[q]) mn[j] = fmaxf(mn[j], x[q][j]);
          // no usable row yet: nothing to rescale or add
          if (mn[j] != -__builtin_inff()) {
            const float al = exp2f(m[j] - mn[j]);  // 0 while m is -inf
            l[j] *= al;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[j][e] *= al;
            m[j] = mn[j];
          }
        }
#pragma unroll
        for (int q = 0; q < kPF; ++q) {
          if (!okb[q]) continue;
          float vv[EPL];
          Vec<T>::unpack(vbuf[q], vv);
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const float p = exp2f(x[q][j] - mn[j]);
            l[j] += p;
#pragma unroll
            for (int e = 0; e < EPL; ++e) o[j][e] = __builtin_fmaf(p, vv[e], o[j][e]);
          }
        }
      }
    }
  }
  // merge row slots of the wave (lanes that differ by multiples of LPR)
#pragma unroll
  for (int off = LPR; off < kWave; off <<= 1) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float mo = __shfl_xor(m[j], off), lo = __shfl_xor(l[j], off);
      float oo[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) oo[e] = __shfl_xor(o[j][e], off);
      float as, ao;
      merge_ml(m[j], l[j], mo, lo, as, ao);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[j][e] = o[j][e] * as + oo[e] * ao;
    }
  }
  if (slot == 0) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      if (sub == 0) {
        s_ml[wid][j][0] = m[j];
        s_ml[wid][j][1] = l[j];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[wid][j][sub * EPL + e] = o[j][e];
    }
  }
  __syncthreads();
  // merge the four waves: thread -> (head j, dim d)
  for (int idx = threadIdx.x; idx < G * D; idx += 256) {
    const int j = idx / D, d = idx % D;
    float mm = s_ml[0][j][0], ll = s_ml[0][j][1], oo = s_o[0][j][d];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      float as, ao;
      merge_ml(mm, ll, s_ml[w][j][0], s_ml[w][j][1], as, ao);
      oo = oo * as + s_o[w][j][d] * ao;
    }
    const int h = g * G + j;
    const int64_t pbase = ((int64_t)b * a.q_heads + h) * a.splits + split;
    a.part_o[pbase * a.v_dim + d] = oo;
    if (d == 0) {
      a.part_ml[pbase * 2 + 0] = mm;
      a.part_ml[pbase * 2 + 1] = ll;
    }
  }
}

// ------------------------------------------------------------------ MLA path

// Sparse MLA decode on bf16 MFMA 32x32x16.  One block per (split of 128
// selected rows, request) with NW waves (one per SIMD); wave w owns query
// heads 32w..32w+31.  The split's 128 latent rows reach LDS by DMA
// (global_load_lds) in four 32-row chunks and stay resident (147 KB):
//   S^T[token][head] = K_chunk (A operand, 32 tokens x 16 dims per step) *
//     Q^T (B operand, the wave's 32 heads over all 36 steps of the 576 dims,
//     loaded from global memory straight into registers), chunk by chunk as
//     each chunk lands (all four are requested at once); P = 2^(x - m) is
//     formed per chunk (bf16, in registers) against a reference m per head,
//     an integer, with x <= m + 8: it becomes ceil(max) at the first usable
//     token and again only when a chunk's max passes m + 8, and then the
//     earlier chunks' P are rescaled by the exact power of two
//     2^(m_old - m_new) (any reference gives the same softmax; the bound
//     keeps P in range and makes rescaling rare);
//   O[:, 0:256] += P * V[:, 0:256], then O[:, 256:512] += P * V[:, 256:512],
//     the V operand fetched with the transposing LDS read (ds_read_b64_tr_b16)
//     that hands each lane one value column of four rows.
// Splitting the value columns across the two passes halves the live
// accumulators (128 instead of 256 per lane) without computing S twice.
// 32x32x16 operand layout: lane l holds A[row l%32][8 k-values of half
// l/32], B[8 k-values of half l/32][col l%32], and C[rows
// 8*(r/4)+4*(l/32)+(r%4), r<16][col l%32].
//
// LDS rows are 72 sixteen-byte units plus four pad units (1216-byte
// stride), and within a row the units are stored XOR-swizzled: data unit u
// of row r sits at position u ^ ((r >> 2) & 7) (which stays inside the
// unit's aligned group of eight).  With that, the 16 rows of an A-fragment
// read and the 4 rows x 64 bytes of a transposed V read each hit 64
// different banks; a 32-row chunk is exactly 38 DMA instructions.
//
// DMA bookkeeping.  Every DMA instruction moves 64 consecutive LDS units and
// always has an active lane, so each wave knows exactly how many it has in
// flight and waits for a chunk with an exact count.  The compiler cannot
// order its own waits against DMA (it would drain all of it before any
// ordinary load or LDS read), so nothing in between does either: the row
// offsets sit in registers (lane l: rows l and l + 64) and are fetched with
// v_readlane, and the K fragments are read by asm blocks that wait for
// their own results.  A row that is not usable (index -1, past kv_len, bad
// page) is filled from the request's first query row instead: any finite
// data will do, its probability is exactly zero.
constexpr int kMlaD = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaChunkRows = 32;
constexpr int kMlaChunks = 4;
constexpr int kMlaSplitRows = kMlaChunkRows * kMlaChunks;  // 128 rows per block
constexpr int kMlaUnits = kMlaD / 8;                       // 72 units per row
constexpr int kMlaStride = kMlaUnits + 4;                  // LDS row stride in units
constexpr int kMlaRowBytes = kMlaStride * 16;              // 1216
constexpr int kMlaChunkUnits = kMlaChunkRows * kMlaStride;  // 2432
constexpr int kMlaChunkInsts = (kMlaChunkUnits + 63) / 64;  // 38 DMA instructions per chunk
constexpr float kMlaHeadroom = 8.0f;                         // P <= 2^8 between reference moves

// swizzle of row r's units (see above)
__host__ __device__ constexpr int mla_swz(int r) { return (r >> 2) & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short shortx4 __attribute__((ext_vector_type(4)));

// Wait until at most N vector memory operations of this wave are in flight
// (the counter holds 63 at most; a smaller count only waits longer), then
// meet the block at a barrier.  One asm block: __syncthreads() would add a
// workgroup fence, for which the compiler drains every DMA in flight.  LDS
// needs no fence: data a DMA has delivered is visible to the whole block.
template <int N>
__device__ __forceinline__ void mla_wait_vmcnt_barrier() {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" : : "i"(N < 63 ? N : 63) : "memory");
}

// Six K fragments (k-steps s0 .. s0+5) of this lane's row; one asm block
// that waits for its own results.  Step s reads base[s & 3] + 128 * (s >> 2)
// (the swizzle permutes units within aligned groups of eight, i.e. within
// four consecutive k-steps).
#define MLA_KF_OFF(S) "v"(addr[(S) & 3]), "i"(128 * ((S) >> 2))
template <int S0>
__device__ __forceinline__ void mla_kfrag6(u32x4 (&f)[6], const uint32_t (&addr)[4]) {
  asm volatile(
      "ds_read_b128 %0, %6 offset:%7\n\t"
      "ds_read_b128 %1, %8 offset:%9\n\t"
      "ds_read_b128 %2, %10 offset:%11\n\t"
      "ds_read_b128 %3, %12 offset:%13\n\t"
      "ds_read_b128 %4, %14 offset:%15\n\t"
      "ds_read_b128 %5, %16 offset:%17\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5])
      : MLA_KF_OFF(S0), MLA_KF_OFF(S0 + 1), MLA_KF_OFF(S0 + 2), MLA_KF_OFF(S0 + 3), MLA_KF_OFF(S0 + 4),
        MLA_KF_OFF(S0 + 5)
      : "memory");
}
#undef MLA_KF_OFF

template <int I, int N, typename F>
__device__ __forceinline__ void mla_static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    mla_static_for<I + 1, N>(f);
  }
}

template <int NW, bool QSTAGE>
__global__ __launch_bounds__(NW * 64, 1) void attn_mla_kernel(AttnArgs a) {
  constexpr int KSTEPS = kMlaD / 16;  // 36
  __shared__ __attribute__((aligned(16))) uint4 s_kv[kMlaSplitRows * kMlaStride];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 31, hf = lane >> 5;
  // Blocks are handed to the 8 XCDs round robin by index.  Block L runs
  // work item (xcd * per + L / 8), xcd = L % 8, so each XCD takes a
  // contiguous run of (request, split) items: a request's splits share one
  // L2 and read its query rows from there.
  int item = blockIdx.x;
  const int nitems = gridDim.x;
  if ((nitems & 7) == 0) item = (item & 7) * (nitems >> 3) + (item >> 3);
  const int b = item / a.splits;
  const int split = item - b * a.splits;
  const int r0 = split * kMlaSplitRows, r1 = min(a.k_sel, r0 + kMlaSplitRows);
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int32_t* sel = a.indices + (int64_t)b * a.k_sel;
  const float c = a.scale * kLog2e;
  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* qrow0 = reinterpret_cast<const char*>(a.q) + (int64_t)b * a.q_heads * kMlaD * 2;
  const int head0 = wid * 32;

  const uint32_t kv0 = (uint32_t)(uintptr_t)(lds_ptr_t)s_kv;
  // ---- byte offsets of rows lane and lane + 64 of the split (-1: not
  // usable); the query fragments are requested between the index and the
  // page-table lookups (B operand: lane l holds head head0 + l%32, dims
  // 16 s + 8 (l/32) .. +8)
  bf16x8 qf[KSTEPS];
  int64_t off_lo, off_hi;
  if constexpr (QSTAGE) {
    // The wave's 32 query rows are contiguous (36 KB): whole-row loads (lane
    // l of load i: 16-byte unit 64 i + l), written to the LDS the latent rows
    // take later, 73 units per row (one pad unit: the fragment reads of 16
    // lanes, rows 73 units apart, then hit distinct banks), read back as
    // fragments (head col, units 2 s + hf).  A fragment load straight from
    // memory touches a different 32-byte piece of a different row in every
    // lane pair; these loads cover 1 KB each.
    constexpr int kQRowUnits = kMlaUnits + 1;  // 73
    static_assert(NW * 32 * kQRowUnits <= kMlaSplitRows * kMlaStride, "the query staging fits the row buffer");
    const int i0 = r0 + lane, i1 = r0 + 64 + lane;
    const int t0 = i0 < r1 ? sel[i0] : -1;
    const int t1 = i1 < r1 ? sel[i1] : -1;
    const uint4* qw = reinterpret_cast<const uint4*>(qrow0 + (int64_t)head0 * kMlaD * 2);
    uint4 qraw[KSTEPS];
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) qraw[i] = qw[64 * i + lane];
    const int64_t e0 = sel_row(a, bt, L, t0, 0, a.k_page_stride, a.k_head_stride, a.k_token_stride, a.k_num_pages);
    const int64_t e1 = sel_row(a, bt, L, t1, 0, a.k_page_stride, a.k_head_stride, a.k_token_stride, a.k_num_pages);
    off_lo = e0 < 0 ? -1 : e0 * 2;
    off_hi = e1 < 0 ? -1 : e1 * 2;
    uint4* qs = s_kv + wid * 32 * kQRowUnits;
#pragma unroll
    for (int i = 0; i < KSTEPS; ++i) {
      const int u = 64 * i + lane;
      qs[(u / kMlaUnits) * kQRowUnits + u % kMlaUnits] = qraw[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, qs[col * kQRowUnits + 2 * s + hf]);
    // every wave holds its fragments before any DMA overwrites the staging
    // (no DMA is in flight yet, so this barrier drains nothing)
    __syncthreads();
  } else {
    const int i0 = r0 + lane, i1 = r0 + 64 + lane;
    const int t0 = i0 < r1 ? sel[i0] : -1;
    const int t1 = i1 < r1 ? sel[i1] : -1;
    const uint4* qp = reinterpret_cast<const uint4*>(qrow0 + (int64_t)(head0 + col) * kMlaD * 2) + hf;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = __builtin_bit_cast(bf16x8, qp[2 * s]);
    const int64_t e0 = sel_row(a, bt, L, t0, 0, a.k_page_stride, a.k_head_stride, a.k_token_stride, a.k_num_pages);
    const int64_t e1 = sel_row(a, bt, L, t1, 0, a.k_page_stride, a.k_head_stride, a.k_token_stride, a.k_num_pages);
    off_lo = e0 < 0 ? -1 : e0 * 2;
    off_hi = e1 < 0 ? -1 : e1 * 2;
  }
  // the query fragments and offsets have landed (a wait the compiler sees,
  // so that it waits for no DMA when the fragments are used)
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  // usable-row masks, rows 0..63 and 64..127
  const uint64_t ok_lo = __ballot(off_lo >= 0), ok_hi = __ballot(off_hi >= 0);

  // ---- DMA of the latent rows, 32-row chunks; wave w issues instructions
  // w, w + NW, ... of each chunk: (38 - w + NW - 1) / NW of them.
  // Instruction i moves LDS units 64 i .. +63 of the chunk; this lane's unit
  // u = 64 i + l is chunk row r = u / 76, position u % 76, which holds data
  // unit position ^ swizzle (pad positions re-read unit 0).  The row's
  // offset (16-byte units, int32) comes from the lane that resolved it; a
  // row that is not usable is filled from the request's first query row:
  // any finite data will do, its probability is exactly zero.
  const int32_t u_lo = off_lo < 0 ? -1 : (int32_t)(off_lo >> 4);
  const int32_t u_hi = off_hi < 0 ? -1 : (int32_t)(off_hi >> 4);
  auto issue_chunk = [&](int j) {
    const int32_t held = j < 2 ? u_lo : u_hi;  // chunk j's rows 32 j .. +31 sit in one half
    const uint32_t cbase = kv0 + 16u * (uint32_t)(j * kMlaChunkUnits);
#pragma unroll
    for (int k = 0; k < (kMlaChunkInsts + NW - 1) / NW; ++k) {
      const int i = wid + NW * k;
      if (i < kMlaChunkInsts) {
        const int u = 64 * i + lane;
        const int r = u / kMlaStride, pos = u - r * kMlaStride;
        const int32_t o = __builtin_amdgcn_ds_bpermute(4 * ((32 * j + r) & 63), held);
        const int du = pos < kMlaUnits ? pos ^ mla_swz(r) : 0;
        const char* src = (o >= 0 ? kb + 16 * (int64_t)o : qrow0) + 16 * du;
        __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(uintptr_t)(cbase + 1024u * i), 16, 0, kLoadStream);
      }
    }
  };
#pragma unroll
  for (int j = 0; j < kMlaChunks; ++j) issue_chunk(j);

  // ---- S^T chunk by chunk as the chunks land.  This lane: head `col`,
  // tokens 32j + 8*(r/4) + 4*hf + (r%4).  Probabilities are formed chunk by
  // chunk against the reference m (-inf while no token is usable); when it
  // moves, the probabilities already formed are scaled by 2^(m_old - m_new),
  // an exact power of two.
  uint32_t pw[kMlaChunks][8];  // bf16 P of each chunk, A-operand layout
  float m_run = -__builtin_inff(), psum = 0.0f;
  // K fragment bases: row col of the chunk, data unit 2t + hf (t = s & 3)
  uint32_t kaddr[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) kaddr[t] = kv0 + (uint32_t)(col * kMlaRowBytes + 16 * ((2 * t + hf) ^ mla_swz(col)));
  mla_static_for<0, kMlaChunks>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    // the later chunks may still be in flight: wait for the rest, then for
    // everyone's
    constexpr int later = kMlaChunks - 1 - j;
    mla_static_for<0, NW>([&](auto wc) {
      constexpr int w = decltype(wc)::value;
      if (wid == w) mla_wait_vmcnt_barrier<later * ((kMlaChunkInsts - w + NW - 1) / NW)>();
    });
    floatx16 st = floatx16{};
    mla_static_for<0, KSTEPS / 6>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      u32x4 kf[6];
      uint32_t ka[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) ka[t] = kaddr[t] + (uint32_t)(j * kMlaChunkRows * kMlaRowBytes);
      mla_kfrag6<6 * g>(kf, ka);
#pragma unroll
      for (int e = 0; e < 6; ++e)
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kf[e]), qf[6 * g + e], st, 0, 0, 0);
    });
    float cmax = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tk = kMlaChunkRows * j + 8 * (r / 4) + 4 * hf + (r % 4);
      const bool ok = ((tk < 64 ? ok_lo : ok_hi) >> (tk & 63)) & 1;
      st[r] = ok ? st[r] * c : -__builtin_inff();
      cmax = fmaxf(cmax, st[r]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));  // both token halves of head `col`
    const bool mv = cmax > m_run + kMlaHeadroom || (m_run == -__builtin_inff() && cmax != -__builtin_inff());
    const float m_new = mv ? ceilf(cmax) : m_run;
    if constexpr (j > 0) {
      // 2^(m_run - m_new) where m moves from a finite value (before the
      // first usable token every P so far is zero)
      if (__ballot(mv && m_run != -__builtin_inff())) {
        const float f = mv && m_run != -__builtin_inff() ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        psum *= f;
#pragma unroll
        for (int jj = 0; jj < j; ++jj)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float lo = bf16_lo(pw[jj][e]) * f, hi = bf16_hi(pw[jj][e]) * f;
            pw[jj][e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){lo, hi}, bf16x2));
          }
      }
    }
    m_run = m_new;
    // masked tokens: exp2(-inf - mref) = 0 (mref finite even with no token)
    const float mref = m_new == -__builtin_inff() ? 0.0f : m_new;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(st[r] - mref);
      const float p1 = __builtin_amdgcn_exp2f(st[r + 1] - mref);
      psum += p0 + p1;
      pw[j][r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){p0, p1}, bf16x2));
    }
  });
  const float m_blk = m_run;

  // ---- O[:, 256*half ...] += P_j V_j.  In k-step ks of chunk j the lane's
  // 8 P values are tokens 32j + 16ks + 4hf + e (e < 4) and 32j + 16ks + 8 +
  // 4hf + (e - 4); the transposing read gives lane i of each 16-lane group
  // the value column i of four rows, lane 4m + c of the group naming row m,
  // columns 4c .. 4c+3.  Group G of the wave covers value columns 16*(G%2) ..
  // +16 of the N tile for k half G/2 = hf.
  // Row 32j + 16ks + 4hf + m (+8 for the second read) has swizzle
  // (4ks + hf + 2*second) & 7 and value column dv = 256*half + 32*cc +
  // 16*(G&1) + 4c lies in data unit 32*half + 4*cc + 2*(G&1) + c/2, byte
  // 8*(c&1) of it.  The lane-dependent part of the position goes into two
  // bases (second read or not); the rest is a constant offset.
  const int g16 = lane & 15, G = lane >> 4;
  const int vm = g16 >> 2, vc = g16 & 3;
  uint32_t vbase[2];
#pragma unroll
  for (int sec = 0; sec < 2; ++sec)
    vbase[sec] = kv0 + (uint32_t)((4 * hf + vm + 8 * sec) * kMlaRowBytes +
                                  16 * ((2 * ((G & 1) ^ sec)) | ((vc >> 1) ^ hf)) + 8 * (vc & 1));
  floatx16 acc[8];
  const int64_t blk = (int64_t)b * a.splits + split;
  uint16_t* po = reinterpret_cast<uint16_t*>(a.part_o) + ((blk * NW + wid) * 16) * (64 * 16);
  // V fragments of one (chunk, k-step) and N tile: two transposed reads.
  auto vload = [&](shortx4 (&v)[2], int half, int step, int cc) {
    const int j = step >> 1, ks = step & 1;
    const uint32_t off = (uint32_t)((32 * j + 16 * ks) * kMlaRowBytes + 16 * (8 * (4 * half + cc / 2) + 4 * ((cc & 1) ^ ks)));
    v[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(uintptr_t)(vbase[0] + off));
    v[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(uintptr_t)(vbase[1] + off));
  };
  // Each MFMA is followed by the two reads for the same N tile one step
  // later, so every read has eight MFMAs of lead while at most 14 reads
  // follow the one being waited for (the LDS counter holds 15).
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = floatx16{};
    shortx4 vb[2][8][2];
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) vload(vb[0][cc], half, 0, cc);
#pragma unroll
    for (int step = 0; step < 2 * kMlaChunks; ++step) {
      const int j = step >> 1, ks = step & 1;
      const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pw[j][4 * ks], pw[j][4 * ks + 1], pw[j][4 * ks + 2], pw[j][4 * ks + 3]});
#pragma unroll
      for (int cc = 0; cc < 8; ++cc) {
        const shortx4 v0 = vb[step & 1][cc][0], v1 = vb[step & 1][cc][1];
        const bf16x8 vv = __builtin_bit_cast(bf16x8, (shortx8){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
        acc[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, vv, acc[cc], 0, 0, 0);
        if (step + 1 < 2 * kMlaChunks) vload(vb[(step + 1) & 1][cc], half, step + 1, cc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // partials in register order, bf16: part_o[((b*splits+split)*NW + w)][n][h][lane][8]:
    // lane l's 16 values of tile n as two halves h of 8 (n < 8: dv 0..255, n >= 8: dv
    // 256..511), so that each store instruction writes 1 KB in one piece
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      u32x4 w0, w1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w0[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){acc[n][2 * e], acc[n][2 * e + 1]}, bf16x2));
        w1[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){acc[n][8 + 2 * e], acc[n][8 + 2 * e + 1]}, bf16x2));
      }
      uint4* dst = reinterpret_cast<uint4*>(po + ((int64_t)(8 * half + n) * 128 + lane) * 8);
      dst[0] = make_uint4(w0[0], w0[1], w0[2], w0[3]);
      dst[64] = make_uint4(w1[0], w1[1], w1[2], w1[3]);
    }
  }
  // m / l per head: part_ml[(b*splits+split)*q_heads + h][2]
  const float l_tot = psum + __shfl_xor(psum, 32);
  if (hf == 0) {
    float* ml = a.part_ml + (blk * a.q_heads + head0 + col) * 2;
    ml[0] = m_blk;
    ml[1] = l_tot;
  }
}

// Combine of the MLA partials: one 512-thread block per (request, wave w,
// quarter of the value columns): thread (tile n, half jh, lane l) owns heads
// 32w + 8(r/4) + 4(l/32) + r%4 (8jh <= r < 8jh + 8) at dv = 128*quarter +
// 32*(n%4) + l%32.  Split weights 2^(m_s - M) / sum_s l_s 2^(m_s - M) are
// computed once per head into LDS while each thread's partials of the first
// 16 splits are already in flight (the two reads do not depend on each
// other); the result is transposed through LDS so output rows are written
// contiguously.
constexpr int kMlaMaxSplits = 64;

__global__ __launch_bounds__(512) void attn_mla_combine_kernel(AttnArgs a, int nw) {
  __shared__ float s_m[kMlaMaxSplits][32], s_l[kMlaMaxSplits][32];
  __shared__ float s_w[kMlaMaxSplits][32];   // weight of split s for head 32w + h
  __shared__ __attribute__((aligned(16))) float s_out[32][128 + 4];  // [head][dv in the quarter], padded
  const int tid = threadIdx.x;
  const int lane = tid & 63, n = tid >> 7;  // tile within the quarter: 0..3
  const int jh = (tid >> 6) & 1;            // which eight of the lane's 16 values
  // the same XCD placement as attn_mla_kernel: a request's items run where
  // its splits ran (blocks go to the 8 XCDs round robin by index)
  int item = blockIdx.x;
  if ((gridDim.x & 7) == 0) item = (item & 7) * (gridDim.x >> 3) + (item >> 3);
  const int quarter = item % 4, w = (item / 4) % nw, b = item / (4 * nw);
  const int col = lane & 31, hf = lane >> 5;
  const int S = a.splits;
  const int tile = 4 * quarter + n;  // N tile of the partial layout (0..15)
  const uint16_t* pbase =
      reinterpret_cast<const uint16_t*>(a.part_o) + ((((int64_t)w * 16 + tile) * 2 + jh) * 64 + lane) * 8;
  const int64_t sstride = (int64_t)nw * 16 * 64 * 16;  // one split's partial, in elements
  // ---- m and l of (split, head) for the first 16 splits (one pair per
  // thread), then this thread's partials of those splits: the pairs land
  // first, so the split weights are formed while the partials are in flight
  float2 ml0 = make_float2(0.0f, 0.0f);
  if (tid < S * 32) {
    const int sp = tid >> 5, h = tid & 31;
    ml0 = *reinterpret_cast<const float2*>(a.part_ml + (((int64_t)b * S + sp) * a.q_heads + 32 * w + h) * 2);
  }
  uint4 q[16];
#pragma unroll
  for (int u = 0; u < 16; ++u)  // (branch-free: fewer splits re-read the last)
    q[u] = *reinterpret_cast<const uint4*>(pbase + ((int64_t)b * S + min(u, S - 1)) * sstride);
  if (tid < S * 32) {
    s_m[tid >> 5][tid & 31] = ml0.x;
    s_l[tid >> 5][tid & 31] = ml0.y;
  }
  for (int i = tid + 512; i < S * 32; i += 512) {  // more than 16 splits
    const int sp = i >> 5, h = i & 31;
    const float* ml = a.part_ml + (((int64_t)b * S + sp) * a.q_heads + 32 * w + h) * 2;
    s_m[sp][h] = ml[0];
    s_l[sp][h] = ml[1];
  }
  __syncthreads();
  if (tid < 32) {
    float mx = -__builtin_inff();
    for (int sp = 0; sp < S; ++sp) mx = fmaxf(mx, s_m[sp][tid]);
    float Ls = 0.0f;
    for (int sp = 0; sp < S; ++sp) {
      const float m = s_m[sp][tid];
      const float e = m == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(m - mx);
      s_w[sp][tid] = e;
      Ls += s_l[sp][tid] * e;
    }
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
    for (int sp = 0; sp < S; ++sp) s_w[sp][tid] *= inv;
  }
  __syncthreads();
  // ---- weighted sum over splits of this thread's 16 partial values
  float o[8];  // values 8jh .. 8jh+7 of the lane's 16
#pragma unroll
  for (int r = 0; r < 8; ++r) o[r] = 0.0f;
  for (int s0 = 0; s0 < S; s0 += 16) {
    if (s0 > 0) {
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (s0 + u < S) q[u] = *reinterpret_cast<const uint4*>(pbase + ((int64_t)b * S + s0 + u) * sstride);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (s0 + u < S) {
        const uint32_t wv[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r0 = 8 * jh + 2 * e;
          o[2 * e] += bf16_lo(wv[e]) * s_w[s0 + u][8 * (r0 / 4) + 4 * hf + (r0 % 4)];
          o[2 * e + 1] += bf16_hi(wv[e]) * s_w[s0 + u][8 * ((r0 + 1) / 4) + 4 * hf + ((r0 + 1) % 4)];
        }
      }
  }
  // ---- transpose to [head][dv] and write rows
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int rr = 8 * jh + r;
    s_out[8 * (rr / 4) + 4 * hf + (rr % 4)][32 * n + col] = o[r];
  }
  __syncthreads();
  if ((reinterpret_cast<uintptr_t>(a.out) & 15) == 0) {
    // eight consecutive values per thread: one 16-byte store (bf16) or two (fp32)
    const int h = tid >> 4, d0 = 8 * (tid & 15);
    const int64_t oi = ((int64_t)b * a.q_heads + 32 * w + h) * kMlaDv + 128 * quarter + d0;
    const float4 v0 = *reinterpret_cast<const float4*>(&s_out[h][d0]);
    const float4 v1 = *reinterpret_cast<const float4*>(&s_out[h][d0 + 4]);
    if (a.out_dtype == 0) {
      float4* dst = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + oi);
      dst[0] = v0;
      dst[1] = v1;
    } else {
      const uint32_t p0 = f32_to_bf16(v0.x) | ((uint32_t)f32_to_bf16(v0.y) << 16);
      const uint32_t p1 = f32_to_bf16(v0.z) | ((uint32_t)f32_to_bf16(v0.w) << 16);
      const uint32_t p2 = f32_to_bf16(v1.x) | ((uint32_t)f32_to_bf16(v1.y) << 16);
      const uint32_t p3 = f32_to_bf16(v1.z) | ((uint32_t)f32_to_bf16(v1.w) << 16);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.out) + oi) = make_uint4(p0, p1, p2, p3);
    }
  } else {
    for (int i = tid; i < 32 * 128; i += 512) {
      const int h = i / 128, d = i % 128;
      const int64_t oi = ((int64_t)b * a.q_heads + 32 * w + h) * kMlaDv + 128 * quarter + d;
      if (a.out_dtype == 0)
        reinterpret_cast<float*>(a.out)[oi] = s_out[h][d];
      else
        reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(s_out[h][d]);
    }
  }
}

// ------------------------------------------------------------------ combine

// out[b][h][:] = sum_s 2^(m_s-M) o_s / sum_s 2^(m_s-M) l_s; zeros if empty.
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int bh = blockIdx.x;
  const int64_t base = (int64_t)bh * a.splits;
  float M = -__builtin_inff();
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, a.part_ml[(base + s) * 2]);
  float Ls = 0.0f;
  if (M != -__builtin_inff())
    for (int s = 0; s < a.splits; ++s) {
      const float m = a.part_ml[(base + s) * 2];
      if (m != -__builtin_inff()) Ls += a.part_ml[(base + s) * 2 + 1] * exp2f(m - M);
    }
  const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
  for (int d = threadIdx.x; d < a.v_dim; d += blockDim.x) {
    float o = 0.0f;
    if (Ls > 0.0f)
      for (int s = 0; s < a.splits; ++s) {
        const float m = a.part_ml[(base + s) * 2];
        if (m != -__builtin_inff()) o += a.part_o[(base + s) * a.v_dim + d] * exp2f(m - M);
      }
    o *= inv;
    if (a.out_dtype == 0)
      reinterpret_cast<float*>(a.out)[(int64_t)bh * a.v_dim + d] = o;
    else
      reinterpret_cast<uint16_t*>(a.out)[(int64_t)bh * a.v_dim + d] = f32_to_bf16(o);
  }
}

// ------------------------------------------------------------------ launch

bool attn_mla_supported(const AttnArgs& a) {
  return a.dtype == 1 && a.head_dim == kMlaD && a.v_dim == kMlaDv && a.num_kv_heads == 1 &&
         (a.q_heads == 32 || a.q_heads == 64 || a.q_heads == 128) && a.k == a.v &&
         a.k_page_stride == a.v_page_stride && a.k_token_stride == a.v_token_stride &&
         a.k_num_pages == a.v_num_pages && (a.k_token_stride % 8) == 0 && (a.k_page_stride % 8) == 0 &&
         (int64_t)a.k_num_pages * a.k_page_stride < ((int64_t)1 << 34) &&  // row offsets: int32 16-byte units
         a.k_sel <= kMlaMaxSplits * kMlaSplitRows;
}

bool attn_vec_supported(const AttnArgs& a) {
  const int G = a.q_heads / a.num_kv_heads;
  return (a.head_dim == 64 || a.head_dim == 128) && a.v_dim == a.head_dim &&
         (G == 1 || G == 2 || G == 4 || G == 8);
}

int attn_rows_per_split(const AttnArgs& a, bool mla) {
  if (mla) return kMlaSplitRows;
  // aim for a few hundred blocks; rows per split a multiple of 32
  const int rows_tot = a.k_sel;
  const int units = a.batch * (mla ? 1 : a.num_kv_heads);
  const int target = mla ? 256 : 512;  // MLA: one 4-wave block per CU
  int want_splits = units >= target ? 1 : (target + units - 1) / units;
  int chunk = (rows_tot + want_splits - 1) / want_splits;
  chunk = ((chunk + 31) / 32) * 32;
  const int min_chunk = 64;
  if (chunk < min_chunk) chunk = min_chunk;
  return chunk;
}

template <typename T, int D>
static hipError_t launch_vec_g(const AttnArgs& a, dim3 grid, hipStream_t st) {
  switch (a.q_heads / a.num_kv_heads) {
    case 1: attn_vec_kernel<T, D, 1><<<grid, 256, 0, st>>>(a); break;
    case 2: attn_vec_kernel<T, D, 2><<<grid, 256, 0, st>>>(a); break;
    case 4: attn_vec_kernel<T, D, 4><<<grid, 256, 0, st>>>(a); break;
    case 8: attn_vec_kernel<T, D, 8><<<grid, 256, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, hipStream_t st) {
  if (a.batch == 0) return hipSuccess;
  hipError_t e;
  if (attn_mla_supported(a)) {
    if (a.chunk != kMlaSplitRows || a.splits > kMlaMaxSplits) return hipErrorInvalidValue;
    dim3 grid(a.splits * a.batch);
    const int nw = a.q_heads / 32;
    static const int qstage = [] {
      const char* e = getenv("SD_MLA_QSTAGE");
      return e && e[0] == '0' ? 0 : 1;
    }();
    switch (nw * 2 + qstage) {
      case 2: attn_mla_kernel<1, false><<<grid, 64, 0, st>>>(a); break;
      case 4: attn_mla_kernel<2, false><<<grid, 128, 0, st>>>(a); break;
      case 8: attn_mla_kernel<4, false><<<grid, 256, 0, st>>>(a); break;
      case 3: attn_mla_kernel<1, true><<<grid, 64, 0, st>>>(a); break;
      case 5: attn_mla_kernel<2, true><<<grid, 128, 0, st>>>(a); break;
      case 9: attn_mla_kernel<4, true><<<grid, 256, 0, st>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    attn_mla_combine_kernel<<<a.batch * nw * 4, 512, 0, st>>>(a, nw);
    return hipGetLastError();
  } else {
    dim3 grid(a.splits, a.batch * a.num_kv_heads);
    if (a.dtype == 0)
      e = a.head_dim == 64 ? launch_vec_g<float, 64>(a, grid, st) : launch_vec_g<float, 128>(a, grid, st);
    else
      e = a.head_dim == 64 ? launch_vec_g<uint16_t, 64>(a, grid, st) : launch_vec_g<uint16_t, 128>(a, grid, st);
  }
  if (e != hipSuccess) return e;
  attn_combine_kernel<<<a.batch * a.q_heads, 128, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sd
