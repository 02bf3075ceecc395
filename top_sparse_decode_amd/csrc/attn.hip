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
// a time, each row slot with its own running (m, l, o); slots and waves are
// merged at the end.
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
  for (int i0 = r0 + wid * RPW; i0 < r1; i0 += 4 * RPW) {
    const int i = i0 + slot;
    const int t = i < r1 ? sel[i] : -1;
    const int64_t ko = sel_row(a, bt, L, t, g, a.k_page_stride, a.k_head_stride, a.k_token_stride, a.k_num_pages);
    const int64_t vo = sel_row(a, bt, L, t, g, a.v_page_stride, a.v_head_stride, a.v_token_stride, a.v_num_pages);
    const bool ok = ko >= 0 && vo >= 0;
    float kv[EPL], vv[EPL];
    if (ok) {
      Vec<T>::unpack(*reinterpret_cast<const uint4*>(kb + ko + sub * EPL), kv);
      Vec<T>::unpack(*reinterpret_cast<const uint4*>(vb + vo + sub * EPL), vv);
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float x = 0.0f;
      if (ok) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) x = __builtin_fmaf(qf[j][e], kv[e], x);
      }
#pragma unroll
      for (int off = LPR / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
      if (ok) {
        const float mn = fmaxf(m[j], x);
        const float al = exp2f(m[j] - mn);
        const float p = exp2f(x - mn);
        l[j] = l[j] * al + p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = o[j][e] * al + p * vv[e];
        m[j] = mn;
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
// heads 32w..32w+31.  All 128 latent rows of the split are fetched at once
// by direct global->LDS loads and stay resident (147 KB of LDS):
//   S^T[token][head] = K_chunk (A operand, 32 tokens x 16 dims per step) *
//     Q^T (B operand, the wave's 32 heads over all 36 steps of the 576 dims,
//     held in registers), for all four 32-row chunks; the block max is then
//     exact, P = 2^(x - max) is formed once (bf16, in registers) and never
//     rescaled;
//   O[:, 0:256] += P * V[:, 0:256], then O[:, 256:512] += P * V[:, 256:512].
// Splitting the value columns across the two passes halves the live
// accumulators (128 instead of 256 per lane) without computing S twice.
// 32x32x16 operand layout: lane l holds A[row l%32][8 k-values of half
// l/32], B[8 k-values of half l/32][col l%32], and C[rows
// 8*(r/4)+4*(l/32)+(r%4), r<16][col l%32].
//
// LDS rows are 72 sixteen-byte units plus one pad unit (1168-byte stride):
// the 32 rows read by one A fragment fall on different banks, and every LDS
// address is affine in the loop indices (immediate offsets).
constexpr int kMlaD = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaChunkRows = 32;
constexpr int kMlaChunks = 4;
constexpr int kMlaSplitRows = kMlaChunkRows * kMlaChunks;  // 128 rows per block
constexpr int kMlaUnits = kMlaD / 8;                       // 72 units per row
constexpr int kMlaStride = kMlaUnits + 1;                  // LDS row stride in units

__device__ __forceinline__ int mla_unit(int row, int unit) { return row * kMlaStride + unit; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int NW>
__global__ __launch_bounds__(NW * 64, 1) void attn_mla_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = kMlaD / 16;  // 36
  __shared__ __attribute__((aligned(16))) uint4 s_kv[kMlaSplitRows * kMlaStride];
  __shared__ int64_t s_off[kMlaSplitRows];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int b = blockIdx.y;
  const int split = blockIdx.x;
  const int r0 = split * kMlaSplitRows, r1 = min(a.k_sel, r0 + kMlaSplitRows);
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int32_t* sel = a.indices + (int64_t)b * a.k_sel;
  const float c = a.scale * kLog2e;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k);
  const int head0 = wid * 32;

  // ---- row offsets of the split (element offset, -1 = not usable)
  for (int r = tid; r < kMlaSplitRows; r += NT) {
    const int i = r0 + r;
    const int t = i < r1 ? sel[i] : -1;
    s_off[r] = sel_row(a, bt, L, t, 0, a.k_page_stride, a.k_head_stride, a.k_token_stride, a.k_num_pages);
  }
  __syncthreads();
  // unusable rows are zero (their probabilities are zero; values must be finite)
  for (int u = tid; u < kMlaSplitRows * kMlaStride; u += NT)
    if (s_off[u / kMlaStride] < 0) s_kv[u] = make_uint4(0, 0, 0, 0);
  // ---- every usable row: one direct global->LDS load per 16-byte unit; a
  // wave's instruction covers 64 consecutive LDS units (pad units: no load)
  for (int ub = wid * 64; ub < kMlaSplitRows * kMlaStride; ub += NT) {
    const int u = ub + lane;
    const int row = u / kMlaStride, slot = u % kMlaStride;
    const int64_t off = s_off[row];
    if (off >= 0 && slot < kMlaUnits)
      __builtin_amdgcn_global_load_lds(kb + off + slot * 8, (lds_ptr_t)&s_kv[ub], 16, 0, 0);
  }
  // Q^T fragments: lane holds head (head0+col), dims 16s + 8hf .. +8
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.q_heads + head0 + col) * kMlaD + 8 * hf;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  floatx16 acc[8];
  uint32_t pw[kMlaChunks][8];  // bf16 P of each chunk, A-operand layout

  // ---- S^T for all 128 rows first, so the block max is exact and P needs
  // no later rescaling.  This lane: head `col`, tokens
  // 32j + 8*(r/4) + 4*hf + (r%4).
  float sc[kMlaChunks][16];
  float cmax = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < kMlaChunks; ++j) {
    floatx16 st = floatx16{};
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, s_kv[mla_unit(kMlaChunkRows * j + col, 2 * s + hf)]);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st, 0, 0, 0);
      // bound the scheduler's look-ahead of LDS reads (register pressure)
      if (s % 6 == 5) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tk = kMlaChunkRows * j + 8 * (r / 4) + 4 * hf + (r % 4);
      sc[j][r] = s_off[tk] >= 0 ? st[r] * c : -__builtin_inff();
      cmax = fmaxf(cmax, sc[j][r]);
    }
  }
  const float m_blk = fmaxf(cmax, __shfl_xor(cmax, 32));
  // masked tokens: exp2(-inf - mref) = 0 (mref finite even with no token)
  const float mref = m_blk == -__builtin_inff() ? 0.0f : m_blk;
  float psum = 0.0f;
#pragma unroll
  for (int j = 0; j < kMlaChunks; ++j)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(sc[j][r] - mref);
      const float p1 = __builtin_amdgcn_exp2f(sc[j][r + 1] - mref);
      psum += p0 + p1;
      pw[j][r / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){p0, p1}, bf16x2));
    }

  // O[:, 256*half ...] += P_j V_j for chunk j (V: first 512 dims of the rows)
  auto pv = [&](int j, int half) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        __builtin_amdgcn_sched_barrier(0);
      const bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pw[j][4 * ks], pw[j][4 * ks + 1], pw[j][4 * ks + 2], pw[j][4 * ks + 3]});
      // In k-step ks the lane's 8 P values are tokens 16ks + 8(p/4) + 4hf +
      // p%4; its V fragments hold those tokens.  Four N tiles at a time: 4
      // dv values (8 bytes) of each of the 8 tokens, dv = 256*half + 8*col + cc.
#pragma unroll
      for (int c0 = 0; c0 < 8; c0 += 4) {
        uint2 vr[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int tk = kMlaChunkRows * j + 16 * ks + 8 * (p / 4) + 4 * hf + (p % 4);
          vr[p] = reinterpret_cast<const uint2*>(&s_kv[mla_unit(tk, 32 * half + col)])[c0 / 4];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cc = c0; cc < c0 + 4; ++cc) {
          // B fragment of N tile cc: element p = V[token p][256*half + 8*col + cc]
          u32x4 bw;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const int q = (cc - c0) / 2;
            const uint32_t lo = q ? vr[2 * w].y : vr[2 * w].x, hi = q ? vr[2 * w + 1].y : vr[2 * w + 1].x;
            bw[w] = (cc & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                             : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
          }
          acc[cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, __builtin_bit_cast(bf16x8, bw), acc[cc], 0, 0, 0);
        }
      }
    }
  };
  // ---- partials in register order: part_o[((b*splits+split)*NW + w)][n][lane][16]
  // (n < 8: dv 0..255, n >= 8: dv 256..511); m / l per head:
  // part_ml[(b*splits+split)*q_heads + h][2]
  const int64_t blk = (int64_t)b * a.splits + split;
  float* po = a.part_o + ((blk * NW + wid) * 16) * (64 * 16);
  auto store = [&](int n0) {
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      float4* dst = reinterpret_cast<float4*>(po + ((int64_t)(n0 + n) * 64 + lane) * 16);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        dst[jj] = make_float4(acc[n][4 * jj], acc[n][4 * jj + 1], acc[n][4 * jj + 2], acc[n][4 * jj + 3]);
    }
  };
  // value columns 0..255, then 256..511, from the same probabilities
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int n = 0; n < 8; ++n) acc[n] = floatx16{};
#pragma unroll
    for (int j = 0; j < kMlaChunks; ++j) pv(j, half);
    store(8 * half);
  }
  const float l_tot = psum + __shfl_xor(psum, 32);
  if (hf == 0) {
    float* ml = a.part_ml + (blk * a.q_heads + head0 + col) * 2;
    ml[0] = m_blk;
    ml[1] = l_tot;
  }
}

// Combine of the MLA partials: one 512-thread block per (request, wave w,
// value half): thread (tile n, lane l) owns heads 32w + 8(r/4) + 4(l/32) + r%4
// (r < 16) at dv = 256*half + 8*(l%32) + n%8.  Split weights
// 2^(m_s - M) / sum_s l_s 2^(m_s - M) are computed once per head into LDS; the
// result is transposed through LDS so output rows are written contiguously.
constexpr int kMlaMaxSplits = 64;

__global__ __launch_bounds__(512) void attn_mla_combine_kernel(AttnArgs a, int nw) {
  __shared__ float s_w[kMlaMaxSplits][32];   // weight of split s for head 32w + h
  __shared__ float s_out[32][256 + 4];       // [head][dv in half], padded
  const int tid = threadIdx.x;
  const int lane = tid & 63, n = tid >> 6;  // tile within the half: 0..7
  const int half = blockIdx.x % 2, w = (blockIdx.x / 2) % nw, b = blockIdx.x / (2 * nw);
  const int col = lane & 31, hf = lane >> 5;
  const int S = a.splits;
  // ---- weights: thread h < 32 handles head 32w + h
  if (tid < 32) {
    const int h = 32 * w + tid;
    float mx = -__builtin_inff();
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, a.part_ml[(((int64_t)b * S + s) * a.q_heads + h) * 2]);
    float Ls = 0.0f;
    for (int s = 0; s < S; ++s) {
      const float* ml = a.part_ml + (((int64_t)b * S + s) * a.q_heads + h) * 2;
      const float e = ml[0] == -__builtin_inff() ? 0.0f : __builtin_amdgcn_exp2f(ml[0] - mx);
      s_w[s][tid] = e;
      Ls += ml[1] * e;
    }
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
    for (int s = 0; s < S; ++s) s_w[s][tid] *= inv;
  }
  __syncthreads();
  // ---- weighted sum over splits of this thread's 16 partial values
  float o[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) o[r] = 0.0f;
  const int tile = 8 * half + n;
  for (int s = 0; s < S; ++s) {
    const int64_t blk = (int64_t)b * S + s;
    const float4* src = reinterpret_cast<const float4*>(a.part_o + (((blk * nw + w) * 16 + tile) * 64 + lane) * 16);
    float v[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 q = src[j];
      v[4 * j] = q.x; v[4 * j + 1] = q.y; v[4 * j + 2] = q.z; v[4 * j + 3] = q.w;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) o[r] += v[r] * s_w[s][8 * (r / 4) + 4 * hf + (r % 4)];
  }
  // ---- transpose to [head][dv] and write rows
#pragma unroll
  for (int r = 0; r < 16; ++r) s_out[8 * (r / 4) + 4 * hf + (r % 4)][8 * col + n] = o[r];
  __syncthreads();
  for (int i = tid; i < 32 * 256; i += 512) {
    const int h = i / 256, d = i % 256;
    const int64_t oi = ((int64_t)b * a.q_heads + 32 * w + h) * kMlaDv + 256 * half + d;
    if (a.out_dtype == 0)
      reinterpret_cast<float*>(a.out)[oi] = s_out[h][d];
    else
      reinterpret_cast<uint16_t*>(a.out)[oi] = f32_to_bf16(s_out[h][d]);
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
    dim3 grid(a.splits, a.batch);
    const int nw = a.q_heads / 32;
    switch (nw) {
      case 1: attn_mla_kernel<1><<<grid, 64, 0, st>>>(a); break;
      case 2: attn_mla_kernel<2><<<grid, 128, 0, st>>>(a); break;
      case 4: attn_mla_kernel<4><<<grid, 256, 0, st>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    attn_mla_combine_kernel<<<a.batch * nw * 2, 512, 0, st>>>(a, nw);
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
