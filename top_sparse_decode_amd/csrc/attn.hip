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

// Sparse MLA decode on bf16 MFMA 32x32x16.  One block per (split, request)
// with NW waves; wave w owns query heads 32w..32w+31.  The selected latent
// rows of a split are staged 32 at a time into LDS (double buffered) and
// shared by every wave:
//   S^T[token][head] = K_tile (A, 32 tokens x 16 dims per step) * Q^T (B,
//                      held in registers for all 36 steps of the 576 dims),
//   O[head][dv]     += P (A, the bf16 probabilities already in registers)
//                      * V (B, read from the same LDS rows, first 512 dims).
// 32x32x16 operand layout: lane l holds A[row l%32][8 k-values of half
// l/32], B[8 k-values of half l/32][col l%32], and
// C[rows 8*(r/4)+4*(l/32)+(r%4), r<16][col l%32].
constexpr int kMlaD = 576;
constexpr int kMlaDv = 512;
constexpr int kMlaRows = 32;
constexpr int kMlaStride = kMlaD + 8;  // LDS row stride (elements)

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_mla_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KSTEPS = kMlaD / 16;  // 36
  __shared__ __attribute__((aligned(16))) uint16_t s_kv[2][kMlaRows][kMlaStride];
  __shared__ int s_ok[2][kMlaRows];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int b = blockIdx.y;
  const int split = blockIdx.x;
  const int r0 = split * a.chunk, r1 = min(a.k_sel, r0 + a.chunk);
  const int cap = min(a.max_kv_len, a.max_pages * a.page_size);
  const int L = clamp_len(a.kv_lens[b], cap);
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int32_t* sel = a.indices + (int64_t)b * a.k_sel;
  const float c = a.scale * kLog2e;
  const uint16_t* kb = reinterpret_cast<const uint16_t*>(a.k);
  const int head0 = wid * 32;

  // Q^T fragments: lane holds head (head0+col), dims 16s + 8hf .. +8
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q) + ((int64_t)b * a.q_heads + head0 + col) * kMlaD + 8 * hf;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qp + 16 * s);
  }

  floatx16 acc[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) acc[n] = floatx16{};
  float m_run = -__builtin_inff();  // per head `col` (both halves agree)
  float l_run = 0.0f;               // partial over this half's tokens

  // staging: thread -> (row tr, 16-byte chunks tc + 8i, i < 9).  K and V are
  // the same latent rows (the launcher checks that the pools alias).
  const int tr = tid / 8 % kMlaRows, tc = tid % 8;
  const int nchunks = (r1 - r0 + kMlaRows - 1) / kMlaRows;
  uint4 pre[9];
  int pre_ok = 0;
  auto fetch = [&](int chunk) {
    const int i = r0 + chunk * kMlaRows + tr;
    const int t = i < r1 ? sel[i] : -1;
    const int64_t ko = sel_row(a, bt, L, t, 0, a.k_page_stride, a.k_head_stride, a.k_token_stride, a.k_num_pages);
    pre_ok = ko >= 0;
#pragma unroll
    for (int q = 0; q < 9; ++q) {
      const int ch = tc + 8 * q;  // 16-byte chunk 0..71 of the 1152-byte row
      pre[q] = pre_ok ? *reinterpret_cast<const uint4*>(kb + ko + ch * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 9; ++q) *reinterpret_cast<uint4*>(&s_kv[buf][tr][(tc + 8 * q) * 8]) = pre[q];
    if (tc == 0) s_ok[buf][tr] = pre_ok;
  };

  // NT threads cover 32 rows x 8 chunk lanes when NT == 256; smaller blocks
  // loop over row groups.
  constexpr int RPASS = NT / 8;  // rows staged per pass
  auto fetch_stash_all = [&](int chunk, int buf) {
    for (int rp = 0; rp < kMlaRows; rp += RPASS) {
      const int row = rp + tid / 8;
      const int i = r0 + chunk * kMlaRows + row;
      const int t = i < r1 ? sel[i] : -1;
      const int64_t ko = sel_row(a, bt, L, t, 0, a.k_page_stride, a.k_head_stride, a.k_token_stride, a.k_num_pages);
      const int ok = ko >= 0;
#pragma unroll
      for (int q = 0; q < 9; ++q) {
        const int ch = tc + 8 * q;
        const uint4 v = ok ? *reinterpret_cast<const uint4*>(kb + ko + ch * 8) : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(&s_kv[buf][row][ch * 8]) = v;
      }
      if (tc == 0) s_ok[buf][row] = ok;
    }
  };

  if (nchunks > 0) {
    if constexpr (NT == 256) {
      fetch(0);
      stash(0);
    } else {
      fetch_stash_all(0, 0);
    }
  }
  __syncthreads();

  for (int ck = 0; ck < nchunks; ++ck) {
    const int buf = ck & 1;
    const bool more = ck + 1 < nchunks;
    if constexpr (NT == 256) {
      if (more) fetch(ck + 1);
    }
    // ---- S^T = K Q^T for 32 tokens x 32 heads
    floatx16 st = floatx16{};
    const uint16_t* arow = &s_kv[buf][col][8 * hf];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(arow + 16 * s);
      st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], st, 0, 0, 0);
    }
    // ---- online softmax for head `col`; this lane's 16 tokens:
    //      token(r) = 8*(r/4) + 4*hf + (r%4)
    float x[16];
    float cmax = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int tk = 8 * (r / 4) + 4 * hf + (r % 4);
      x[r] = s_ok[buf][tk] ? st[r] * c : -__builtin_inff();
      cmax = fmaxf(cmax, x[r]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = (m_new == -__builtin_inff()) ? 1.0f : exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.0f;
    uint32_t pw[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = (x[r] == -__builtin_inff()) ? 0.0f : exp2f(x[r] - m_new);
      const float p1 = (x[r + 1] == -__builtin_inff()) ? 0.0f : exp2f(x[r + 1] - m_new);
      psum += p0 + p1;
      pw[r / 2] = uint32_t(f32_to_bf16(p0)) | (uint32_t(f32_to_bf16(p1)) << 16);
    }
    l_run = l_run * alpha + psum;
    // rescale O rows (heads) whose max moved; O rows are heads
    // 8*(r/4)+4*hf+(r%4), the lane that owns head h's alpha is lane h.
    if (__ballot(alpha != 1.0f)) {
      float ar[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) ar[r] = __shfl(alpha, 8 * (r / 4) + 4 * hf + (r % 4));
#pragma unroll
      for (int n = 0; n < 16; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[n][r] *= ar[r];
    }
    // ---- O += P V over the 32 tokens: two k-steps of 16 tokens.  In k-step
    // ks the lane's 8 P values are tokens 16ks + 8(p/4) + 4hf + p%4 (p<8),
    // so its V fragment must hold those tokens too.
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 pa = __builtin_bit_cast(bf16x8, u32x4{pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]});
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // rows of the 8 tokens, 8 dv values each: dv = 256*half + 8*col + cc
        u32x4 vr[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          const int tk = 16 * ks + 8 * (p / 4) + 4 * hf + (p % 4);
          vr[p] = *reinterpret_cast<const u32x4*>(&s_kv[buf][tk][256 * half + 8 * col]);
        }
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
          // B fragment of N tile (half, cc): element p = V[token p][dv cc]
          u32x4 bw;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t lo = vr[2 * w][cc / 2], hi = vr[2 * w + 1][cc / 2];
            // pick the 16-bit half cc%2 of each
            bw[w] = (cc & 1) ? __builtin_amdgcn_perm(hi, lo, 0x07060302u)
                             : __builtin_amdgcn_perm(hi, lo, 0x05040100u);
          }
          acc[8 * half + cc] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              pa, __builtin_bit_cast(bf16x8, bw), acc[8 * half + cc], 0, 0, 0);
        }
      }
    }
    if constexpr (NT == 256) {
      if (more) stash(buf ^ 1);
    } else {
      if (more) fetch_stash_all(ck + 1, buf ^ 1);
    }
    __syncthreads();
  }

  // ---- partials: m, l per head; O[head][dv]
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const int64_t pb = ((int64_t)b * a.q_heads + head0) * a.splits + split;
  if (hf == 0) {
    const int64_t p = pb + (int64_t)col * a.splits;
    a.part_ml[p * 2 + 0] = m_run;
    a.part_ml[p * 2 + 1] = l_tot;
  }
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    const int half = n / 8, cc = n % 8;
    const int dv = 256 * half + 8 * col + cc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = 8 * (r / 4) + 4 * hf + (r % 4);
      a.part_o[(pb + (int64_t)h * a.splits) * kMlaDv + dv] = acc[n][r];
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
         a.k_num_pages == a.v_num_pages && (a.k_token_stride % 8) == 0 && (a.k_page_stride % 8) == 0;
}

bool attn_vec_supported(const AttnArgs& a) {
  const int G = a.q_heads / a.num_kv_heads;
  return (a.head_dim == 64 || a.head_dim == 128) && a.v_dim == a.head_dim &&
         (G == 1 || G == 2 || G == 4 || G == 8);
}

int attn_rows_per_split(const AttnArgs& a, bool mla) {
  // aim for a few hundred blocks; rows per split a multiple of 32
  const int rows_tot = a.k_sel;
  const int units = a.batch * (mla ? 1 : a.num_kv_heads);
  int want_splits = units >= 512 ? 1 : (512 + units - 1) / units;
  int chunk = (rows_tot + want_splits - 1) / want_splits;
  chunk = ((chunk + 31) / 32) * 32;
  const int min_chunk = mla ? 128 : 64;
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
    dim3 grid(a.splits, a.batch);
    switch (a.q_heads / 32) {
      case 1: attn_mla_kernel<1><<<grid, 64, 0, st>>>(a); break;
      case 2: attn_mla_kernel<2><<<grid, 128, 0, st>>>(a); break;
      case 4: attn_mla_kernel<4><<<grid, 256, 0, st>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    e = hipGetLastError();
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
