// tri.hip -- TriAttention selection modes: normalize the per-head score rows,
// reduce them by mode, then the library's top-k.
//
// "Add TriAttention KV-cache compression method" (Summary) puts a
// normalize/reduce step between paged-K scoring and TopK / tie settlement and
// names three eviction modes (union, per_head, per_layer_perhead); its Main
// Files name score normalization and union reduction.  The pages give no
// formula, so the library fixes one evaluation and keeps to it bit for bit:
//
//   per member row m = (layer, request b, KV head g), over its finite scores
//   at t < kv_len[b] (n of them):
//     P_c  = sum_{t % 256 == c} (double)s_t, t ascending, binary64 adds;
//     mu   = (P_0 + P_1 + ... + P_255, in order) / n;
//     var  = (the same sums of d_t * d_t, d_t = (double)s_t - mu) / n;
//     z_t  = (float)(((double)s_t - mu) / sqrt(var)), 0 when var == 0,
//            -inf for a non-finite score or t >= kv_len[b];
//   reduced row: r_t = max over the mode's members of z_t, members visited
//   layer by layer and head by head, a later member replacing the running
//   value only when strictly larger.
//
// Kernels: tri_stats_kernel (one 256-thread block per member row: thread c
// owns the tokens t = c + 256 i, so its partial is exactly P_c and the loads
// are coalesced; rows up to 4096 tokens stay in registers between the two
// passes) and tri_reduce_kernel (a token per lane, the members split into
// four ordered quarters).  Selection then runs on the reduced rows.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace sd {

constexpr int kTriThreads = 256;
constexpr int kTriRegs = 16;  // tokens per thread kept in registers (rows up to 4096)
constexpr int kTriSpan = 4096;  // tokens per block of the one-slice reduce

__global__ __launch_bounds__(kTriThreads) void tri_stats_kernel(TriArgs a) {
  __shared__ double s_part[kTriThreads];
  __shared__ double s_mu;
  const int m = blockIdx.x;  // member row (layer, b, g)
  const int tid = threadIdx.x;
  const int b = (m / a.groups) % a.batch;
  const int L = clamp_len(a.kv_lens[b], a.row_stride);
  const float* row = a.scores + (int64_t)m * a.row_stride;
  if (a.lens && (m % a.groups) == 0 && tid == 0) a.lens[m / a.groups] = a.kv_lens[b];
  const bool resident = L <= kTriThreads * kTriRegs;
  float x[kTriRegs];
  double part = 0.0;
  int n = 0;
  if (resident) {
#pragma unroll
    for (int i = 0; i < kTriRegs; ++i) {
      const int t = tid + kTriThreads * i;
      x[i] = t < L ? row[t] : -__builtin_inff();
    }
#pragma unroll
    for (int i = 0; i < kTriRegs; ++i)
      if (__builtin_isfinite(x[i])) {
        part = __dadd_rn(part, (double)x[i]);
        ++n;
      }
  } else {
    for (int t = tid; t < L; t += kTriThreads) {
      const float v = row[t];
      if (__builtin_isfinite(v)) {
        part = __dadd_rn(part, (double)v);
        ++n;
      }
    }
  }
  s_part[tid] = part;
  // n over the block (exact integer sum)
  int nn = wave_sum(n);
  __shared__ int s_n[kTriThreads / 64];
  if ((tid & 63) == 0) s_n[tid >> 6] = nn;
  __syncthreads();
  const int total = s_n[0] + s_n[1] + s_n[2] + s_n[3];
  if (tid == 0) {
    double s1 = 0.0;
    for (int c = 0; c < kTriThreads; ++c) s1 = __dadd_rn(s1, s_part[c]);
    s_mu = total > 0 ? __ddiv_rn(s1, (double)total) : 0.0;
  }
  __syncthreads();
  const double mu = s_mu;
  part = 0.0;
  if (resident) {
#pragma unroll
    for (int i = 0; i < kTriRegs; ++i)
      if (__builtin_isfinite(x[i])) {
        const double d = __dsub_rn((double)x[i], mu);
        part = __dadd_rn(part, __dmul_rn(d, d));
      }
  } else {
    for (int t = tid; t < L; t += kTriThreads) {
      const float v = row[t];
      if (__builtin_isfinite(v)) {
        const double d = __dsub_rn((double)v, mu);
        part = __dadd_rn(part, __dmul_rn(d, d));
      }
    }
  }
  __syncthreads();  // every thread has read s_mu
  s_part[tid] = part;
  __syncthreads();
  if (tid == 0) {
    double s2 = 0.0;
    for (int c = 0; c < kTriThreads; ++c) s2 = __dadd_rn(s2, s_part[c]);
    const double sigma = total > 0 ? __dsqrt_rn(__ddiv_rn(s2, (double)total)) : 0.0;
    a.stats[2 * (int64_t)m] = mu;
    a.stats[2 * (int64_t)m + 1] = sigma;
  }
}

__device__ __forceinline__ float tri_z(float s, double mu, double sigma) {
  if (!__builtin_isfinite(s)) return -__builtin_inff();
  if (sigma == 0.0) return 0.0f;
  return __double2float_rn(__ddiv_rn(__dsub_rn((double)s, mu), sigma));
}

// Lane = token.  SLICES = 4 (rows with many members): one block per
// (64-token tile, output row), wave j takes the j-th quarter of the row's
// members (in order), and the four partial maxima are combined in wave
// order.  SLICES = 1: each wave takes its own 64 tokens and all members.  A
// later value replaces the running one only when strictly larger, within a
// wave and across waves, so the result is the first member attaining the
// maximum, as in a single pass over the members.
template <int SLICES>
__global__ __launch_bounds__(kTriThreads) void tri_reduce_kernel(TriArgs a) {
  __shared__ float s_part[kTriThreads / 64][64];
  const int o = blockIdx.y;  // output row
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  // members of output row o: (layer l, head g), l in [l0, l0 + nl), g in [g0, g0 + ng)
  int b, g0, ng, nl, l0;
  if (a.mode == 0) {        // per layer, per head: the member itself
    l0 = o / (a.batch * a.groups);
    b = (o / a.groups) % a.batch;
    g0 = o % a.groups;
    ng = 1;
    nl = 1;
  } else if (a.mode == 1) {  // per head: over layers
    l0 = 0;
    b = o / a.groups;
    g0 = o % a.groups;
    ng = 1;
    nl = a.layers;
  } else {                   // union: over layers and heads
    l0 = 0;
    b = o;
    g0 = 0;
    ng = a.groups;
    nl = a.layers;
  }
  const int nm = nl * ng;
  const int per = (nm + SLICES - 1) / SLICES;
  const int j0 = SLICES == 1 ? 0 : min(nm, wid * per), j1 = SLICES == 1 ? nm : min(nm, j0 + per);
  const int L = clamp_len(a.kv_lens[b], a.row_stride);
  // running max of z over members [j0, j1) at token t
  auto reduce = [&](int t) {
    float r = -__builtin_inff();
    if (t >= L) return r;
    int j = j0;
    // eight members at a time: their loads are in flight together
    for (; j + 8 <= j1; j += 8) {
      float x[8];
      int64_t m[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int jj = j + u;
        m[u] = ((int64_t)(l0 + jj / ng) * a.batch + b) * a.groups + g0 + jj % ng;
        x[u] = a.scores[m[u] * a.row_stride + t];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float z = tri_z(x[u], a.stats[2 * m[u]], a.stats[2 * m[u] + 1]);
        if (z > r) r = z;
      }
    }
    for (; j < j1; ++j) {
      const int64_t m = ((int64_t)(l0 + j / ng) * a.batch + b) * a.groups + g0 + j % ng;
      const float z = tri_z(a.scores[m * a.row_stride + t], a.stats[2 * m], a.stats[2 * m + 1]);
      if (z > r) r = z;
    }
    return r;
  };
  float* out = a.reduced + (int64_t)o * a.row_stride;
  if constexpr (SLICES == 1) {
    // the block covers kTriSpan tokens, kTriThreads apart per thread
    const int tend = min(a.row_stride, (int)(blockIdx.x + 1) * kTriSpan);
    for (int t = blockIdx.x * kTriSpan + threadIdx.x; t < tend; t += kTriThreads) out[t] = reduce(t);
  } else {
    const int t = blockIdx.x * 64 + lane;
    s_part[wid][lane] = reduce(t);
    __syncthreads();
    if (wid == 0 && t < a.row_stride) {
      float v = s_part[0][lane];
#pragma unroll
      for (int w = 1; w < SLICES; ++w) {
        const float z = s_part[w][lane];
        if (z > v) v = z;
      }
      out[t] = v;
    }
  }
}

// The same reduction with four consecutive tokens per lane and 16-byte loads
// (rows whose stride is a multiple of four floats): a wave reads a member's
// 256 tokens with one instruction.  SLICES = 4: one block per (256-token
// tile, output row), wave j takes the j-th quarter of the members, partial
// maxima combined in wave order; SLICES = 1: a block covers kTriSpan tokens.
// Per token the arithmetic and the order are those of tri_reduce_kernel.
template <int SLICES>
__global__ __launch_bounds__(kTriThreads) void tri_reduce4_kernel(TriArgs a) {
  __shared__ float4 s_part[kTriThreads / 64][64];
  const int o = blockIdx.y;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int b, g0, ng, nl, l0;
  if (a.mode == 0) {
    l0 = o / (a.batch * a.groups);
    b = (o / a.groups) % a.batch;
    g0 = o % a.groups;
    ng = 1;
    nl = 1;
  } else if (a.mode == 1) {
    l0 = 0;
    b = o / a.groups;
    g0 = o % a.groups;
    ng = 1;
    nl = a.layers;
  } else {
    l0 = 0;
    b = o;
    g0 = 0;
    ng = a.groups;
    nl = a.layers;
  }
  const int nm = nl * ng;
  const int per = (nm + SLICES - 1) / SLICES;
  const int j0 = SLICES == 1 ? 0 : min(nm, wid * per), j1 = SLICES == 1 ? nm : min(nm, j0 + per);
  const int L = clamp_len(a.kv_lens[b], a.row_stride);
  auto member = [&](int j) { return ((int64_t)(l0 + j / ng) * a.batch + b) * a.groups + g0 + j % ng; };
  // running max of z over members [j0, j1) at tokens t0 .. t0 + 3 (t0 + 3 < row_stride)
  auto reduce4 = [&](int t0) {
    float r[4] = {-__builtin_inff(), -__builtin_inff(), -__builtin_inff(), -__builtin_inff()};
    if (t0 >= L) return make_float4(r[0], r[1], r[2], r[3]);
    int j = j0;
    for (; j + 4 <= j1; j += 4) {
      float4 x[4];
      int64_t m[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        m[u] = member(j + u);
        x[u] = *reinterpret_cast<const float4*>(a.scores + m[u] * a.row_stride + t0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double mu = a.stats[2 * m[u]], sg = a.stats[2 * m[u] + 1];
        const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z = t0 + e < L ? tri_z(xs[e], mu, sg) : -__builtin_inff();
          if (z > r[e]) r[e] = z;
        }
      }
    }
    for (; j < j1; ++j) {
      const int64_t m = member(j);
      const float4 x = *reinterpret_cast<const float4*>(a.scores + m * a.row_stride + t0);
      const double mu = a.stats[2 * m], sg = a.stats[2 * m + 1];
      const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float z = t0 + e < L ? tri_z(xs[e], mu, sg) : -__builtin_inff();
        if (z > r[e]) r[e] = z;
      }
    }
    return make_float4(r[0], r[1], r[2], r[3]);
  };
  float* out = a.reduced + (int64_t)o * a.row_stride;
  if constexpr (SLICES == 1) {
    const int tend = min(a.row_stride, (int)(blockIdx.x + 1) * kTriSpan);
    for (int t0 = blockIdx.x * kTriSpan + 4 * threadIdx.x; t0 < tend; t0 += 4 * kTriThreads)
      *reinterpret_cast<float4*>(out + t0) = reduce4(t0);
  } else {
    const int t0 = blockIdx.x * 256 + 4 * lane;
    s_part[wid][lane] = t0 < a.row_stride ? reduce4(t0) : make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();
    if (wid == 0 && t0 < a.row_stride) {
      float4 v = s_part[0][lane];
#pragma unroll
      for (int w = 1; w < SLICES; ++w) {
        const float4 z = s_part[w][lane];
        if (z.x > v.x) v.x = z.x;
        if (z.y > v.y) v.y = z.y;
        if (z.z > v.z) v.z = z.z;
        if (z.w > v.w) v.w = z.w;
      }
      *reinterpret_cast<float4*>(out + t0) = v;
    }
  }
}

int tri_out_rows(int layers, int batch, int groups, int mode) {
  return mode == 0 ? layers * batch * groups : (mode == 1 ? batch * groups : batch);
}

hipError_t launch_tri(const TriArgs& a, hipStream_t st) {
  const int members = a.layers * a.batch * a.groups;
  const int out_rows = tri_out_rows(a.layers, a.batch, a.groups, a.mode);
  if (members == 0 || a.row_stride == 0) return hipSuccess;
  tri_stats_kernel<<<members, kTriThreads, 0, st>>>(a);
  const int nm = a.mode == 0 ? 1 : (a.mode == 1 ? a.layers : a.layers * a.groups);
  const bool vec = (a.row_stride % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.reduced) & 15) == 0;
  if (vec && nm >= 16)
    tri_reduce4_kernel<4><<<dim3((a.row_stride + 255) / 256, out_rows), kTriThreads, 0, st>>>(a);
  else if (vec)
    tri_reduce4_kernel<1><<<dim3((a.row_stride + kTriSpan - 1) / kTriSpan, out_rows), kTriThreads, 0, st>>>(a);
  else if (nm >= 16)
    tri_reduce_kernel<4><<<dim3((a.row_stride + 63) / 64, out_rows), kTriThreads, 0, st>>>(a);
  else
    tri_reduce_kernel<1><<<dim3((a.row_stride + kTriSpan - 1) / kTriSpan, out_rows), kTriThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sd
