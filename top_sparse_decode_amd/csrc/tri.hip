// tri.hip -- TriAttention selection modes: normalize the per-head score rows,
// reduce them by mode, then the library's top-k.
//
// "Add TriAttention KV-cache compression method" (Summary) puts a
// normalize/reduce step between paged-K scoring and TopK / tie settlement and
// names three eviction modes (union, per_head, per_layer_perhead); its Main
// Files name score normalization and union reduction.  The pages give no
// formula; the library computes the plain population z-score, with its sums
// taken in token order like every other reduction of the library:
//
//   per member row m = (layer, request b, KV head g), over its finite scores
//   at t < kv_len[b] (n of them), every binary64 operation rounded on its own:
//     mu   = (((0 + s_t0) + s_t1) + ...) / n, t ascending;
//     var  = (((0 + d_t0*d_t0) + d_t1*d_t1) + ...) / n, d_t = (double)s_t - mu;
//     z_t  = (float)(((double)s_t - mu) / sqrt(var)), 0 when var == 0,
//            -inf for a non-finite score or t >= kv_len[b];
//   reduced row: r_t = max over the mode's members of z_t, members visited
//   layer by layer and head by head, a later member replacing the running
//   value only when strictly larger.
//
// Kernels: tri_stats_stream_kernel (one lane per member row walks its row in
// token order, 64 rows per wave, the rows streaming through an LDS ring by
// DMA; tri_stats_kernel is the same walk for rows that are not whole 16-byte
// units) and tri_reduce_kernel /
// tri_reduce4_kernel (a token per lane, the members split into four ordered
// quarters).  Selection then runs on the reduced rows.
#include "common.h"
#include "kernels.h"

#include <math.h>

namespace sd {

constexpr int kTriThreads = 256;
constexpr int kTriSpan = 4096;  // tokens per block of the one-slice reduce

// Statistics: the sums are chains of dependent binary64 additions, one chain
// per member row, so the work is spread as one lane per row.  A wave owns
// kTriRows rows (lanes 0 .. kTriRows-1 run the chains).  Tiles of kTriTile
// tokens of those rows come in with one coalesced load per row and 64-token
// piece (lane l: token 64 i + l), sit in registers while the previous tile's
// chains run, and reach the owning lanes through LDS (row stride padded by
// one float).  Both passes read the row from memory; the second pass finds
// most of it in the last-level cache.
constexpr int kTriRows = 16;
constexpr int kTriTile = 256;
constexpr int kTriPieces = kTriTile / 64;
constexpr int kTriWaves = kTriThreads / 64;

__global__ __launch_bounds__(kTriThreads) void tri_stats_kernel(TriArgs a) {
  __shared__ float s_tile[kTriWaves][kTriRows][kTriTile + 1];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int members = a.layers * a.batch * a.groups;
  const int m0 = (blockIdx.x * kTriWaves + wid) * kTriRows;  // first row of this wave
  if (m0 >= members) return;
  const int nrows = min(kTriRows, members - m0);
  // lane r < nrows owns row m0 + r; Lr is its kv_len, Lmax the wave's longest
  int Lr = 0;
  if (lane < nrows) {
    const int m = m0 + lane;
    const int b = (m / a.groups) % a.batch;
    Lr = clamp_len(a.kv_lens[b], a.row_stride);
    if (a.lens && (m % a.groups) == 0) a.lens[m / a.groups] = a.kv_lens[b];
  }
  const int Lmax = wave_max(Lr);
  const float* base = a.scores + (int64_t)m0 * a.row_stride;
  float (*tile)[kTriTile + 1] = s_tile[wid];
  // tile loads: row r, tokens t0 + 64 i + lane (in bounds of the row; tokens
  // past the row's kv_len are loaded only if the row is that long, else -inf)
  auto load_tile = [&](int t0, float (&v)[kTriRows][kTriPieces]) {
#pragma unroll
    for (int r = 0; r < kTriRows; ++r) {
      const int Lrow = __shfl(Lr, r);
#pragma unroll
      for (int i = 0; i < kTriPieces; ++i) {
        const int t = t0 + 64 * i + lane;
        v[r][i] = (r < nrows && t < Lrow) ? base[(int64_t)r * a.row_stride + t] : -__builtin_inff();
      }
    }
  };
  auto store_tile = [&](const float (&v)[kTriRows][kTriPieces]) {
#pragma unroll
    for (int r = 0; r < kTriRows; ++r)
#pragma unroll
      for (int i = 0; i < kTriPieces; ++i) tile[r][64 * i + lane] = v[r][i];
  };
  // one pass: the chain over the row in token order; `second` selects the
  // squared deviations from mu
  auto pass = [&](bool second, double mu, int& n) -> double {
    double acc = 0.0;
    n = 0;
    float v[kTriRows][kTriPieces];
    load_tile(0, v);
    for (int t0 = 0; t0 < Lmax; t0 += kTriTile) {
      store_tile(v);
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      // the next tile's loads go out before this tile's chains run
      if (t0 + kTriTile < Lmax) load_tile(t0 + kTriTile, v);
      if (lane < nrows) {
        const int tend = min(kTriTile, Lr - t0);
        for (int j = 0; j < tend; ++j) {
          const float x = tile[lane][j];
          if (__builtin_isfinite(x)) {
            if (second) {
              const double d = __dsub_rn((double)x, mu);
              acc = __dadd_rn(acc, __dmul_rn(d, d));
            } else {
              acc = __dadd_rn(acc, (double)x);
            }
            ++n;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    return acc;
  };
  int n = 0;
  const double s1 = pass(false, 0.0, n);
  const double mu = n > 0 ? __ddiv_rn(s1, (double)n) : 0.0;
  const double s2 = pass(true, mu, n);
  if (lane < nrows) {
    const double sigma = n > 0 ? __dsqrt_rn(__ddiv_rn(s2, (double)n)) : 0.0;
    a.stats[2 * (int64_t)(m0 + lane)] = mu;
    a.stats[2 * (int64_t)(m0 + lane) + 1] = sigma;
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

// Statistics, streamed: wave w (a block of its own) owns member rows
// 64 w .. 64 w + 63, lane r the chain of row 64 w + r.  The rows come in as
// 64-token tiles (64 rows x 256 bytes, 16 KB) through a five-stage LDS ring
// by DMA (global_load_lds), the two passes back to back as one sequence of
// tiles (the second pass's loads do not depend on mu).  DMA instruction i of
// a tile moves rows 4i .. 4i+3: lane l takes 16 bytes (4 tokens) of row
// 4i + l/16 into LDS position l%16 of that row, holding data chunk
// (l%16) ^ (row%16); lane r then reads its own row four tokens at a time
// (ds_read_b128 at chunk position (j/4) ^ (r%16)): the 16 lanes of each
// 256-byte phase hit 16 different 4-bank groups.  A token past the row's
// kv_len, or not finite, adds +0.0 to the chain, which leaves every partial
// sum unchanged (a sum of binary64 values starting at +0.0 is never -0.0),
// so the chain rounds exactly as the token-order definition above.
// Requires 16-byte aligned rows (row_stride % 4 == 0, aligned pointer).
constexpr int kTsStages = 5;
constexpr int kTsTok = 64;                          // tokens per tile
constexpr int kTsTileBytes = 64 * kTsTok * 4;       // 16 KB
constexpr int kTsInsts = kTsTileBytes / 1024;       // 16 DMA instructions per tile
static_assert(kTsInsts * (kTsStages - 2) <= 63, "the DMA counter holds the tiles in flight");

// The 16 b128 reads of this lane's row in one tile (64 tokens), one wait.
__device__ __forceinline__ void ts_read_row(float4 (&v)[16], const uint32_t (&addr)[16]) {
  asm volatile(
      "ds_read_b128 %0, %16\n\tds_read_b128 %1, %17\n\tds_read_b128 %2, %18\n\tds_read_b128 %3, %19\n\t"
      "ds_read_b128 %4, %20\n\tds_read_b128 %5, %21\n\tds_read_b128 %6, %22\n\tds_read_b128 %7, %23\n\t"
      "ds_read_b128 %8, %24\n\tds_read_b128 %9, %25\n\tds_read_b128 %10, %26\n\tds_read_b128 %11, %27\n\t"
      "ds_read_b128 %12, %28\n\tds_read_b128 %13, %29\n\tds_read_b128 %14, %30\n\tds_read_b128 %15, %31\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
        "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
      : "v"(addr[0]), "v"(addr[1]), "v"(addr[2]), "v"(addr[3]), "v"(addr[4]), "v"(addr[5]), "v"(addr[6]),
        "v"(addr[7]), "v"(addr[8]), "v"(addr[9]), "v"(addr[10]), "v"(addr[11]), "v"(addr[12]), "v"(addr[13]),
        "v"(addr[14]), "v"(addr[15])
      : "memory");
}

__global__ __launch_bounds__(64) void tri_stats_stream_kernel(TriArgs a) {
  __shared__ __attribute__((aligned(1024))) float s_ring[kTsStages][64 * kTsTok];
  const int lane = threadIdx.x;
  const int members = a.layers * a.batch * a.groups;
  const int m0 = blockIdx.x * 64;
  const int nrows = min(64, members - m0);
  int Lr = 0;
  if (lane < nrows) {
    const int m = m0 + lane;
    const int b = (m / a.groups) % a.batch;
    Lr = clamp_len(a.kv_lens[b], a.row_stride);
    if (a.lens && (m % a.groups) == 0) a.lens[m / a.groups] = a.kv_lens[b];
  }
  const int Lmax = wave_max(Lr);
  const int ntiles = (Lmax + kTsTok - 1) / kTsTok;
  const int nseq = 2 * ntiles;  // both passes
  // DMA slots of this lane: instruction i, row 4i + l/16 (rows past the
  // wave's last read row 0), data chunk (l%16) ^ (row%16)
  const int prow = lane >> 4, ppos = lane & 15;
  const float* rbase = a.scores + (int64_t)m0 * a.row_stride;
  const uint32_t ring0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)s_ring;
  auto issue = [&](int k) __attribute__((always_inline)) {  // tile k of the sequence into stage k % S
    const int T = k < ntiles ? k : k - ntiles;
    const uint32_t dst = ring0 + (uint32_t)((k % kTsStages) * kTsTileBytes);
#pragma unroll
    for (int i = 0; i < kTsInsts; ++i) {
      const int r = 4 * i + prow;
      const int rr = r < nrows ? r : 0;
      const int c = ppos ^ (r & 15);
      // 16 bytes inside the row: tiles stop at the wave's longest kv_len <= row_stride,
      // and row_stride is a whole number of 4-token chunks
      const int t = min(kTsTok * T + 4 * c, a.row_stride - 4);
      __builtin_amdgcn_global_load_lds(rbase + (int64_t)rr * a.row_stride + t,
                                       (__attribute__((address_space(3))) void*)(uintptr_t)(dst + 1024u * i), 16, 0,
                                       kLoadStream);
    }
  };
  uint32_t raddr[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) raddr[q] = ring0 + (uint32_t)(lane * 256 + 16 * (q ^ (lane & 15)));

  for (int k = 0; k < min(nseq, kTsStages - 1); ++k) issue(k);
  double acc = 0.0, mu = 0.0;
  int n = 0;
  for (int k = 0; k < nseq; ++k) {
    const int ahead = min(nseq - 1 - k, kTsStages - 2);  // later tiles in flight
    if (ahead >= 3) asm volatile("s_waitcnt vmcnt(48)" ::: "memory");
    else if (ahead == 2) asm volatile("s_waitcnt vmcnt(32)" ::: "memory");
    else if (ahead == 1) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    float4 v[16];
    uint32_t ra[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) ra[q] = raddr[q] + (uint32_t)((k % kTsStages) * kTsTileBytes);
    ts_read_row(v, ra);
    // the stage just read is free: the tile S - 1 ahead goes there
    if (k + kTsStages - 1 < nseq) issue(k + kTsStages - 1);
    const bool second = k >= ntiles;  // (wave-uniform)
    const int t0 = kTsTok * (second ? k - ntiles : k);
    if (k == ntiles) {  // first pass done
      mu = n > 0 ? __ddiv_rn(acc, (double)n) : 0.0;
      acc = 0.0;
    }
    // this lane's 64 values; a token past kv_len reads as NaN (only in the
    // tile that crosses it), so that "finite" alone decides what counts
    float xv[64];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      xv[4 * q] = v[q].x;
      xv[4 * q + 1] = v[q].y;
      xv[4 * q + 2] = v[q].z;
      xv[4 * q + 3] = v[q].w;
    }
    if (__builtin_amdgcn_ballot_w64(t0 + kTsTok > Lr) != 0) {
#pragma unroll
      for (int j = 0; j < 64; ++j) xv[j] = t0 + j < Lr ? xv[j] : __builtin_nanf("");
    }
    // groups of 16 values, kept apart so that their masks do not all live at once
    if (!second) {
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        const bool ok = __builtin_isfinite(xv[j]);
        acc = __dadd_rn(acc, (double)(ok ? xv[j] : 0.0f));
        n += ok;
        if ((j & 15) == 15) __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 64; ++j) {
        const double d = __dsub_rn((double)xv[j], mu);
        const double dd = __dmul_rn(d, d);
        acc = __dadd_rn(acc, __builtin_isfinite(xv[j]) ? dd : 0.0);
        if ((j & 15) == 15) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  if (ntiles == 0) mu = 0.0;
  if (lane < nrows) {
    const double sigma = n > 0 ? __dsqrt_rn(__ddiv_rn(acc, (double)n)) : 0.0;
    a.stats[2 * (int64_t)(m0 + lane)] = mu;
    a.stats[2 * (int64_t)(m0 + lane) + 1] = sigma;
  }
}

hipError_t launch_tri(const TriArgs& a, hipStream_t st) {
  const int members = a.layers * a.batch * a.groups;
  const int out_rows = tri_out_rows(a.layers, a.batch, a.groups, a.mode);
  if (members == 0 || a.row_stride == 0) return hipSuccess;
  const bool rows16 = (a.row_stride % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0;
  if (rows16) {
    tri_stats_stream_kernel<<<(members + 63) / 64, 64, 0, st>>>(a);
  } else {
    const int stat_blocks = (members + kTriWaves * kTriRows - 1) / (kTriWaves * kTriRows);
    tri_stats_kernel<<<stat_blocks, kTriThreads, 0, st>>>(a);
  }
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
