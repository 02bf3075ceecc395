// tri.hip -- TriAttention selection modes: normalize the per-head score rows,
// reduce them by mode, then the library's top-k.
//
// "Add TriAttention KV-cache compression method" (Summary) puts a
// normalize/reduce step between paged-K scoring and TopK / tie settlement and
// names three eviction modes (union, per_head, per_layer_perhead); its Main
// Files name score normalization and union reduction.  The pages give no
// formula; the library computes the plain population z-score with exactly
// rounded sums (no order of summation enters the result):
//
//   per member row m = (layer, request b, KV head g), over its finite scores
//   at t < kv_len[b] (n of them), every binary64 operation rounded on its own:
//     mu   = S1 / n, S1 = the exact sum of the scores rounded once to binary64;
//     var  = S2 / n, S2 = the same for the d_t * d_t, d_t = (double)s_t - mu;
//     z_t  = (float)(((double)s_t - mu) / sqrt(var)), 0 when var == 0,
//            -inf for a non-finite score or t >= kv_len[b];
//   reduced row: r_t = max over the mode's members of z_t, members visited
//   layer by layer and head by head, a later member replacing the running
//   value only when strictly larger.
//
// Kernels: tri_stats_kernel (one block per member row, the sums split over
// exact grids so that the tokens are summed in parallel; per layer and head
// it also writes the member's z row and/or selects from it) and
// tri_reduce_kernel / tri_reduce4_kernel (a token per lane, the members split
// into ordered slices whose maxima meet in order).  Selection then runs on
// the reduced rows.
#include "common.h"
#include "kernels.h"
#include "wave_select.h"

#include <math.h>
#include <stdlib.h>

#include <type_traits>

namespace sd {

constexpr int kTriThreads = 256;
constexpr int kTriSpan = 4096;  // tokens per block of the one-slice reduce

// Statistics.  Both sums are exactly rounded, so their terms may be added in
// any order: a member row is spread over one block (thread c of its T
// threads holds tokens 4 (c + T i) .. +3 when the row is held in registers),
// and the partial sums meet in any order.  The error-free extraction of Rump,
// Ogita and Oishi splits a term over a fixed grid: with sigma = 1.5 * 2^k and
// |v| < 2^(k-1), h = (v + sigma) - sigma is v rounded to a multiple of
// G = 2^(k-52), and v - h is exact.  k comes from a bound M on |v| (from the
// row's extremes) and the term count n: k = log2 M + 1 + ceil(log2 n), so
// every partial sum of the h of one grid is a multiple of G below 2^53 G,
// hence exact in any order, across lanes and waves too.
//  * S1 (the scores): one grid first; binary32 scores within about 2^15 of
//    the largest are taken whole, and only where some term is not does a
//    second pass add a second grid 2^(51 - ceil(log2 n)) finer, whose
//    leftovers are at most half its step each.
//  * S2 (the squared deviations): one grid exactly (A1) plus its leftovers,
//    each at most G1 / 2, in plain binary64 (R1), which is within
//    E = n^2 G1 2^-54 (1 + 2^-18) of their exact sum in any order.
//  * The final rounding (round_two): s = RN(A1 + A2) (or A1 + R1) stands
//    when s is not a power of two and its exact TwoSum error plus the
//    leftover bound stays below half of s's last place; else S2 takes the
//    second grid exactly too, and both decide by the 128-bit integer form
//    (the grids' sum T in units of the finer grid: RN(T - n/2) = RN(T + n/2)).
//  * A row where that fails too (scores spanning more than about 2^54, or a
//    sum within about 2^-21 of a rounding midpoint), and every row when
//    asked, is summed in a long accumulator of 64-bit words spanning all of
//    binary64 (word w in lane w), exact for any input.
constexpr int kLongWords = 35;  // bit 0 = 2^-1074; 2240 bits hold 2^31 terms of any binary64 magnitude

// shared state of a row's block of W waves
template <int W>
struct TsShared {
  int n[W];
  float vmax[W], vmin[W];
  double part1[W][2], part2[W][2];
  int rest1[W], rest1b[W], rest2[W];
  uint64_t words[W][4][kLongWords];  // per wave: positive words, their carries, negative words, carries
  uint64_t tot[2][kLongWords];
  double sum;
};

__device__ __forceinline__ int ceil_log2(int n) { return n <= 1 ? 0 : 32 - __clz(n - 1); }

// e with v < 2^(e+1) for a finite v > 0 (floor(log2 v) for a normal v)
__device__ __forceinline__ int exponent_bound(double v) {
  return (int)(((uint64_t)__double_as_longlong(v) >> 52) & 0x7FF) - 1023;
}

// one grid of the extraction: v rounded to a multiple of the grid of sigma
__device__ __forceinline__ double grid_part(double v, double sigma) { return __dsub_rn(__dadd_rn(v, sigma), sigma); }

// The nearest binary64 to mag * 2^e, ties to even.  The callers' values lie
// in binary64's normal range.
__device__ double round_mag(unsigned __int128 mag, int e) {
  if (mag == 0) return 0.0;
  const uint64_t hi = (uint64_t)(mag >> 64), lo = (uint64_t)mag;
  const int p = hi ? 127 - __clzll((long long)hi) : 63 - __clzll((long long)lo);  // top bit
  if (p <= 52) return ldexp((double)lo, e);
  const int sh = p - 52;
  uint64_t mant = (uint64_t)(mag >> sh);
  const unsigned __int128 rem = mag & (((unsigned __int128)1 << sh) - 1);
  const unsigned __int128 half = (unsigned __int128)1 << (sh - 1);
  if (rem > half || (rem == half && (mant & 1))) ++mant;  // 2^53 is still exact
  return ldexp((double)mant, e + sh);
}

__device__ double round_int(__int128 v, int e) {
  if (v < 0) return -round_mag((unsigned __int128)(-v), e);
  return round_mag((unsigned __int128)v, e);
}

// The exactly rounded sum from two grids: A1, A2 multiples of G1 = G2 2^s
// and G2 = 2^g2 below 2^53 of their steps, plus a remainder of at most
// n G2 / 2 when `rest`.  False when the remainder could change the rounding.
__device__ bool round_two(double A1, double A2, int g2, int s, bool rest, int n, double& out) {
  // A1 + A2 rounded once is the exactly rounded total when nothing is left
  const double sum = __dadd_rn(A1, A2);
  if (!rest) {
    out = sum;
    return true;
  }
  // with a remainder R, |R| <= r G2: sum + e (e from TwoSum, exact) is
  // A1 + A2, and sum stands when |e| + r G2 stays below half its gap to
  // either neighbour (a power of two, with its closer lower neighbour, and
  // anything near that bound take the integer form below)
  const int64_t r = (n + 1) / 2;
  {
    const double bb = __dsub_rn(sum, A1);
    const double e = __dadd_rn(__dsub_rn(A1, __dsub_rn(sum, bb)), __dsub_rn(A2, bb));
    const uint64_t sb = (uint64_t)__double_as_longlong(sum);
    const int ex = (int)((sb >> 52) & 0x7FF);
    if (sum != 0.0 && (sb & ((1ull << 52) - 1)) != 0 && ex > 53) {
      const double half_ulp = ldexp(1.0, ex - 1023 - 53);
      const double lhs = __dadd_rn(fabs(e), ldexp((double)r, g2));  // within a relative 2^-53 of the exact
      if (lhs <= half_ulp * (1.0 - 0x1p-40)) {
        out = sum;
        return true;
      }
    }
  }
  const int64_t a1 = (int64_t)ldexp(A1, -(g2 + s));  // integers of at most 53 bits: exact
  const int64_t a2 = (int64_t)ldexp(A2, -g2);
  const __int128 T = ((__int128)a1 << s) + a2;
  out = round_int(T - r, g2);
  return out == round_int(T + r, g2);
}

// Long accumulation: lane w holds word w of the positive terms' magnitudes
// and of the negative terms', and the carries out of them.
struct TsLong {
  uint64_t p, n;
  uint64_t cp, cn;
};

// adds the binary64 term with the given bits (the same in every lane)
__device__ __forceinline__ void long_add(TsLong& acc, uint64_t bits, int lane) {
  const int ef = (int)((bits >> 52) & 0x7FF);
  const uint64_t m = (bits & ((1ull << 52) - 1)) | (ef ? (1ull << 52) : 0);
  const int pos = (ef ? ef : 1) - 1;  // m's lowest bit stands for 2^(pos - 1074)
  const int wi = pos >> 6, sh = pos & 63;
  const uint64_t lo = m << sh, hi = (m >> 1) >> (63 - sh);
  const uint64_t add = lane == wi ? lo : (lane == wi + 1 ? hi : 0);
  const bool neg = (bits >> 63) != 0;
  const uint64_t op = acc.p, on = acc.n;
  acc.p = op + (neg ? 0 : add);
  acc.n = on + (neg ? add : 0);
  acc.cp += acc.p < op ? 1 : 0;
  acc.cn += acc.n < on ? 1 : 0;
}

// Thread 0: the waves' words summed with their carries, the difference of
// the positive and negative totals rounded to the nearest binary64.
template <int W>
__device__ double long_round(TsShared<W>& sh) {
  for (int sgn = 0; sgn < 2; ++sgn) {
    unsigned __int128 carry = 0;
    for (int w = 0; w < kLongWords; ++w) {
      unsigned __int128 t = carry;
      for (int v = 0; v < W; ++v) {
        t += sh.words[v][2 * sgn][w];
        if (w > 0) t += sh.words[v][2 * sgn + 1][w - 1];
      }
      sh.tot[sgn][w] = (uint64_t)t;
      carry = t >> 64;
    }
  }
  int cmp = 0;
  for (int w = kLongWords - 1; w >= 0 && cmp == 0; --w)
    if (sh.tot[0][w] != sh.tot[1][w]) cmp = sh.tot[0][w] > sh.tot[1][w] ? 1 : -1;
  if (cmp == 0) return 0.0;
  uint64_t* big = sh.tot[cmp > 0 ? 0 : 1];
  const uint64_t* small = sh.tot[cmp > 0 ? 1 : 0];
  uint64_t borrow = 0;
  for (int w = 0; w < kLongWords; ++w) {
    const uint64_t x = big[w], y = small[w];
    big[w] = x - y - borrow;
    borrow = (x < y || (x == y && borrow)) ? 1 : 0;
  }
  int top = -1;
  for (int w = kLongWords - 1; w >= 0 && top < 0; --w)
    if (big[w]) top = 64 * w + 63 - __clzll((long long)big[w]);
  double mag;
  if (top <= 52) {
    mag = ldexp((double)big[0], -1074);
  } else {
    const int q = top - 52;  // lowest kept bit
    const int wq = q >> 6, bq = q & 63;
    uint64_t mant = big[wq] >> bq;
    if (bq) mant |= big[wq + 1] << (64 - bq);
    mant &= (1ull << 53) - 1;
    const int rb = q - 1;
    const bool round = (big[rb >> 6] >> (rb & 63)) & 1;
    bool sticky = (big[rb >> 6] & ((1ull << (rb & 63)) - 1)) != 0;
    for (int w = 0; w < (rb >> 6) && !sticky; ++w) sticky = big[w] != 0;
    if (round && (sticky || (mant & 1))) ++mant;
    mag = ldexp((double)mant, q - 1074);
  }
  return cmp > 0 ? mag : -mag;
}

// z of a score from its member's mu, sigma and rinv = RN(1 / sigma): the
// binary64 quotient (s - mu) / sigma, correctly rounded, then rounded to
// binary32.  q = (s - mu) * rinv is within 2.5 binary64 ulps of that quotient
// (two roundings of relative size 2^-53 each, plus the quotient's own half
// ulp), so q rounds to the same binary32 unless it lies within 3 ulps of a
// binary32 rounding midpoint (its 29 bits below binary32's last place within
// 3 of 2^28) or below binary32's normal range; those few take the division.
// Binade edges are binary32 values, far from any midpoint, so they need no
// care.
__device__ __forceinline__ float tri_z(float s, double mu, double sigma, double rinv) {
  if (!__builtin_isfinite(s)) return -__builtin_inff();
  if (sigma == 0.0) return 0.0f;
  const double d = __dsub_rn((double)s, mu);
  const double q = __dmul_rn(d, rinv);
  const uint64_t b = (uint64_t)__double_as_longlong(q);
  const uint32_t low = (uint32_t)b & 0x1FFFFFFFu;
  const uint32_t ex = (uint32_t)(b >> 52) & 0x7FFu;
  if (low - ((1u << 28) - 3u) > 6u && ex >= 1023u - 126u) return __double2float_rn(q);
  return __double2float_rn(__ddiv_rn(d, sigma));
}

// The same z without the division: `exact` is set where the product is not
// safe (near a binary32 midpoint or tiny); the caller then uses tri_z.
__device__ __forceinline__ float tri_z_product(float s, double mu, double sigma, double rinv, bool& exact) {
  exact = false;
  if (!__builtin_isfinite(s)) return -__builtin_inff();
  if (sigma == 0.0) return 0.0f;
  const double q = __dmul_rn(__dsub_rn((double)s, mu), rinv);
  const uint64_t b = (uint64_t)__double_as_longlong(q);
  const uint32_t low = (uint32_t)b & 0x1FFFFFFFu;
  const uint32_t ex = (uint32_t)(b >> 52) & 0x7FFu;
  exact = !(low - ((1u << 28) - 3u) > 6u && ex >= 1023u - 126u);
  return __double2float_rn(q);
}

template <bool B>
struct TsFlag {
  static constexpr bool value = B;
};

// The statistics of member row m, by a block of W waves (every thread takes
// part).  NV > 0: the row is in xv, NV 16-byte units per thread; NV == 0:
// every pass reads the row again.  With one wave the partial results meet
// in registers alone.
template <int NV, int W, bool ZROWS, bool SEL>
__device__ __forceinline__ void tri_stats_row(const TriArgs& a, TsShared<W>& sh, int m, int kv_len,
                                              float (&xv)[NV > 0 ? 4 * NV : 1],
                                              WaveSelectSmem<(SEL && NV > 0 ? NV : 1)>& ssel) {
  constexpr int T = 64 * W;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int Lr = clamp_len(kv_len, a.row_stride);
  if (threadIdx.x == 0 && a.lens && (m % a.groups) == 0) a.lens[m / a.groups] = kv_len;
  const float* row = a.scores + (int64_t)m * a.row_stride;
  const float nan = __builtin_nanf("");
  if constexpr (NV > 0) {
    // tokens at or past kv_len read as NaN, so that "finite" alone decides
    // what counts (units wholly past it were never loaded)
    if (Lr < 4 * NV * T) {
#pragma unroll
      for (int j = 0; j < 4 * NV; ++j)
        if (4 * (threadIdx.x + T * (j / 4)) + j % 4 >= Lr) xv[j] = nan;
    }
  }
  // every token of the thread (a wave-uniform trip count)
  auto each = [&](auto&& body) __attribute__((always_inline)) {
    if constexpr (NV > 0) {
#pragma unroll
      for (int j = 0; j < 4 * NV; ++j) body(xv[j]);
    } else {
      for (int t0 = 64 * wid; t0 < Lr; t0 += T) {
        const int t = t0 + lane;
        body(t < Lr ? row[t] : nan);
      }
    }
  };
  // the exact sum of term(x) over the row by long accumulation (every thread gets it)
  auto long_sum = [&](auto&& term) __attribute__((always_inline)) -> double {
    TsLong acc{0, 0, 0, 0};
    each([&](float x) {
      const double v = term(x);
      const uint64_t bits = (uint64_t)__double_as_longlong(v);
      uint64_t live = __builtin_amdgcn_ballot_w64(v != 0.0);
      while (live) {
        const int j = __builtin_ctzll(live);
        live &= live - 1;
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)bits, j);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(bits >> 32), j);
        long_add(acc, ((uint64_t)hi << 32) | lo, lane);
      }
    });
    if (lane < kLongWords) {
      sh.words[wid][0][lane] = acc.p;
      sh.words[wid][1][lane] = acc.cp;
      sh.words[wid][2][lane] = acc.n;
      sh.words[wid][3][lane] = acc.cn;
    }
    __syncthreads();
    if (threadIdx.x == 0) sh.sum = long_round(sh);
    __syncthreads();
    return sh.sum;
  };

  // count and extremes of the finite scores (maxima skip NaN; an infinite
  // score sends them to a second look that skips it)
  int n = 0;
  float vmax = -__builtin_inff(), vmin = __builtin_inff();
  each([&](float x) {
    n += __builtin_popcountll(__builtin_amdgcn_ballot_w64(__builtin_isfinite(x)));  // per wave
    vmax = fmaxf(vmax, x);
    vmin = fminf(vmin, x);
  });
  vmax = wave_max(vmax);
  vmin = -wave_max(-vmin);
  if constexpr (W > 1) {
    if (lane == 0) {
      sh.n[wid] = n;
      sh.vmax[wid] = vmax;
      sh.vmin[wid] = vmin;
    }
    __syncthreads();
    n = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      n += sh.n[w];
      vmax = fmaxf(vmax, sh.vmax[w]);
      vmin = fminf(vmin, sh.vmin[w]);
    }
  }
  if (n > 0 && (vmax == __builtin_inff() || vmin == -__builtin_inff())) {
    if constexpr (W > 1) __syncthreads();  // every thread has read the slots
    vmax = -__builtin_inff();
    vmin = __builtin_inff();
    each([&](float x) {
      const bool ok = __builtin_isfinite(x);
      vmax = ok ? fmaxf(vmax, x) : vmax;
      vmin = ok ? fminf(vmin, x) : vmin;
    });
    vmax = wave_max(vmax);
    vmin = -wave_max(-vmin);
    if constexpr (W > 1) {
      if (lane == 0) {
        sh.vmax[wid] = vmax;
        sh.vmin[wid] = vmin;
      }
      __syncthreads();
#pragma unroll
      for (int w = 0; w < W; ++w) {
        vmax = fmaxf(vmax, sh.vmax[w]);
        vmin = fminf(vmin, sh.vmin[w]);
      }
    }
  }
  // every token of every thread present and finite: no selects below
  const bool all_live = NV > 0 && n == 4 * NV * T;
  const bool force_long = a.exact_slow != 0;
  const int c = ceil_log2(n);
  double mu = 0.0, sigma = 0.0;
  if (n > 0) {
    // S1: the exactly rounded sum of the finite scores
    auto val = [&](float x) __attribute__((always_inline)) { return __builtin_isfinite(x) ? (double)x : 0.0; };
    double s1 = 0.0;
    const double amax = fmax(fabs((double)vmax), fabs((double)vmin));
    if (amax != 0.0) {
      const int k1 = exponent_bound(amax) + 2 + c, k2 = k1 - 51 + c;
      bool done = false;
      if (!force_long && k2 - 52 >= -1022) {
        const double g1 = ldexp(1.5, k1), g2 = ldexp(1.5, k2);
        // the first grid alone: binary32 scores within about 2^15 of the
        // largest are taken whole by it; the second grid only where some
        // term is not (a second pass over the registers)
        double A1 = 0.0, A2 = 0.0;
        bool rem = false, rest = false;
        auto pass1 = [&](auto live) __attribute__((always_inline)) {
          each([&](float x) {
            const double v = decltype(live)::value ? (double)x : val(x);
            const double h1 = grid_part(v, g1);
            A1 = __dadd_rn(A1, h1);
            rem = rem || v != h1;
          });
        };
        auto pass2 = [&](auto live) __attribute__((always_inline)) {
          each([&](float x) {
            const double v = decltype(live)::value ? (double)x : val(x);
            const double h1 = grid_part(v, g1), l1 = __dsub_rn(v, h1);
            const double h2 = grid_part(l1, g2);
            A2 = __dadd_rn(A2, h2);
            rest = rest || l1 != h2;
          });
        };
        if (all_live) pass1(TsFlag<true>{});
        else pass1(TsFlag<false>{});
        A1 = wave_sum(A1);
        bool brem = __builtin_amdgcn_ballot_w64(rem) != 0;
        if constexpr (W > 1) {
          if (lane == 0) {
            sh.part1[wid][0] = A1;
            sh.rest1[wid] = brem;
          }
          __syncthreads();
          A1 = 0.0;
          brem = false;
#pragma unroll
          for (int w = 0; w < W; ++w) {
            A1 = __dadd_rn(A1, sh.part1[w][0]);
            brem = brem || sh.rest1[w] != 0;
          }
        }
        bool brest = false;
        if (brem) {
          if (all_live) pass2(TsFlag<true>{});
          else pass2(TsFlag<false>{});
          A2 = wave_sum(A2);
          brest = __builtin_amdgcn_ballot_w64(rest) != 0;
          if constexpr (W > 1) {
            if (lane == 0) {
              sh.part1[wid][1] = A2;
              sh.rest1b[wid] = brest;
            }
            __syncthreads();
            A2 = 0.0;
            brest = false;
#pragma unroll
            for (int w = 0; w < W; ++w) {
              A2 = __dadd_rn(A2, sh.part1[w][1]);
              brest = brest || sh.rest1b[w] != 0;
            }
          }
        }
        done = round_two(A1, A2, k2 - 52, 51 - c, brest, n, s1);
      }
      if (!done) s1 = long_sum(val);
    }
    mu = __ddiv_rn(s1, (double)n);
    // S2: the exactly rounded sum of RN(RN(x - mu)^2); its largest term is
    // that of an extreme score (both roundings are monotone)
    auto sq = [&](float x) __attribute__((always_inline)) {
      const double d = __dsub_rn((double)x, mu);
      return __builtin_isfinite(x) ? __dmul_rn(d, d) : 0.0;
    };
    double s2 = 0.0;
    const double dmax = fmax(fabs(__dsub_rn((double)vmax, mu)), fabs(__dsub_rn((double)vmin, mu)));
    const double ddmax = __dmul_rn(dmax, dmax);
    if (ddmax != 0.0) {
      const int k1 = exponent_bound(ddmax) + 2 + c, k2 = k1 - 51 + c;
      bool done = false;
      if (!force_long && k2 - 52 >= -1022) {
        const double g1 = ldexp(1.5, k1), g2 = ldexp(1.5, k2);
        auto term = [&](auto live, float x) __attribute__((always_inline)) {
          if constexpr (decltype(live)::value) {
            const double d = __dsub_rn((double)x, mu);
            return __dmul_rn(d, d);
          } else {
            return sq(x);
          }
        };
        // The first grid exactly (A1) and what it leaves summed in plain
        // binary64 (R1): every leftover is at most G1 / 2, so R1 is within
        // E = gamma_{n-1} n G1 / 2 <= n^2 G1 2^-54 (1 + 2^-18) of their exact
        // sum, in any order.  With s = RN(A1 + R1) and e its exact TwoSum
        // error, the total lies within |e| + E of s: s stands when that is
        // below half of s's last place (s not a power of two).  Otherwise the
        // second grid is taken exactly.
        {
          double A1 = 0.0, R1 = 0.0;
          auto pass1 = [&](auto live) __attribute__((always_inline)) {
            each([&](float x) {
              const double v = term(live, x);
              const double h1 = grid_part(v, g1);
              A1 = __dadd_rn(A1, h1);
              R1 = __dadd_rn(R1, __dsub_rn(v, h1));
            });
          };
          if (all_live) pass1(TsFlag<true>{});
          else pass1(TsFlag<false>{});
          A1 = wave_sum(A1);
          R1 = wave_sum(R1);
          if constexpr (W > 1) {
            if (lane == 0) {
              sh.part2[wid][0] = A1;
              sh.part2[wid][1] = R1;
            }
            __syncthreads();
            A1 = R1 = 0.0;
#pragma unroll
            for (int w = 0; w < W; ++w) {
              A1 = __dadd_rn(A1, sh.part2[w][0]);
              R1 = __dadd_rn(R1, sh.part2[w][1]);
            }
            __syncthreads();  // the slots are read again below
          }
          const double sum = __dadd_rn(A1, R1);
          const double bb = __dsub_rn(sum, A1);
          const double e = __dadd_rn(__dsub_rn(A1, __dsub_rn(sum, bb)), __dsub_rn(R1, bb));
          const uint64_t sb = (uint64_t)__double_as_longlong(sum);
          const int ex = (int)((sb >> 52) & 0x7FF);
          if (sum != 0.0 && (sb & ((1ull << 52) - 1)) != 0 && ex > 53 && n <= (1 << 26)) {
            const double E = ldexp((double)n * (double)n, k1 - 52 - 54) * (1.0 + 0x1p-18);
            const double lhs = __dadd_rn(fabs(e), E);
            if (lhs <= ldexp(1.0, ex - 1023 - 53) * (1.0 - 0x1p-40)) {
              s2 = sum;
              done = true;
            }
          }
        }
        double A1 = 0.0, A2 = 0.0;
        bool brest = false;
        if (!done) {
          bool rest = false;
          auto pass = [&](auto live) __attribute__((always_inline)) {
            each([&](float x) {
              const double v = term(live, x);
              const double h1 = grid_part(v, g1), l1 = __dsub_rn(v, h1);
              const double h2 = grid_part(l1, g2);
              A1 = __dadd_rn(A1, h1);
              A2 = __dadd_rn(A2, h2);
              rest = rest || l1 != h2;
            });
          };
          if (all_live) pass(TsFlag<true>{});
          else pass(TsFlag<false>{});
          A1 = wave_sum(A1);
          A2 = wave_sum(A2);
          brest = __builtin_amdgcn_ballot_w64(rest) != 0;
          if constexpr (W > 1) {
            if (lane == 0) {
              sh.part2[wid][0] = A1;
              sh.part2[wid][1] = A2;
              sh.rest2[wid] = brest;
            }
            __syncthreads();
            A1 = A2 = 0.0;
            brest = false;
#pragma unroll
            for (int w = 0; w < W; ++w) {
              A1 = __dadd_rn(A1, sh.part2[w][0]);
              A2 = __dadd_rn(A2, sh.part2[w][1]);
              brest = brest || sh.rest2[w] != 0;
            }
          }
          done = round_two(A1, A2, k2 - 52, 51 - c, brest, n, s2);
        }
      }
      if (!done) s2 = long_sum(sq);
    }
    sigma = __dsqrt_rn(__ddiv_rn(s2, (double)n));
  }
  const double rinv = sigma > 0.0 ? __ddiv_rn(1.0, sigma) : 0.0;
  if (threadIdx.x == 0) {
    a.stats[4 * (int64_t)m] = mu;
    a.stats[4 * (int64_t)m + 1] = sigma;
    a.stats[4 * (int64_t)m + 2] = rinv;
  }
  if constexpr (NV > 0 && ZROWS) {
    // per layer and head the reduced row is the member's own z: written from
    // the registers (reduced rows 16-byte aligned, row_stride % 4 == 0)
    {
      float* out = a.reduced + (int64_t)m * a.row_stride;
      // the product form first; a lane with any unsafe product writes its
      // row again with the division (rare)
      bool slow = false;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int t = 4 * (threadIdx.x + T * i);
        bool e0, e1, e2, e3;
        const float4 z = make_float4(tri_z_product(xv[4 * i], mu, sigma, rinv, e0),
                                     tri_z_product(xv[4 * i + 1], mu, sigma, rinv, e1),
                                     tri_z_product(xv[4 * i + 2], mu, sigma, rinv, e2),
                                     tri_z_product(xv[4 * i + 3], mu, sigma, rinv, e3));
        slow = slow || e0 || e1 || e2 || e3;
        if (t < a.row_stride) *reinterpret_cast<float4*>(out + t) = z;
      }
      if (__builtin_amdgcn_ballot_w64(slow) != 0 && slow) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int t = 4 * (threadIdx.x + T * i);
          if (t < a.row_stride)
            *reinterpret_cast<float4*>(out + t) =
                make_float4(tri_z(xv[4 * i], mu, sigma, rinv), tri_z(xv[4 * i + 1], mu, sigma, rinv),
                            tri_z(xv[4 * i + 2], mu, sigma, rinv), tri_z(xv[4 * i + 3], mu, sigma, rinv));
        }
      }
    }
  }
  if constexpr (NV > 0 && W == 1 && SEL) {
    // per layer and head, the member's selection from the z it has just
    // formed (the lanes hold positions as the one-wave selection expects)
    {
      const int k = a.sel_k;
      int32_t* out = a.sel_indices + (int64_t)m * k;
      if (Lr <= k) {
        for (int i = lane; i < k; i += 64) out[i] = i < Lr ? i : -1;
        if (a.sel_counts && lane == 0) a.sel_counts[m] = Lr;
      } else {
        uint32_t key[NV][4];
        uint32_t kmin1 = 0xFFFFFFFFu, kmax = 0u;
        bool slow = false;  // some element's z needs the division (rare)
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bool ex;
            const float z = tri_z_product(xv[4 * i + e], mu, sigma, rinv, ex);
            slow = slow || ex;
            key[i][e] = max(wave_key(z), 1u);
          }
        if (__builtin_amdgcn_ballot_w64(slow) != 0 && slow) {
          // such a lane forms all its z again with the division, reading its
          // scores again (each below kv_len; the others are not used)
#pragma unroll
          for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = 4 * (lane + 64 * i) + e;
              if (t < Lr) key[i][e] = max(wave_key(tri_z(row[t], mu, sigma, rinv)), 1u);
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 4 * (lane + 64 * i) + e;
            uint32_t kk = t < Lr ? key[i][e] : 0u;
            asm volatile("" : "+v"(kk));  // the scores are not kept beside their keys
            key[i][e] = kk;
            kmin1 = min(kmin1, kk - 1u);
            kmax = max(kmax, kk);
          }
        const uint32_t kmin = uniform_u32(wave_min_u32(kmin1)) + 1u;
        kmax = uniform_u32(wave_max_u32(kmax));
        wave_select<NV>(key, kmin, kmax, k, out, nullptr, ssel);
        if (a.sel_counts && lane == 0) a.sel_counts[m] = k;
      }
    }
  }
}

// Row m into registers: thread c of the T = 64 W takes tokens
// 4 (c + T i) .. +3 when the unit starts below kv_len (others hold NaN).
// Rows of at most 4 T NV tokens, 16-byte aligned, row_stride % 4 == 0.
template <int NV, int W>
__device__ __forceinline__ void tri_load_row(const TriArgs& a, int m, int kv_len, float (&xv)[4 * NV]) {
  constexpr int T = 64 * W;
  const int Lr = clamp_len(kv_len, a.row_stride);
  const float* row = a.scores + (int64_t)m * a.row_stride;
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int t = 4 * (threadIdx.x + T * i);
    float4 q = make_float4(nan, nan, nan, nan);
    if (t < Lr) q = *reinterpret_cast<const float4*>(row + t);  // t + 3 < row_stride
    xv[4 * i] = q.x;
    xv[4 * i + 1] = q.y;
    xv[4 * i + 2] = q.z;
    xv[4 * i + 3] = q.w;
  }
}

__device__ __forceinline__ int tri_kv_len(const TriArgs& a, int m) { return a.kv_lens[(m / a.groups) % a.batch]; }

// One block of W waves per member row.  NV > 0: the row is held in
// registers (NV 16-byte units per thread); NV == 0: read again in every pass.
// ZROWS: also the member's z row (per layer and head); SEL: also its
// selection (per layer and head, one wave per row).  Separate instances, so
// that the plain statistics keep their registers.
template <int NV, int W, bool ZROWS = false, bool SEL = false>
__global__ __launch_bounds__(64 * W) void tri_stats_kernel(TriArgs a) {
  __shared__ TsShared<W> sh;
  __shared__ WaveSelectSmem<(SEL && NV > 0 ? NV : 1)> ssel;
  const int len = tri_kv_len(a, blockIdx.x);
  if constexpr (NV > 0) {
    float cur[4 * NV];
    tri_load_row<NV, W>(a, blockIdx.x, len, cur);
    tri_stats_row<NV, W, ZROWS, SEL>(a, sh, blockIdx.x, len, cur, ssel);
  } else {
    float none[1] = {0.0f};
    tri_stats_row<0, W, false, false>(a, sh, blockIdx.x, len, none, ssel);
  }
}

bool tri_fuses_select(const TriArgs& a) {
  return a.mode == 0 && (a.row_stride % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 &&
         a.row_stride <= 4096;
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
        const float z = tri_z(x[u], a.stats[4 * m[u]], a.stats[4 * m[u] + 1], a.stats[4 * m[u] + 2]);
        if (z > r) r = z;
      }
    }
    for (; j < j1; ++j) {
      const int64_t m = ((int64_t)(l0 + j / ng) * a.batch + b) * a.groups + g0 + j % ng;
      const float z = tri_z(a.scores[m * a.row_stride + t], a.stats[4 * m], a.stats[4 * m + 1], a.stats[4 * m + 2]);
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
// 256 tokens with one instruction.  SLICES > 1: one block of SLICES waves per
// (256-token tile, output row), wave j takes the j-th of SLICES ordered
// parts of the members, partial maxima combined in wave order; SLICES = 1: a
// block of kTriThreads covers kTriSpan tokens.  Per token the arithmetic and
// the order are those of tri_reduce_kernel.
template <int SLICES>
__global__ __launch_bounds__(SLICES > 1 ? 64 * SLICES : kTriThreads) void tri_reduce4_kernel(TriArgs a) {
  __shared__ float4 s_part[SLICES][64];
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
        const double mu = a.stats[4 * m[u]], sg = a.stats[4 * m[u] + 1], ri = a.stats[4 * m[u] + 2];
        const float xs[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float z = t0 + e < L ? tri_z(xs[e], mu, sg, ri) : -__builtin_inff();
          if (z > r[e]) r[e] = z;
        }
      }
    }
    for (; j < j1; ++j) {
      const int64_t m = member(j);
      const float4 x = *reinterpret_cast<const float4*>(a.scores + m * a.row_stride + t0);
      const double mu = a.stats[4 * m], sg = a.stats[4 * m + 1], ri = a.stats[4 * m + 2];
      const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float z = t0 + e < L ? tri_z(xs[e], mu, sg, ri) : -__builtin_inff();
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

hipError_t launch_tri(const TriArgs& args, hipStream_t st) {
  TriArgs a = args;
  // SD_TRI_EXACT_SLOW=1 (tests): every sum by long accumulation
  const char* slow = getenv("SD_TRI_EXACT_SLOW");
  a.exact_slow = (slow && slow[0] == '1') ? 1 : 0;
  const int members = a.layers * a.batch * a.groups;
  const int out_rows = tri_out_rows(a.layers, a.batch, a.groups, a.mode);
  if (members == 0 || a.row_stride == 0) return hipSuccess;
  const bool rows16 = (a.row_stride % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0;
  // per layer and head, rows held in registers give their z rows at once
  // (not at all when the kernel also selects and the caller does not read them)
  const bool fused_sel = a.sel_indices != nullptr;
  a.z_rows = (a.mode == 0 && rows16 && a.row_stride <= 16384 && (reinterpret_cast<uintptr_t>(a.reduced) & 15) == 0 &&
              (!fused_sel || a.want_reduced))
                 ? 1 : 0;
  // rows held in registers: one wave per row up to 4096 tokens (up to 64 per
  // lane), four waves up to 16384; longer rows, or rows that are not whole
  // 16-byte units, are read again in every pass.  Per layer and head, the
  // z rows (when read) and the selection (when asked) come from the same
  // kernel.
  const bool zr = a.z_rows != 0;
  if (rows16 && a.row_stride <= 4096) {
    const int nv = a.row_stride <= 1024 ? 4 : (a.row_stride <= 2048 ? 8 : 16);
    auto go = [&](auto nvc) {
      constexpr int NV = decltype(nvc)::value;
      if (fused_sel && zr) tri_stats_kernel<NV, 1, true, true><<<members, 64, 0, st>>>(a);
      else if (fused_sel) tri_stats_kernel<NV, 1, false, true><<<members, 64, 0, st>>>(a);
      else if (zr) tri_stats_kernel<NV, 1, true, false><<<members, 64, 0, st>>>(a);
      else tri_stats_kernel<NV, 1><<<members, 64, 0, st>>>(a);
    };
    if (nv == 4) go(std::integral_constant<int, 4>{});
    else if (nv == 8) go(std::integral_constant<int, 8>{});
    else go(std::integral_constant<int, 16>{});
  } else if (rows16 && a.row_stride <= 8192) {
    if (zr) tri_stats_kernel<8, 4, true><<<members, 256, 0, st>>>(a);
    else tri_stats_kernel<8, 4><<<members, 256, 0, st>>>(a);
  } else if (rows16 && a.row_stride <= 16384) {
    if (zr) tri_stats_kernel<16, 4, true><<<members, 256, 0, st>>>(a);
    else tri_stats_kernel<16, 4><<<members, 256, 0, st>>>(a);
  } else {
    tri_stats_kernel<0, 4><<<members, 256, 0, st>>>(a);
  }
  // per layer and head with the z rows written (or not wanted): no reduce pass
  if (zr || fused_sel) return hipGetLastError();
  const int nm = a.mode == 0 ? 1 : (a.mode == 1 ? a.layers : a.layers * a.groups);
  const bool vec = (a.row_stride % 4) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(a.reduced) & 15) == 0;
  if (vec && nm >= 128)
    tri_reduce4_kernel<16><<<dim3((a.row_stride + 255) / 256, out_rows), 1024, 0, st>>>(a);
  else if (vec && nm >= 16)
    tri_reduce4_kernel<4><<<dim3((a.row_stride + 255) / 256, out_rows), 256, 0, st>>>(a);
  else if (vec)
    tri_reduce4_kernel<1><<<dim3((a.row_stride + kTriSpan - 1) / kTriSpan, out_rows), kTriThreads, 0, st>>>(a);
  else if (nm >= 16)
    tri_reduce_kernel<4><<<dim3((a.row_stride + 63) / 64, out_rows), kTriThreads, 0, st>>>(a);
  else
    tri_reduce_kernel<1><<<dim3((a.row_stride + kTriSpan - 1) / kTriSpan, out_rows), kTriThreads, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace sd
