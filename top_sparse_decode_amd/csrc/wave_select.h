// wave_select.h -- selection of the k largest keys of one row by one wave,
// the row's keys in registers (lane l: positions 4 (l + 64 i) .. +3).
//
// Used for rows of at most 256 NI tokens: by the standalone selection when
// there are many such rows, and by the TriAttention per-layer-per-head path
// on the z values it has just formed.
//  1. The k-th largest key is narrowed by histograms of 256 bins over the
//     candidate key range [lo, hi] (bins by the top 8 bits of key - lo; four
//     copies in LDS, lane l counting into copy l % 4, so that lanes with
//     equal bins meet less often), each pass keeping the bin that holds it
//     and counting the keys above that bin.  A bin of at most 64 keys is
//     ranked directly (each entry counts the entries ahead of it in (key
//     desc, position asc) order), and a range narrowed to one key keeps its
//     lowest positions.  Order-preserving keys cluster by binade, so the bin
//     of a typical k-th key is small after one or two passes.
//  2. Emission in position order: wave scans of the band and kept counts
//     give each kept token its output slot.
#pragma once

#include "common.h"

namespace sd {

constexpr int kWaveBins = 256;
constexpr int kWaveCopies = 4;
constexpr int kWaveCopyStride = kWaveBins + 8;  // copies start 8 banks apart
constexpr int kWaveRank = 64;  // band sizes ranked directly (one entry per lane)

// inclusive prefix sum over the wave by data-parallel moves within rows of 16
// lanes, then row broadcasts (no LDS)
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// exclusive prefix over the wave; total (uniform) gets the sum
__device__ __forceinline__ int wave_excl_scan(int v, int& total) {
  const int inc = wave_incl_scan_dpp(v);
  total = __builtin_amdgcn_readlane(inc, 63);
  return inc - v;
}

__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// order-preserving key of a score (larger score, larger key; -0 is made +0
// first); callers give tokens past the row's length key 0, and raise the one
// NaN key that would be 0 to 1 (NaN scores give an unspecified selection)
__device__ __forceinline__ uint32_t wave_key(float x) {
  const uint32_t u = __float_as_uint(x + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

template <int NI>
struct WaveSelectSmem {
  // four histogram copies, then one spill slot per lane (keys outside [lo, hi])
  __attribute__((aligned(16))) int hist[kWaveCopies * kWaveCopyStride + 64];
  uint32_t bkey[kWaveRank], bpos[kWaveRank];
  uint32_t kbits[NI * 8];  // kept band positions, one bit per position
};

// The k positions of the largest keys (key desc, position asc), written in
// ascending order to out[0 .. k) (and wb when not null).  key: the row's
// keys, 0 past its length L (> k) and at least 1 below it; kmin / kmax: the
// smallest and largest live key (uniform).
template <int NI>
__device__ __forceinline__ void wave_select(const uint32_t (&key)[NI][4], uint32_t kmin, uint32_t kmax, int k,
                                            int32_t* out, int32_t* wb, WaveSelectSmem<NI>& sh) {
  const int lane = threadIdx.x & 63;
  auto put = [&](int i, int v) {
    out[i] = v;
    if (wb) wb[i] = v;
  };
  // position of element (i, e) of this lane, recomputed at each use (no
  // per-element positions held in registers)
  auto pos_of = [&](int i, int e) {
    int l4 = 4 * lane;
    asm volatile("" : "+v"(l4));
    return l4 + 256 * i + e;
  };
  // ---- 1. the k-th largest: keys in [lo, hi] hold it, `above` tokens exceed hi
  uint32_t lo = kmin, hi = kmax;
  int above = 0;
  bool ranked = false;
  while (lo < hi) {
    const uint32_t span = hi - lo;
    const int shift = max(0, 32 - __clz(span) - 8);  // (hi - lo) >> shift < 256
#pragma unroll
    for (int c = 0; c < kWaveCopies; ++c)
      *reinterpret_cast<int4*>(&sh.hist[c * kWaveCopyStride + 4 * lane]) = make_int4(0, 0, 0, 0);
    __builtin_amdgcn_wave_barrier();
    const int copy = (lane % kWaveCopies) * kWaveCopyStride;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // keys outside [lo, hi] (and those past L) count in the lane's own
        // spill slot: no per-token branch
        const uint32_t d = key[i][e] - lo;
        const int bin = d <= span ? copy + (int)(d >> shift) : kWaveCopies * kWaveCopyStride + lane;
        atomicAdd(&sh.hist[bin], 1);
      }
    __builtin_amdgcn_wave_barrier();
    int h[4] = {0, 0, 0, 0};
#pragma unroll
    for (int c = 0; c < kWaveCopies; ++c) {
      const int4 h4 = *reinterpret_cast<const int4*>(&sh.hist[c * kWaveCopyStride + 4 * lane]);
      h[0] += h4.x; h[1] += h4.y; h[2] += h4.z; h[3] += h4.w;
    }
    const int c4 = h[0] + h[1] + h[2] + h[3];
    int tot;
    const int before = wave_excl_scan(c4, tot);
    const int after = tot - before - c4;  // keys in the bins of higher lanes
    const int need = k - above;            // 1 <= need <= keys in [lo, hi]
    // the lane whose bins reach `need` counting down from the top bin
    const bool mine = after < need && after + c4 >= need;
    int j = 3, sup = after;                // sup: keys in bins above bin 4 lane + j
    if (mine) {
      while (j > 0 && sup + h[j] < need) sup += h[j--];
    }
    const uint64_t who = __builtin_amdgcn_ballot_w64(mine);
    const int src = who ? __builtin_ctzll(who) : 0;
    const int bstar = __builtin_amdgcn_readlane(4 * lane + j, src);
    above += __builtin_amdgcn_readlane(sup, src);
    const int nband = __builtin_amdgcn_readlane(mine ? h[j] : 0, src);
    __builtin_amdgcn_wave_barrier();
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)bstar << shift);
    const uint64_t nhi = min((uint64_t)hi, nlo + ((1ull << shift) - 1));
    lo = (uint32_t)nlo;
    hi = (uint32_t)nhi;
    if (lo < hi && nband <= kWaveRank) {
      ranked = true;
      break;
    }
  }
  // band: keys in [lo, hi]; `need` of them are kept
  const int need = k - above;
  const uint32_t bspan = hi - lo;

  int kbase = 0;
  if (ranked) {
    // a short band: its entries to LDS (any order), each ranked by one lane;
    // the kept ones set their position's bit
    if (lane < NI * 8 / 4) *reinterpret_cast<uint4*>(&sh.kbits[4 * lane]) = make_uint4(0, 0, 0, 0);
    int nb = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool in = key[i][e] - lo <= bspan;
        const uint64_t m = __builtin_amdgcn_ballot_w64(in);
        if (m) {
          const int pos = nb + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
          if (in && pos < kWaveRank) {
            sh.bkey[pos] = key[i][e];
            sh.bpos[pos] = pos_of(i, e);
          }
          nb += __builtin_popcountll(m);
        }
      }
    __builtin_amdgcn_wave_barrier();
    if (lane < nb && lane < kWaveRank) {
      // entries ahead of this one: larger key, or equal key at a lower position
      const uint32_t mk = sh.bkey[lane], mp = sh.bpos[lane];
      int rank = 0;
      for (int q = 0; q < nb; ++q) {
        const uint32_t qk = sh.bkey[q], qp = sh.bpos[q];
        rank += (qk > mk || (qk == mk && qp < mp)) ? 1 : 0;
      }
      if (rank < need) atomicOr(&sh.kbits[mp >> 5], 1u << (mp & 31));
    }
    __builtin_amdgcn_wave_barrier();
    // ---- 2. emission in position order: kept = above the band, or a kept
    // band entry
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const uint32_t bits = sh.kbits[8 * i + (lane >> 3)] >> (4 * (lane & 7));  // this lane's 4 positions
      int keep[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) keep[e] = (key[i][e] > hi || ((bits >> e) & 1u)) ? 1 : 0;
      int tot;
      int kpos = kbase + wave_excl_scan(keep[0] + keep[1] + keep[2] + keep[3], tot);
      kbase += tot;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (keep[e] && kpos < k) put(kpos++, pos_of(i, e));
    }
  } else {
    // ---- 2'. emission in position order when the band is one key (or
    // every live key is equal): its first `need` positions are kept
    int bbase = 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      int f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = (key[i][e] - lo <= bspan) ? 1 : 0;
      int tot;
      int bpos = bbase + wave_excl_scan(f[0] + f[1] + f[2] + f[3], tot);
      bbase += tot;
      int keep[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        keep[e] = (key[i][e] > hi || (f[e] && bpos < need)) ? 1 : 0;
        bpos += f[e];
      }
      int kpos = kbase + wave_excl_scan(keep[0] + keep[1] + keep[2] + keep[3], tot);
      kbase += tot;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (keep[e] && kpos < k) put(kpos++, pos_of(i, e));
    }
  }
}

}  // namespace sd
