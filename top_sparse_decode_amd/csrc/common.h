// common.h -- internal helpers shared by the HIP kernels of libsparse_decode.
// gfx950 (CDNA4): 64-lane wavefronts, 160 KB LDS per CU, bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short shortx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef int intx8 __attribute__((ext_vector_type(8)));

// bfloat16 is the upper half of a binary32: widening is exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Cache policy of global_load_lds for data read once per call (indexer K,
// gathered latent rows): the non-temporal hint.  Those streams then do not
// displace what is reused (queries, partials, scores) from the caches, and
// dirty partial results of the previous step are not written back while the
// next step streams.
constexpr int kLoadStream = 2;
constexpr int kLoadReuse = 0;

// OCP FP8 E4M3 byte `B` of a 32-bit word -> binary32 (exact; codes 0x7F and
// 0xFF decode to NaN).  gfx950's conversion implements the OCP encoding.
template <int B>
__device__ __forceinline__ float fp8_to_f32(uint32_t w) { return __builtin_amdgcn_cvt_f32_fp8((int)w, B); }

// Four E4M3 codes -> their dequantized values decode(code) * scale, each
// product rounded once (the library's dequantization).
__device__ __forceinline__ void fp8x4_dequant(uint32_t w, float scale, float* v) {
  v[0] = __fmul_rn(fp8_to_f32<0>(w), scale);
  v[1] = __fmul_rn(fp8_to_f32<1>(w), scale);
  v[2] = __fmul_rn(fp8_to_f32<2>(w), scale);
  v[3] = __fmul_rn(fp8_to_f32<3>(w), scale);
}

// Smallest E4M3 code whose value is >= x, for finite 0 <= x <= 448.
__device__ __forceinline__ uint32_t fp8_round_up(float x) {
  if (!(x > 0.0f)) return 0u;
  if (x < 0.015625f) return (uint32_t)__builtin_ceilf(x * 512.0f);  // subnormals m * 2^-9 (8 = 2^-6)
  const uint32_t u = __float_as_uint(x);
  uint32_t r = (u >> 20) - (120u << 3);  // biased exponent and top 3 mantissa bits
  if (u & 0xFFFFFu) ++r;                 // round up (a carry moves into the exponent)
  return r < 0x7Eu ? r : 0x7Eu;
}

// Offset of the row scale of (page, KV head g, slot) in an fp8 pool's scale array.
__device__ __forceinline__ int64_t fp8_scale_index(int page, int g, int slot, int num_kv_heads, int page_size) {
  return ((int64_t)page * num_kv_heads + g) * page_size + slot;
}

// binary32 -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return uint16_t((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Smallest bfloat16 >= x for finite x >= 0 (bits in the low half).
__device__ __forceinline__ uint32_t bf16_round_up(float x) {
  uint32_t u = __float_as_uint(x);
  if (u & 0xFFFFu) u += 0x10000u;
  return u >> 16;
}

// Order-preserving key: larger float -> larger key; -0 maps like +0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o);
    v = v > w ? v : w;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

// Inclusive scan over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int w = __shfl_up(v, o);
    if (lane >= o) v += w;
  }
  return v;
}

// Exclusive scan over a block of NT threads (NT/64 <= 64 waves).  `tmp` needs
// NT/64 ints of shared memory.  Returns the exclusive prefix; *total gets the
// block sum.  Contains __syncthreads.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int* tmp, int* total) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int inc = wave_incl_scan(v);
  if (lane == 63) tmp[wid] = inc;
  __syncthreads();
  int wsum = lane < NW ? tmp[lane] : 0;
  int winc = wave_incl_scan(wsum);
  int wexcl = __shfl(winc, wid) - __shfl(wsum, wid);
  int tot = __shfl(winc, NW - 1);
  __syncthreads();
  *total = tot;
  return wexcl + inc - v;
}

// Data that blocks of one launch hand to each other (read after the writer
// has announced it through an atomic counter): device-coherent stores and
// loads (agent-scope atomic accesses, coherent across the XCDs' L2 caches),
// no cache-wide fences.
__device__ __forceinline__ void st_coherent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_coherent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_coherent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_coherent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int2 ld_coherent2(const int32_t* p) {
  const uint64_t v = ld_coherent(reinterpret_cast<const uint64_t*>(p));
  return int2{(int)(uint32_t)v, (int)(uint32_t)(v >> 32)};
}

// v + (v of lane ^ 16), then + (that of lane ^ 32): the sum over a lane's
// four 16-lane rows, in every lane, by gfx950's lane-swap instructions (VALU
// only, no LDS permute).  Each add takes its own value first, so the result
// equals `v += shfl_xor(v, 16); v += shfl_xor(v, 32)` bit for bit (a
// floating-point add is commutative).
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Wait until this thread's stores and atomics have completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" : : : "memory"); }

__device__ __forceinline__ int clamp_len(int L, int cap) { return L < 0 ? 0 : (L > cap ? cap : L); }

}  // namespace sd
