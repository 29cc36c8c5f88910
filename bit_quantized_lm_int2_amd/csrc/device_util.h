// Device helpers shared by the HIP kernels of libi2h (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace i2h {

constexpr int kGroup = 128;   // quantisation group along k
constexpr int kBlockN = 64;   // vocab columns per candidate block
constexpr int kWave = 64;

// Exact widening of a bf16 bit pattern (in the low 16 bits of b) to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t b) { return __uint_as_float(b & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving map of a (non-NaN) float to uint32: a < b  <=>  key(a) < key(b), and
// a == b  <=>  key(a) == key(b); -0.0 and +0.0 compare equal, so both map to the key of +0.0.
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_ordered_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// 64-bit ranking key: higher score first, then lower token index. An invalid entry (idx < 0)
// maps to 0, below every valid key (a valid key's high word is >= key(-FLT_MAX) = 0x00800000).
__device__ __forceinline__ uint64_t rank_key(float score, int32_t idx) {
  if (idx < 0) return 0ull;
  return ((uint64_t)ordered_key(score) << 32) | (uint64_t)(~(uint32_t)idx);
}
__device__ __forceinline__ int32_t rank_key_idx(uint64_t k) {
  return k == 0ull ? -1 : (int32_t)(~(uint32_t)k);
}
__device__ __forceinline__ float rank_key_score(uint64_t k) {
  return k == 0ull ? -__builtin_inff() : from_ordered_key((uint32_t)(k >> 32));
}

// Bitonic sort of n (a power of two) 64-bit keys in LDS, descending, by the whole block.
__device__ __forceinline__ void block_sort_desc(uint64_t* s, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = threadIdx.x; t < (n >> 1); t += blockDim.x) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool desc = (i & size) == 0;
        const uint64_t a = s[i], b = s[j];
        if ((a < b) == desc) { s[i] = b; s[j] = a; }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// The 64-bit value of lane `src` (each half read as uint32, so nothing is sign-extended).
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// Descending bitonic sort of 64*KPL keys held KPL per lane; key index i = e * 64 + lane.
template <int KPL>
__device__ __forceinline__ void wave_sort_keys(uint64_t (&k)[KPL], int lane) {
  constexpr int n = 64 * KPL;
#pragma unroll
  for (int size = 2; size <= n; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 64) {
        const int es = stride / 64;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          if ((e & es) != 0) continue;
          const bool desc = ((e * 64) & size) == 0;
          const uint64_t a = k[e], b = k[e + es];
          const bool sw = desc ? (a < b) : (a > b);
          k[e] = sw ? b : a;
          k[e + es] = sw ? a : b;
        }
      } else {
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          const uint64_t o = shfl_xor_u64(k[e], stride);
          const bool lower = (lane & stride) == 0;
          const bool desc = ((e * 64 + lane) & size) == 0;
          const bool keep_max = lower == desc;
          const bool o_gt = o > k[e];
          k[e] = (keep_max == o_gt) ? o : k[e];
        }
      }
    }
  }
}

}  // namespace i2h
