// Ranking within a wave (gfx950, wave64) on fp64-coded keys, with DPP and permlane exchanges.
//
// A ranking key (score, token) is coded as the double with bits 0x3FF << 52 | ordered_key(score)
// << 20 | (0xFFFFF - token): every valid key lies in [1, 2), double order is (score descending,
// token ascending), and 0.0 marks an empty slot. Tokens must be below 2^20 (N <= 524288). A
// compare-exchange is then v_max_f64 + v_min_f64, and the partner of lane ^ s comes from quad
// permutes (s = 1, 2), row shifts (s = 4, 8) or the permlane swaps (s = 16, 32) instead of an
// LDS permute, which keeps the dependent chain of a bitonic network short.
#pragma once
#include "device_util.h"

namespace i2h {

__device__ __forceinline__ double token_key(float score, int32_t token) {
  if (token < 0) return 0.0;
  const uint64_t b = 0x3FF0000000000000ull | ((uint64_t)ordered_key(score) << 20) |
                     (uint64_t)(0xFFFFFu - (uint32_t)token);
  return __builtin_bit_cast(double, b);
}
__device__ __forceinline__ int32_t token_key_token(double k) {
  if (!(k > 0.0)) return -1;
  return (int32_t)(0xFFFFFu - (uint32_t)(__builtin_bit_cast(uint64_t, k) & 0xFFFFFull));
}
__device__ __forceinline__ float token_key_score(double k) {
  if (!(k > 0.0)) return -__builtin_inff();
  return from_ordered_key((uint32_t)(__builtin_bit_cast(uint64_t, k) >> 20));
}

// The 32-bit value of lane ^ S (S = 1, 2, 4, 8, 16, 32).
template <int S>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  const int lane = threadIdx.x & 63;
  if constexpr (S == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
  } else if constexpr (S == 4 || S == 8) {
    const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + S, 0xF, 0xF, false);  // lane + S
    const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x110 + S, 0xF, 0xF, false);  // lane - S
    return (lane & S) ? dn : up;
  } else if constexpr (S == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? p[0] : p[1];
  } else {
    static_assert(S == 32, "lane_xor: S in 1, 2, 4, 8, 16, 32");
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? p[0] : p[1];
  }
}

template <int S>
__device__ __forceinline__ double lane_xor_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = lane_xor<S>((uint32_t)u), hi = lane_xor<S>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, (hi << 32) | lo);
}

__device__ __forceinline__ double lane_xor_f64(double v, int s) {  // s a constant after unrolling
  switch (s) {
    case 1: return lane_xor_f64<1>(v);
    case 2: return lane_xor_f64<2>(v);
    case 4: return lane_xor_f64<4>(v);
    case 8: return lane_xor_f64<8>(v);
    case 16: return lane_xor_f64<16>(v);
    default: return lane_xor_f64<32>(v);
  }
}

// Descending bitonic sort of the 64 * KPL keys of a wave, KPL per lane, key index e * 64 + lane.
// With NMAX < 64 (KPL = 1) only the stages up to NMAX run: each aligned run of NMAX lanes is
// sorted on its own, lanes 0 .. NMAX - 1 descending.
template <int KPL, int NMAX = 64 * KPL>
__device__ __forceinline__ void wave_sort_f64(double (&k)[KPL]) {
  const int lane = threadIdx.x & 63;
  static_assert(NMAX == 64 * KPL || (KPL == 1 && NMAX >= 2 && (NMAX & (NMAX - 1)) == 0), "NMAX: a power of two");
#pragma unroll
  for (int size = 2; size <= NMAX; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 64) {
        const int es = stride / 64;
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          if ((e & es) != 0) continue;
          const bool desc = ((e * 64) & size) == 0;
          const double hi = __builtin_fmax(k[e], k[e + es]), lo = __builtin_fmin(k[e], k[e + es]);
          k[e] = desc ? hi : lo;
          k[e + es] = desc ? lo : hi;
        }
      } else {
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          const double o = lane_xor_f64(k[e], stride);
          const bool lower = (lane & stride) == 0;
          const bool desc = ((e * 64 + lane) & size) == 0;
          k[e] = (lower == desc) ? __builtin_fmax(k[e], o) : __builtin_fmin(k[e], o);
        }
      }
    }
  }
}

// a (lane i holds the i-th best of a descending 64-list) becomes the 64 best of a and b (b held
// the same way), descending: max(a[i], b[63 - i]) is bitonic, then six half-cleaner stages.
__device__ __forceinline__ double wave_merge64_f64(double a, const double* b_lds) {
  const int lane = threadIdx.x & 63;
  double v = __builtin_fmax(a, b_lds[63 - lane]);
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) {
    const double o = lane_xor_f64(v, s);
    v = (lane & s) == 0 ? __builtin_fmax(v, o) : __builtin_fmin(v, o);
  }
  return v;
}

}  // namespace i2h
