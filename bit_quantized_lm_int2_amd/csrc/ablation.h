// The design alternatives of the coarse contraction, built into the production kernels so that
// each differs from the chosen design in one property only.
//
// radiance_drafthead.py, module docstring (its measured alternatives): quantisation group 64
// instead of 128 (twice the scales, and the per-group scale and zero work on the accumulator
// doubles); a contiguous-4 byte layout instead of the quarter split (byte j holds the codes of
// k = 4j .. 4j + 3, so the four codes of a byte share one group and no mask-only dequant exists);
// the scale and zero applied to every weight of a dequantised bf16 tile instead of to the
// accumulator.
#pragma once
#include "dequant.h"

namespace i2h {

constexpr int kVarDesign = 0;  // group 128, quarter-split bytes, scale and zero on the accumulator
constexpr int kVarG64 = 1;     // group 64
constexpr int kVarC4 = 2;      // contiguous-4 bytes
constexpr int kVarWTile = 3;   // every weight S (1 + v/4) - ZS in bf16 before the dot

// Eight weights k .. k + 7 of the contiguous-4 layout as bf16 1 + v/4, natural k order. hv: the
// two bytes of the run, code j (k + j) at bits 2j, 2j + 1. Each code is moved to bits 5-6 of its
// half: the four codes of a byte sit at four different places, so a mask alone cannot read them.
__device__ __forceinline__ bf16x8 dequant8_c4(uint32_t hv) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t t = hv >> (4 * j);
    r[j] = ((t << 5) & 0x60u) | ((t << 19) & 0x00600000u) | 0x3F803F80u;
  }
  return __builtin_bit_cast(bf16x8, r);
}

// The dequantised weight tile from the mask dequant's values c = 1 + v / (4 f) (dequant.h): with
// s1 = f S and z1 = (f - 1) S + ZS, s1 c - z1 = S (1 + v/4) - ZS; the product s1 c is exact (at
// most 16 significant bits), so the FMA rounds the weight once in fp32, as an fp32 product and
// difference would, and the result is rounded to bf16 (nearest even) for the bf16 dot.
__device__ __forceinline__ bf16x8 tile8_fold(const bf16x8& c, float s1, float z1) {
  const u32x4 u = __builtin_bit_cast(u32x4, c);
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = (__bf16)__builtin_fmaf(s1, __uint_as_float(u[j] << 16), -z1);
    o[2 * j + 1] = (__bf16)__builtin_fmaf(s1, __uint_as_float(u[j] & 0xffff0000u), -z1);
  }
  return o;
}

}  // namespace i2h
