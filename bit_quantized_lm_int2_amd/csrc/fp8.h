// FP8 e4m3 weight bytes (a per-channel FP8 head with a per-row fp32 scale).
//
// radiance_drafthead.py, _rerank_exact (FP8 branch): a byte decodes by bit arithmetic, with no
// hardware fp8 conversion: sign bit 7, exponent field e = bits 3-6, mantissa m = bits 0-2, value
// m * 2^-9 when e = 0, else (1 + m/8) * 2^(e - 7). Every value is exact in fp32 (0x7F, a NaN code
// of e4m3fn, reads as 480). The weight is that value times the row's fp32 scale.
#pragma once
#include "device_util.h"

namespace i2h {

__device__ __forceinline__ float fp8_e4m3_value(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u, m = b & 7u;
  const float mag = e != 0u ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
  return (b & 0x80u) ? -mag : mag;
}

// Byte i (0..7) of two dwords.
__device__ __forceinline__ uint32_t byte_of(uint32_t lo, uint32_t hi, int i) {
  return ((i < 4 ? lo : hi) >> (8 * (i & 3))) & 0xffu;
}

}  // namespace i2h
