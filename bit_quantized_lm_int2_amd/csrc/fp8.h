// FP8 e4m3 weight bytes (a per-channel FP8 head with a per-row fp32 scale).
//
// radiance_drafthead.py, _rerank_exact (FP8 branch): a byte decodes by bit arithmetic, with no
// hardware fp8 conversion: sign bit 7, exponent field e = bits 3-6, mantissa m = bits 0-2, value
// m * 2^-9 when e = 0, else (1 + m/8) * 2^(e - 7). Every value is exact in fp32 (0x7F, a NaN code
// of e4m3fn, reads as 480). The weight is that value times the row's fp32 scale.
#pragma once
#include "device_util.h"

namespace i2h {

// The 7 low bits placed at bits 20-26 of an fp32 read as 2^(e - 127) (1 + m/8) for e > 0 and as
// the subnormal m * 2^-129 for e = 0; times 2^120 (exact: a power-of-two scaling, fp32 denormals
// kept) that is the formula's value, 0x7F included. The sign bit goes to bit 31.
__device__ __forceinline__ float fp8_e4m3_value(uint32_t b) {
  const uint32_t bits = ((b & 0x7fu) << 20) | ((b & 0x80u) << 24);
  return __uint_as_float(bits) * 0x1p120f;
}

// Byte i (0..7) of two dwords.
__device__ __forceinline__ uint32_t byte_of(uint32_t lo, uint32_t hi, int i) {
  return ((i < 4 ? lo : hi) >> (8 * (i & 3))) & 0xffu;
}

}  // namespace i2h
