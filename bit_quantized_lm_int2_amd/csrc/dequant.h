// Bit-pattern dequantisation of quarter-split int2 codes into bf16 MFMA operands (gfx950).
//
// radiance_drafthead.py, module docstring and _draft_head_int2: a 2-bit code v is read as the
// bf16 value 1 + v/4 straight from its bits, 0x3F80 | v << 5, with no multiply.
//
// Quarters 0-2 are dequantised with a mask alone. The code bits of quarter t of the low byte of
// each bf16 half sit at mantissa bits 2t, 2t+1, so (d & (3 << 2t)) | 0x3F80 reads as 1 + v/D with
// D = 128, 32, 8 for t = 0, 1, 2 (quarter 3 keeps a shift, D = 4). With f = D/4 the group's dot
// P' = sum x (1 + v/D) = xs + dot/D gives
//   S P - xs ZS = (f S) P' - xs ((f - 1) S + ZS),  P = xs + dot/4,
// so the bias change folds into the per-group scale and zero applied to the accumulator; f S and
// (f - 1) S + ZS are exact in fp32 (at most 13 significant bits each).
#pragma once
#include "device_util.h"

namespace i2h {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// (a & m) | o in one VALU op. gfx9 VOP3 encodings take no literal, so with constant m and o the
// compiler emits v_and + v_or with literals; with m and o held in VGPRs (vconst) it selects one
// v_and_or_b32. Plain C rather than inline asm, so that the compiler sees the VGPR it writes:
// its MFMA hazard checks (a VALU write to a register a multi-pass MFMA still reads) need that.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t m, uint32_t o) { return (a & m) | o; }

// An ordering point for v: no instruction, but the compiler must assume v changes here, so work
// computed from v cannot be hoisted above it (keeps each slice's dequant next to its MFMAs
// instead of all of a stage's operands being live at once).
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }

// A 32-bit constant the compiler cannot fold (kept in a VGPR).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

struct DqConst {
  uint32_t one, m0, m1, m2, m3;
};

__device__ __forceinline__ DqConst dq_const() {
  return DqConst{vconst(0x3F803F80u), vconst(0x00030003u), vconst(0x000C000Cu), vconst(0x00300030u),
                 vconst(0x00600060u)};
}

// d0/d1: four packed bytes each, raw. The weights come out in k order (0, 2, 1, 3) per four
// bytes, so the x operand is stored in that order. h0/h1 = d0 >> 8, d1 >> 8.
template <int T>
__device__ __forceinline__ bf16x8 dequant8_mask(uint32_t d0, uint32_t d1, uint32_t h0, uint32_t h1,
                                                const DqConst& c) {
  u32x4 r;
  if constexpr (T < 3) {
    const uint32_t m = T == 0 ? c.m0 : (T == 1 ? c.m1 : c.m2);
    r[0] = and_or(d0, m, c.one);
    r[1] = and_or(h0, m, c.one);
    r[2] = and_or(d1, m, c.one);
    r[3] = and_or(h1, m, c.one);
  } else {
    r[0] = and_or(d0 >> 1, c.m3, c.one);
    r[1] = and_or(d0 >> 9, c.m3, c.one);
    r[2] = and_or(d1 >> 1, c.m3, c.one);
    r[3] = and_or(d1 >> 9, c.m3, c.one);
  }
  return __builtin_bit_cast(bf16x8, r);
}

constexpr float kBiasF[4] = {32.f, 8.f, 2.f, 1.f};  // D/4 for quarters 0..3

// 16 bytes of x (eight k in order) rearranged to the weight order of dequant8_mask:
// [x0 x2 x1 x3 x4 x6 x5 x7].
__device__ __forceinline__ u32x4 x_pair_order(const u32x4& v) {
  u32x4 o;
  o[0] = __builtin_amdgcn_perm(v[1], v[0], 0x05040100u);
  o[1] = __builtin_amdgcn_perm(v[1], v[0], 0x07060302u);
  o[2] = __builtin_amdgcn_perm(v[3], v[2], 0x05040100u);
  o[3] = __builtin_amdgcn_perm(v[3], v[2], 0x07060302u);
  return o;
}

}  // namespace i2h
