// Quantise and pack a bf16 head into int2 quarter-split codes plus premultiplied bf16 scales.
//
// radiance_drafthead.py, _quantize_head_now: per (row n, group of 128 consecutive k) an
// asymmetric min/max quantiser at 2 bits; byte j of a packed row carries the codes of
// k = j, Q+j, 2Q+j, 3Q+j (Q = K/4); S = bf16(4 sc), ZS = bf16(4 sc + zp sc).
//
// The bytes j = 128 gb + i (i = 0..127) of span gb of a packed row draw on four quantisation
// groups, one per quarter t (k = tQ + 128 gb + i, group t*NG + gb with NG = K/512), so the
// lanes that read the four quarters' 128-k stretches (256 contiguous bytes each) hold every
// input of 128 packed bytes and of four S/ZS pairs.
//
// Bit-exactness: the page evaluates these steps as separate eager fp32 kernels. This file is
// built with -ffp-contract=off and correctly rounded fp32 division, and the pragma below keeps
// any multiply-add from being fused. It is also built without NaN semantics (min / max need no
// quieting): W must be finite.
#include "device_util.h"
#include "fp8.h"
#include "host_util.h"

#pragma clang fp contract(off)

#ifndef I2H_PACK_MAX_WG
#define I2H_PACK_MAX_WG 65536  // workgroups at most (grid-stride loop beyond)
#endif
#ifndef I2H_PACK_STEPS
#define I2H_PACK_STEPS 2  // loop steps per wave at least, before the cap
#endif

namespace i2h {
namespace {

// Reductions over the 4 lanes of a quad (the lanes that share one quantisation group): two DPP
// quad permutes (lane ^ 1, lane ^ 2); built without NaN semantics, each step is one v_min/v_max
// with a DPP operand.
template <int CTRL>
__device__ __forceinline__ float quad_perm(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_min(float v) {
  v = fminf(v, quad_perm<0xB1>(v));
  return fminf(v, quad_perm<0x4E>(v));
}
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, quad_perm<0xB1>(v));
  return fmaxf(v, quad_perm<0x4E>(v));
}

__device__ __forceinline__ float clamp03(float v) { return fminf(fmaxf(v, 0.0f), 3.0f); }

// d / 3 correctly rounded (d >= 0): q = RN(d * RN(1/3)), then one FMA residual correction. The
// residual d - 3q is exact in one FMA, and an exhaustive check over every non-negative finite
// fp32 d (subnormals included) finds the corrected quotient equal to the IEEE quotient.
__device__ __forceinline__ float div3_rn(float d) {
  constexpr float kThird = 1.0f / 3.0f;
  const float q = __fmul_rn(d, kThird);
  return __builtin_fmaf(__builtin_fmaf(-q, 3.0f, d), kThird, q);
}

// fl(a / b) from y = fl(1 / b) (both IEEE round-to-nearest-even) with one FMA correction:
// q0 = fl(a y) is within an ulp or two of a / b, the residual a - b q0 is exact in one FMA, and
// fl(q0 + r y) is the correctly rounded quotient. An exhaustive check over every fp32 significand
// of b and every bf16 significand of a (the sign and powers of two change nothing while no
// intermediate overflows or underflows) finds no exception. For |a / b| below 2^-75 the residual
// may underflow; such quotients are far below the 0.5 that a code can turn on.
__device__ __forceinline__ float quot_rn(float a, float b, float y) {
  const float q0 = __fmul_rn(a, y);
  return __builtin_fmaf(__builtin_fmaf(-b, q0, a), y, q0);
}

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {  // finite f
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

constexpr int kPackWaves = 4;

// Work is cut into units (row n, span gb): the 128 packed bytes n*Q + 128 gb .. +127, made from
// the four groups (n, t*NG + gb), t = 0..3. Unit u = n*NG + gb, so the unit's packed bytes start
// at 128 u. A wave takes four consecutive units per step (a quad, which may straddle rows) and
// steps through quads with the grid's wave count as stride, loading the next quad's weights
// before it works on the current one.
// Lane l = 16 t + 4 g + p works on quarter t of unit 4 quad + g: it loads 16 bytes at 64-byte
// steps, 32 weights of group (n, t*NG + gb) at offsets 32 c + 8 p + e (c = 0..3, e = 0..7), so
// each load instruction reads 64 contiguous bytes per group and the quad of lanes p = 0..3
// together holds the whole group. After the group's min / max (quad reductions), scale, zero and
// codes, lane (t, g, p) holds the 2-bit codes of output bytes 32 c + 8 p + e of its unit for
// quarter t; two permlane swap rounds (rows t ^ 1, then t ^ 2) OR the four quarters together,
// shifting each field into bits 2t on the way, and leave lane (t, g, p) with bytes
// 32 t + 8 p .. +7, which it stores. Lane p = 0 of each (t, g) writes its group's S and ZS.
// FP8: the weight is an FP8 head (e4m3 bytes Wv with a per-row fp32 scale); each weight is the
// decoded byte times the row's scale (one fp32 product, as the page's quantiser sees it). Those
// fp32 weights have full 24-bit significands, for which the exhaustive check of quot_rn (over
// bf16 numerators) says nothing, so their codes use the IEEE division.
template <bool FP8>
__global__ __launch_bounds__(kPackWaves * kWave) void pack_kernel(
    const void* __restrict__ Wv, const float* __restrict__ wscale, int64_t ldw, int N, int K,
    uint8_t* __restrict__ packed, uint16_t* __restrict__ S, uint16_t* __restrict__ ZS) {
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane >> 4, g = (lane >> 2) & 3, p = lane & 3;
  const int Q = K >> 2;
  const int NG = Q / kGroup;  // spans (units) per row
  const int KG = K / kGroup;  // groups per row
  const int units = N * NG;   // <= 2^30 (host check)
  const int quads = (units + 3) >> 2;
  const int wstep = gridDim.x * kPackWaves;
  const int q0 = blockIdx.x * kPackWaves + (threadIdx.x >> 6);
  if (q0 >= quads) return;  // wave-uniform
  // (row, span) of this lane's unit, advanced by 4 * wstep units per step without a division
  const int ustep = 4 * wstep;
  const int dn = ustep / NG, dgb = ustep - dn * NG;
  int u = 4 * q0 + g;
  int n = u / NG, gb = u - n * NG;
  float vs = 0.f;  // the row scale of the loaded weights (FP8)
  auto load = [&](u32x4 (&v)[4], int un, int ugb) {
    const int nc = un < N ? un : N - 1;  // past the last unit: a valid row, never stored
    const int64_t off = (int64_t)nc * ldw + t * Q + ugb * kGroup + 8 * p;  // in weights
    if constexpr (FP8) {
      typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
      const uint8_t* src = static_cast<const uint8_t*>(Wv) + off;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x2 b = *reinterpret_cast<const u32x2*>(src + 32 * c);
        v[c] = u32x4{b[0], b[1], 0u, 0u};
      }
      vs = wscale[nc];
    } else {
      const uint16_t* src = static_cast<const uint16_t*>(Wv) + off;
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = *reinterpret_cast<const u32x4*>(src + 32 * c);
    }
  };
  u32x4 v[4];
  load(v, n, gb);
  for (int qd = q0; qd < quads; qd += wstep) {
    float w[32];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if constexpr (FP8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) w[8 * c + e] = __fmul_rn(fp8_e4m3_value(byte_of(v[c][0], v[c][1], e)), vs);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w[8 * c + 2 * e] = bf16_lo(v[c][e]);
          w[8 * c + 2 * e + 1] = bf16_hi(v[c][e]);
        }
      }
    }
    const int cu = u, cn = n, cgb = gb;
    u += ustep;
    n += dn;
    gb += dgb;
    if (gb >= NG) {
      gb -= NG;
      ++n;
    }
    load(v, n, gb);
    float lo = w[0], hi = w[0];
#pragma unroll
    for (int e = 1; e < 32; ++e) {
      lo = fminf(lo, w[e]);
      hi = fmaxf(hi, w[e]);
    }
    lo = quad_min(lo);
    hi = quad_max(hi);
    const float sc = fmaxf(div3_rn(__fadd_rn(hi, -lo)), 1e-8f);
    float zp, q[32];
    if constexpr (FP8) {
      zp = clamp03(rintf(__fdiv_rn(-lo, sc)));
#pragma unroll
      for (int e = 0; e < 32; ++e) q[e] = clamp03(rintf(__fadd_rn(__fdiv_rn(w[e], sc), zp)));
    } else {
      // The page's codes clamp(rint(fl(fl(w / sc) + zp)), 0, 3), with each quotient from quot_rn.
      // The rounding to an integer is left to the byte conversion below (clamping to [0, 3] first
      // gives the same code).
      // Groups whose quotients could overflow, or whose 1 / sc could leave the normal range, take
      // the IEEE division throughout (never met by a real head).
      const bool wide = !(sc < 0x1p100f) || !(fmaxf(hi, -lo) < 0x1p100f);
      const float y = __fdiv_rn(1.0f, sc);
      zp = clamp03(__builtin_rintf(quot_rn(-lo, sc, y)));
#pragma unroll
      for (int e = 0; e < 32; ++e) q[e] = clamp03(__fadd_rn(quot_rn(w[e], sc, y), zp));
      if (__builtin_amdgcn_ballot_w64(wide) != 0ull) {
        if (wide) {
          zp = clamp03(rintf(__fdiv_rn(-lo, sc)));
#pragma unroll
          for (int e = 0; e < 32; ++e) q[e] = clamp03(rintf(__fadd_rn(__fdiv_rn(w[e], sc), zp)));
        }
      }
    }
    // codes as bytes: v_cvt_pk_u8_f32 rounds to nearest with ties to even (as rint does) and
    // saturates; word (c, h) holds bytes 32 c + 8 p + 4 h .. +3
    uint32_t wd[4][2];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t acc = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_cvt_pk_u8_f32(q[8 * c + 4 * h + e], e, acc);
        wd[c][h] = acc;
      }
    }
    // Round 1 (rows t, t ^ 1): after the swap of (wd[c], wd[c + 1]), c even, both results hold
    // the word c + (t & 1) of rows 2(t >> 1) and 2(t >> 1) + 1, in that order.
    // Round 2 (rows t, t ^ 2): after the swap of (x, y), both results hold the word t of rows
    // {0, 1} and of rows {2, 3}, in that order.
    uint32_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto a = __builtin_amdgcn_permlane16_swap(wd[0][h], wd[1][h], false, false);
      const uint32_t x = a[0] | (a[1] << 2);
      const auto b = __builtin_amdgcn_permlane16_swap(wd[2][h], wd[3][h], false, false);
      const uint32_t y = b[0] | (b[1] << 2);
      const auto z = __builtin_amdgcn_permlane32_swap(x, y, false, false);
      out[h] = z[0] | (z[1] << 4);
    }
    if (cu < units) {
      uint32_t* dst = reinterpret_cast<uint32_t*>(packed + (int64_t)cu * kGroup + 32 * t + 8 * p);
      dst[0] = out[0];
      dst[1] = out[1];
      if (p == 0) {
        const float s4 = __fmul_rn(4.0f, sc);
        const float zs = __fadd_rn(s4, __fmul_rn(zp, sc));
        const int64_t at = (int64_t)cn * KG + t * NG + cgb;
        S[at] = (uint16_t)bf16_bits_rne(s4);
        ZS[at] = (uint16_t)bf16_bits_rne(zs);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// The int4 head (radiance_drafthead.py, _quantize_head_now with BITS = 4): codes 0..15, byte j of
// a packed row [K/2 bytes] holds k = j (bits 0-3) and K/2 + j (bits 4-7); S = bf16(16 sc),
// ZS = bf16(16 sc + zp sc). Same exact arithmetic as pack_kernel (bf16 numerators, quot_rn).
//
// A unit is (row n, span gb): packed bytes 128 gb .. +127 of the row, i.e. group gb of the first
// half and group KG/2 + gb of the second. One wave per unit; lane l = 32 t + i (half t) holds the
// 4 weights k = t K/2 + 128 gb + 4 i .. +3; a half's min / max is a 32-lane reduction (DPP row
// rotations, then the permlane16 swap); lanes i and 32 + i combine their nibbles with the
// permlane32 swap and lanes 0..31 write 4 bytes each.
// ---------------------------------------------------------------------------------------------
template <int S>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + S, 0xF, 0xF, true));
}
__device__ __forceinline__ float half_min(float v) {  // over the 32 lanes of a half-wave
  v = fminf(v, row_ror<1>(v));
  v = fminf(v, row_ror<2>(v));
  v = fminf(v, row_ror<4>(v));
  v = fminf(v, row_ror<8>(v));
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fminf(v, __uint_as_float((threadIdx.x & 16) ? p[0] : p[1]));
}
__device__ __forceinline__ float half_max(float v) {
  v = fmaxf(v, row_ror<1>(v));
  v = fmaxf(v, row_ror<2>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<8>(v));
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(v, __uint_as_float((threadIdx.x & 16) ? p[0] : p[1]));
}
__device__ __forceinline__ float clamp15(float v) { return fminf(fmaxf(v, 0.0f), 15.0f); }

__global__ __launch_bounds__(kPackWaves * kWave) void pack4_kernel(const uint16_t* __restrict__ W, int64_t ldw, int N,
                                                                    int K, uint8_t* __restrict__ packed,
                                                                    uint16_t* __restrict__ S, uint16_t* __restrict__ ZS) {
  typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane >> 5, i = lane & 31;
  const int H = K >> 1, NS = H / kGroup, KG = K / kGroup;
  const int64_t units = (int64_t)N * NS;
  const int64_t wstep = (int64_t)gridDim.x * kPackWaves;
  for (int64_t u = (int64_t)blockIdx.x * kPackWaves + (threadIdx.x >> 6); u < units; u += wstep) {
    const int64_t n = u / NS;
    const int gb = (int)(u - n * NS);
    const u32x2 v = *reinterpret_cast<const u32x2*>(W + n * ldw + t * H + gb * kGroup + 4 * i);
    const float w[4] = {bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1])};
    const float lo = half_min(fminf(fminf(w[0], w[1]), fminf(w[2], w[3])));
    const float hi = half_max(fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3])));
    const float sc = fmaxf(__fdiv_rn(__fadd_rn(hi, -lo), 15.0f), 1e-8f);
    const bool wide = !(sc < 0x1p100f) || !(fmaxf(hi, -lo) < 0x1p100f);
    const float y = __fdiv_rn(1.0f, sc);
    float zp = clamp15(__builtin_rintf(quot_rn(-lo, sc, y)));
    float q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e] = clamp15(__fadd_rn(quot_rn(w[e], sc, y), zp));
    if (__builtin_amdgcn_ballot_w64(wide) != 0ull) {
      if (wide) {
        zp = clamp15(rintf(__fdiv_rn(-lo, sc)));
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = clamp15(rintf(__fadd_rn(__fdiv_rn(w[e], sc), zp)));
      }
    }
    // codes as bytes (v_cvt_pk_u8_f32: nearest, ties to even), the second half's shifted by 4
    uint32_t b = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) b = __builtin_amdgcn_cvt_pk_u8_f32(q[e], e, b);
    b <<= 4 * t;
    const auto pr = __builtin_amdgcn_permlane32_swap(b, b, false, false);
    b |= (lane & 32) ? pr[0] : pr[1];
    if (t == 0) *reinterpret_cast<uint32_t*>(packed + n * H + gb * kGroup + 4 * i) = b;
    if (i == 0) {
      const float s16 = __fmul_rn(16.0f, sc);
      const float zs = __fadd_rn(s16, __fmul_rn(zp, sc));
      const int64_t at = n * KG + t * (KG / 2) + gb;
      S[at] = (uint16_t)bf16_bits_rne(s16);
      ZS[at] = (uint16_t)bf16_bits_rne(zs);
    }
  }
}

}  // namespace
}  // namespace i2h

extern "C" int i2h_sizes(int64_t N, int64_t K, int64_t* packed_bytes, int64_t* scale_elems) {
  if (!packed_bytes || !scale_elems) return I2H_ERR_ARG;
  if (N < 1 || i2h::check_k(K) != I2H_OK) return I2H_ERR_SHAPE;
  *packed_bytes = N * (K / 4);
  *scale_elems = N * (K / I2H_GROUP);
  return I2H_OK;
}

namespace i2h {
namespace {
template <bool FP8>
int pack_launch(const void* W, const float* wscale, int64_t ldw, int64_t N, int64_t K, uint8_t* packed, uint16_t* S,
                uint16_t* ZS, hipStream_t stream) {
  if (!W || !packed || !S || !ZS || (FP8 && !wscale)) return I2H_ERR_ARG;
  if (N < 1 || check_k(K) != I2H_OK || ldw < K) return I2H_ERR_SHAPE;
  if (!aligned(W, FP8 ? 8 : 16) || ldw % 8 != 0 || !aligned(packed, 16) || !aligned(S, 16) || !aligned(ZS, 16) ||
      (FP8 && !aligned(wscale, 4)))
    return I2H_ERR_ALIGN;
  // units (row, 128-byte span) are counted in 32 bits, with room for the grid stride
  if (N * (K / 512) > (int64_t)1 << 30) return I2H_ERR_SHAPE;
  const int64_t quads = (N * (K / 512) + 3) / 4;
  const int64_t per_wg = (int64_t)kPackWaves * I2H_PACK_STEPS;
  int64_t grid = (quads + per_wg - 1) / per_wg;
  grid = grid < 1 ? 1 : (grid > I2H_PACK_MAX_WG ? I2H_PACK_MAX_WG : grid);
  hipLaunchKernelGGL(pack_kernel<FP8>, dim3((unsigned)grid), dim3(kPackWaves * kWave), 0, stream, W, wscale, ldw,
                     (int)N, (int)K, packed, S, ZS);
  return check_launch();
}
}  // namespace
}  // namespace i2h

extern "C" int i2h_pack(const uint16_t* W, int64_t ldw, int64_t N, int64_t K, uint8_t* packed,
                        uint16_t* S, uint16_t* ZS, void* stream) {
  return i2h::pack_launch<false>(W, nullptr, ldw, N, K, packed, S, ZS, (hipStream_t)stream);
}

extern "C" int i2h_pack_fp8(const uint8_t* W8, const float* wscale, int64_t ldw, int64_t N, int64_t K,
                            uint8_t* packed, uint16_t* S, uint16_t* ZS, void* stream) {
  return i2h::pack_launch<true>(W8, wscale, ldw, N, K, packed, S, ZS, (hipStream_t)stream);
}

extern "C" int i2h_pack4(const uint16_t* W, int64_t ldw, int64_t N, int64_t K, uint8_t* packed, uint16_t* S,
                         uint16_t* ZS, void* stream) {
  using namespace i2h;
  if (!W || !packed || !S || !ZS) return I2H_ERR_ARG;
  if (N < 1 || K <= 0 || K % (2 * I2H_GROUP) != 0 || K > I2H_MAX_K || ldw < K) return I2H_ERR_SHAPE;
  if (!aligned(W, 8) || ldw % 4 != 0 || !aligned(packed, 16) || !aligned(S, 2) || !aligned(ZS, 2))
    return I2H_ERR_ALIGN;
  if (N > (int64_t)1 << 31) return I2H_ERR_SHAPE;
  const int64_t units = N * (K / 256);
  const int64_t grid = (units + kPackWaves * 4 - 1) / (kPackWaves * 4);
  hipLaunchKernelGGL(pack4_kernel, dim3((unsigned)(grid < 65536 ? grid : 65536)), dim3(kPackWaves * kWave), 0,
                     (hipStream_t)stream, W, ldw, (int)N, (int)K, packed, S, ZS);
  return check_launch();
}
