// Quantise and pack a bf16 head into int2 quarter-split codes plus premultiplied bf16 scales.
//
// radiance_drafthead.py, _quantize_head_now: per (row n, group of 128 consecutive k) an
// asymmetric min/max quantiser at 2 bits; byte j of a packed row carries the codes of
// k = j, Q+j, 2Q+j, 3Q+j (Q = K/4); S = bf16(4 sc), ZS = bf16(4 sc + zp sc).
//
// The bytes j = 128 gb + i (i = 0..127) of span gb of a packed row draw on four quantisation
// groups, one per quarter t (k = tQ + 128 gb + i, group t*NG + gb with NG = K/512), so one wave
// that reads the four quarters' 128-k stretches (256 contiguous bytes each) holds every input of
// 128 packed bytes and of four S/ZS pairs.
//
// Bit-exactness: the page evaluates these steps as separate eager fp32 kernels. This file is
// built with -ffp-contract=off and correctly rounded fp32 division, and the pragma below keeps
// any multiply-add from being fused.
#include "device_util.h"
#include "host_util.h"

#pragma clang fp contract(off)

namespace i2h {
namespace {

// 16-lane min / max (lanes 16r .. 16r+15 hold one quantisation group): four DPP row rotations
// (by 1, 2, 4, 8) leave every lane of the row with the reduction of all 16.
template <int S>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + S, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_min(float v) {
  v = fminf(v, row_ror<1>(v));
  v = fminf(v, row_ror<2>(v));
  v = fminf(v, row_ror<4>(v));
  return fminf(v, row_ror<8>(v));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, row_ror<1>(v));
  v = fmaxf(v, row_ror<2>(v));
  v = fmaxf(v, row_ror<4>(v));
  return fmaxf(v, row_ror<8>(v));
}

__device__ __forceinline__ float clamp03(float v) { return fminf(fmaxf(v, 0.0f), 3.0f); }

// The code clamp(rint(fl(fl(a / b) + c)), 0, 3) (IEEE fp32 division and addition, as the page
// evaluates it) is first formed from fma(a, 1/b, c) with 1/b from v_rcp_f32 (at most 1 ulp): that
// argument lies within a few ulps of the exact sum, which changes the rounded code only when the
// sum is within that distance of a half-integer. Those cases set `near` (exact ties among them)
// and are redone by the caller with the exact division, so the conversion of the clamped value
// to a byte (round to nearest) never meets a tie.
__device__ __forceinline__ float code_arg(float a, float rb, float c, bool& near) {
  const float sm = __builtin_fmaf(a, rb, c);
  near = near || fabsf(__builtin_amdgcn_fractf(sm) - 0.5f) < 0x1p-16f;
  return clamp03(sm);
}

constexpr int kPackWaves = 8;
constexpr int kPackUnroll = 4;  // rows a wave loads before it computes

// Wave w handles span gb = w % NG of rows w / NG, w / NG + rstep, ... (the grid holds a multiple
// of NG waves, so rstep = waves / NG). Lane l = 16 t + i holds k = tQ + 128 gb + 8i .. +7 of
// quarter t (one 16-byte load): the 16 lanes of a DPP row hold one quantisation group. Lane
// (t, i) forms the 2-bit codes of its 8 weights at bits 2t of 8 bytes; OR-ing the four quarters'
// lanes (lane ^ 16, lane ^ 32: the gfx950 permlane swaps) gives packed bytes 8i .. 8i+7, written
// by quarter 0's lane; lane i = 0 of each quarter writes its group's S and ZS.
__global__ __launch_bounds__(kPackWaves * kWave) void pack_kernel(
    const uint16_t* __restrict__ W, int64_t ldw, int N, int K, uint8_t* __restrict__ packed,
    uint16_t* __restrict__ S, uint16_t* __restrict__ ZS) {
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  const int lane = threadIdx.x & (kWave - 1);
  const int t = lane >> 4, i = lane & 15;
  const int Q = K >> 2;
  const int NG = Q / kGroup;  // 128-byte spans per packed row
  const int KG = K / kGroup;  // groups per row
  const int wid = blockIdx.x * kPackWaves + (threadIdx.x >> 6);
  const int gb = wid % NG;
  const int rstep = gridDim.x * kPackWaves / NG;
  const uint16_t* wcol = W + (int64_t)t * Q + gb * kGroup + 8 * i;
  uint8_t* pcol = packed + gb * kGroup + 8 * i;
  const int scol = t * NG + gb;
  for (int n0 = wid / NG; n0 < N; n0 += rstep * kPackUnroll) {
    u32x4 v[kPackUnroll];
#pragma unroll
    for (int j = 0; j < kPackUnroll; ++j) {
      const int n = n0 + j * rstep;
      v[j] = n < N ? *reinterpret_cast<const u32x4*>(wcol + (int64_t)n * ldw) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kPackUnroll; ++j) {
      const int n = n0 + j * rstep;
      if (n >= N) break;  // wave-uniform
      float w[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w[2 * e] = bf16_lo(v[j][e]);
        w[2 * e + 1] = bf16_hi(v[j][e]);
      }
      float lo = fminf(fminf(fminf(w[0], w[1]), fminf(w[2], w[3])), fminf(fminf(w[4], w[5]), fminf(w[6], w[7])));
      float hi = fmaxf(fmaxf(fmaxf(w[0], w[1]), fmaxf(w[2], w[3])), fmaxf(fmaxf(w[4], w[5]), fmaxf(w[6], w[7])));
      lo = row16_min(lo);
      hi = row16_max(hi);
      const float sc = fmaxf(__fdiv_rn(__fadd_rn(hi, -lo), 3.0f), 1e-8f);
      // 1 / sc can be subnormal for huge groups: such groups take the exact division throughout
      bool near = !(sc < 0x1p100f);
      const float r = __builtin_amdgcn_rcpf(sc);
      float zp = __builtin_rintf(code_arg(-lo, r, 0.0f, near));
      float q[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) q[e] = code_arg(w[e], r, zp, near);
      if (__builtin_amdgcn_ballot_w64(near) != 0ull) {
        if (near) {
          zp = clamp03(rintf(__fdiv_rn(-lo, sc)));
#pragma unroll
          for (int e = 0; e < 8; ++e) q[e] = clamp03(rintf(__fadd_rn(__fdiv_rn(w[e], sc), zp)));
        }
      }
      // codes as bytes (exact: integral or off a tie), then each quarter's at bits 2t
      uint32_t lo4 = 0, hi4 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo4 = __builtin_amdgcn_cvt_pk_u8_f32(q[e], e, lo4);
        hi4 = __builtin_amdgcn_cvt_pk_u8_f32(q[4 + e], e, hi4);
      }
      lo4 <<= 2 * t;
      hi4 <<= 2 * t;
      {
        const auto a = __builtin_amdgcn_permlane16_swap(lo4, lo4, false, false);
        lo4 |= (lane & 16) ? a[0] : a[1];
        const auto b = __builtin_amdgcn_permlane16_swap(hi4, hi4, false, false);
        hi4 |= (lane & 16) ? b[0] : b[1];
        const auto c = __builtin_amdgcn_permlane32_swap(lo4, lo4, false, false);
        lo4 |= (lane & 32) ? c[0] : c[1];
        const auto d = __builtin_amdgcn_permlane32_swap(hi4, hi4, false, false);
        hi4 |= (lane & 32) ? d[0] : d[1];
      }
      if (t == 0) {
        uint32_t* dst = reinterpret_cast<uint32_t*>(pcol + (int64_t)n * Q);
        dst[0] = lo4;
        dst[1] = hi4;
      }
      if (i == 0) {
        const float s4 = __fmul_rn(4.0f, sc);
        const float zs = __fadd_rn(s4, __fmul_rn(zp, sc));
        const int64_t at = (int64_t)n * KG + scol;
        S[at] = (uint16_t)f32_to_bf16_rne(s4);
        ZS[at] = (uint16_t)f32_to_bf16_rne(zs);
      }
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

extern "C" int i2h_pack(const uint16_t* W, int64_t ldw, int64_t N, int64_t K, uint8_t* packed,
                        uint16_t* S, uint16_t* ZS, void* stream) {
  using namespace i2h;
  if (!W || !packed || !S || !ZS) return I2H_ERR_ARG;
  if (N < 1 || check_k(K) != I2H_OK || ldw < K) return I2H_ERR_SHAPE;
  if (!aligned(W, 16) || ldw % 8 != 0 || !aligned(packed, 16) || !aligned(S, 16) || !aligned(ZS, 16))
    return I2H_ERR_ALIGN;
  if (N > (int64_t)1 << 30) return I2H_ERR_SHAPE;
  // a multiple of NG waves (each wave keeps one span), about 8 rows per wave at large N
  const int64_t NG = K / 512;
  const int64_t per = (N + 7) / 8 < 2048 ? (N + 7) / 8 : 2048;
  const int grid = (int)(NG * (per < 1 ? 1 : per));
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(kPackWaves * kWave), 0, (hipStream_t)stream, W,
                     ldw, (int)N, (int)K, packed, S, ZS);
  return check_launch();
}
