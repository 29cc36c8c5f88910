// Quantise and pack a bf16 head into int2 quarter-split codes plus premultiplied bf16 scales.
//
// radiance_drafthead.py, _quantize_head_now: per (row n, group of 128 consecutive k) an
// asymmetric min/max quantiser at 2 bits; byte j of a packed row carries the codes of
// k = j, Q+j, 2Q+j, 3Q+j (Q = K/4); S = bf16(4 sc), ZS = bf16(4 sc + zp sc).
//
// One wave owns one (row, 128-byte span of the packed row). The span's bytes j = 128 gb + i
// (i = 0..127) draw on four quantisation groups, one per quarter t (k = tQ + 128 gb + i, group
// t*NG + gb with NG = K/512), and each lane holds two consecutive k of every quarter, so the
// wave holds all 128 values of each of its four groups: min/max are wave reductions, and the
// lane's two packed bytes come out of registers. Reads are 256 contiguous bytes per quarter.
//
// Bit-exactness: the page evaluates these steps as separate eager fp32 kernels. This file is
// built with -ffp-contract=off and correctly rounded fp32 division, and the pragma below keeps
// any multiply-add from being fused.
#include "device_util.h"
#include "host_util.h"

#pragma clang fp contract(off)

namespace i2h {
namespace {

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float clamp03(float v) { return fminf(fmaxf(v, 0.0f), 3.0f); }

constexpr int kPackWaves = 4;

__global__ __launch_bounds__(kPackWaves * kWave) void pack_kernel(
    const uint16_t* __restrict__ W, int64_t ldw, int64_t N, int K, uint8_t* __restrict__ packed,
    uint16_t* __restrict__ S, uint16_t* __restrict__ ZS) {
  const int lane = threadIdx.x & (kWave - 1);
  const int Q = K >> 2;
  const int NG = Q / kGroup;       // 128-byte spans per packed row
  const int KG = K / kGroup;       // groups per row
  const int64_t units = N * NG;
  const int64_t stride = (int64_t)gridDim.x * kPackWaves;
  for (int64_t u = (int64_t)blockIdx.x * kPackWaves + (threadIdx.x >> 6); u < units; u += stride) {
    const int64_t n = u / NG;
    const int gb = (int)(u - n * NG);
    const uint16_t* row = W + n * ldw + gb * kGroup + 2 * lane;
    uint32_t wv[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) wv[t] = *reinterpret_cast<const uint32_t*>(row + (int64_t)t * Q);
    uint32_t b0 = 0, b1 = 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float w0 = bf16_lo(wv[t]);
      const float w1 = bf16_hi(wv[t]);
      const float lo = wave_min(fminf(w0, w1));
      const float hi = wave_max(fmaxf(w0, w1));
      const float sc = fmaxf(__fdiv_rn(__fadd_rn(hi, -lo), 3.0f), 1e-8f);
      const float zp = clamp03(rintf(__fdiv_rn(-lo, sc)));
      const float q0 = clamp03(rintf(__fadd_rn(__fdiv_rn(w0, sc), zp)));
      const float q1 = clamp03(rintf(__fadd_rn(__fdiv_rn(w1, sc), zp)));
      b0 |= (uint32_t)q0 << (2 * t);
      b1 |= (uint32_t)q1 << (2 * t);
      if (lane == t) {
        const float s4 = __fmul_rn(4.0f, sc);
        const float zs = __fadd_rn(s4, __fmul_rn(zp, sc));
        const int64_t at = n * KG + (int64_t)t * NG + gb;
        S[at] = (uint16_t)f32_to_bf16_rne(s4);
        ZS[at] = (uint16_t)f32_to_bf16_rne(zs);
      }
    }
    *reinterpret_cast<uint16_t*>(packed + n * Q + gb * kGroup + 2 * lane) = (uint16_t)(b0 | (b1 << 8));
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
  const int64_t units = N * (K / 512);
  const int64_t want = (units + kPackWaves - 1) / kPackWaves;
  const int grid = (int)(want < 16384 ? want : 16384);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(kPackWaves * kWave), 0, (hipStream_t)stream, W,
                     ldw, N, (int)K, packed, S, ZS);
  return check_launch();
}
