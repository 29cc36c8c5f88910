// Exact rerank of the selected tokens against the bf16 weight rows.
//
// radiance_drafthead.py, _rerank_exact: one exact logit per (row m, selected token), the dot
// of x[m] with the token's bf16 weight row, accumulated in fp32 (each bf16 x bf16 product is
// exact in fp32).
//
// One wave per (m, j): 64 lanes x 16-byte loads cover 512 k per step of both x and the
// gathered row, then a wave reduction. The gathered rows are a few hundred KB per call.
#include "device_util.h"
#include "host_util.h"

namespace i2h {
namespace {

typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__global__ __launch_bounds__(256) void rerank_kernel(const uint16_t* __restrict__ x,
                                                     const uint16_t* __restrict__ W, int64_t ldw, int N,
                                                     int K, const int32_t* __restrict__ sel, int M, int R,
                                                     float* __restrict__ ex) {
  const int lane = threadIdx.x & 63;
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= (int64_t)M * R) return;
  const int n = sel[u];
  if (n < 0 || n >= N) {
    if (lane == 0) ex[u] = -__builtin_inff();
    return;
  }
  const int m = (int)(u / R);
  const uint16_t* xr = x + (int64_t)m * K + 8 * lane;
  const uint16_t* wr = W + (int64_t)n * ldw + 8 * lane;
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 512) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + k0);
    const u32x4 wv = *reinterpret_cast<const u32x4*>(wr + k0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc0 = fmaf(bf16_lo(xv[e]), bf16_lo(wv[e]), acc0);
      acc1 = fmaf(bf16_hi(xv[e]), bf16_hi(wv[e]), acc1);
    }
  }
  float acc = acc0 + acc1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) ex[u] = acc;
}

}  // namespace

int rerank_launch(const uint16_t* x, int64_t M, const uint16_t* W, int64_t ldw, int64_t N, int64_t K,
                  const int32_t* sel, int R, float* exact, hipStream_t s) {
  if (!x || !W || !sel || !exact) return I2H_ERR_ARG;
  if (M < 1 || N < 1 || N > ((int64_t)1 << 31) - 1 || check_k(K) != I2H_OK || ldw < K ||
      M * R > ((int64_t)1 << 32))
    return I2H_ERR_SHAPE;
  if (R < 1 || R > I2H_MAX_R) return I2H_ERR_LIMIT;
  if (!aligned(x, 16) || !aligned(W, 16) || ldw % 8 != 0 || !aligned(sel, 4) || !aligned(exact, 4))
    return I2H_ERR_ALIGN;
  const int64_t waves = M * R;
  hipLaunchKernelGGL(rerank_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, x, W, ldw, (int)N,
                     (int)K, sel, (int)M, R, exact);
  return check_launch();
}

}  // namespace i2h

extern "C" int i2h_rerank(const uint16_t* x, int64_t M, const uint16_t* W, int64_t ldw, int64_t N,
                          int64_t K, const int32_t* sel, int R, float* exact, void* stream) {
  return i2h::rerank_launch(x, M, W, ldw, N, K, sel, R, exact, (hipStream_t)stream);
}
