// Exact rerank of the selected tokens against the bf16 weight rows.
//
// radiance_drafthead.py, _rerank_exact: one exact logit per (row m, selected token), the dot
// of x[m] with the token's bf16 weight row, accumulated in fp32 (each bf16 x bf16 product is
// exact in fp32).
//
// One wave per (m, j): 64 lanes x 16-byte loads cover 512 k per step of both x and the
// gathered row, then a wave reduction. The gathered rows are a few hundred KB per call.
#include "device_util.h"
#include "fp8.h"
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

// The same dots against an FP8 head: rows of e4m3 bytes times a per-row fp32 scale (each weight
// one fp32 product, as radiance_drafthead.py, _rerank_exact computes it), with the lane mapping
// and summation order of rerank_kernel (8 weights per lane per 512-k step).
__global__ __launch_bounds__(256) void rerank_fp8_kernel(const uint16_t* __restrict__ x,
                                                         const uint8_t* __restrict__ W8, int64_t ldw, int N, int K,
                                                         const float* __restrict__ wscale,
                                                         const int32_t* __restrict__ sel, int M, int R,
                                                         float* __restrict__ ex) {
  typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
  const int lane = threadIdx.x & 63;
  const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= (int64_t)M * R) return;
  const int n = sel[u];
  if (n < 0 || n >= N) {
    if (lane == 0) ex[u] = -__builtin_inff();
    return;
  }
  const int m = (int)(u / R);
  const float sc = wscale[n];
  const uint16_t* xr = x + (int64_t)m * K + 8 * lane;
  const uint8_t* wr = W8 + (int64_t)n * ldw + 8 * lane;
  float acc0 = 0.f, acc1 = 0.f;
#pragma unroll 4
  for (int k0 = 0; k0 < K; k0 += 512) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + k0);
    const u32x2 wv = *reinterpret_cast<const u32x2*>(wr + k0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc0 = fmaf(bf16_lo(xv[e]), __fmul_rn(fp8_e4m3_value(byte_of(wv[0], wv[1], 2 * e)), sc), acc0);
      acc1 = fmaf(bf16_hi(xv[e]), __fmul_rn(fp8_e4m3_value(byte_of(wv[0], wv[1], 2 * e + 1)), sc), acc1);
    }
  }
  float acc = acc0 + acc1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (lane == 0) ex[u] = acc;
}

// Rerank and finalize in one kernel for R <= 64: one workgroup per row, each wave reranks
// every 16th selected token, then one wave sorts the row's R exact keys (score descending,
// token index ascending) and writes the best k. exact (optional) receives the R scores.
__global__ __launch_bounds__(1024) void rerank_finalize_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, int64_t ldw, int N, int K,
    const int32_t* __restrict__ sel, int R, int k, float* __restrict__ ex, int32_t* __restrict__ oi,
    float* __restrict__ ov) {
  __shared__ uint64_t keys[64];
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint16_t* xr = x + (int64_t)m * K + 8 * lane;
  for (int j = wave; j < R; j += 16) {
    const int n = sel[(int64_t)m * R + j];
    float acc = -__builtin_inff();
    if (n >= 0 && n < N) {
      const uint16_t* wr = W + (int64_t)n * ldw + 8 * lane;
      float a0 = 0.f, a1 = 0.f;
#pragma unroll 4
      for (int k0 = 0; k0 < K; k0 += 512) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + k0);
        const u32x4 wv = *reinterpret_cast<const u32x4*>(wr + k0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a0 = fmaf(bf16_lo(xv[e]), bf16_lo(wv[e]), a0);
          a1 = fmaf(bf16_hi(xv[e]), bf16_hi(wv[e]), a1);
        }
      }
      acc = a0 + a1;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    }
    if (lane == 0) {
      if (ex != nullptr) ex[(int64_t)m * R + j] = acc;
      keys[j] = rank_key(acc, n);
    }
  }
  __syncthreads();
  if (wave == 0) {
    uint64_t kk[1] = {lane < R ? keys[lane] : 0ull};
    wave_sort_keys<1>(kk, lane);
    if (lane < k) {
      oi[(int64_t)m * k + lane] = rank_key_idx(kk[0]);
      ov[(int64_t)m * k + lane] = rank_key_score(kk[0]);
    }
  }
}

}  // namespace

int rerank_finalize_launch(const uint16_t* x, int64_t M, const uint16_t* W, int64_t ldw, int64_t N,
                           int64_t K, const int32_t* sel, int R, int k, float* exact, int32_t* out_idx,
                           float* out_val, hipStream_t s) {
  if (R > 64) {
    if (!exact) return I2H_ERR_ARG;
    const int st = rerank_launch(x, M, W, ldw, N, K, sel, R, exact, s);
    return st != I2H_OK ? st : finalize_launch(exact, sel, M, R, k, out_idx, out_val, s);
  }
  if (!x || !W || !sel || !out_idx || !out_val) return I2H_ERR_ARG;
  if (M < 1 || M > (1 << 30) || N < 1 || N > ((int64_t)1 << 31) - 1 || check_k(K) != I2H_OK || ldw < K)
    return I2H_ERR_SHAPE;
  if (R < 1 || k < 1 || k > R) return I2H_ERR_LIMIT;
  if (!aligned(x, 16) || !aligned(W, 16) || ldw % 8 != 0 || !aligned(sel, 4) || !aligned(out_idx, 4) ||
      !aligned(out_val, 4) || (exact && !aligned(exact, 4)))
    return I2H_ERR_ALIGN;
  hipLaunchKernelGGL(rerank_finalize_kernel, dim3((unsigned)M), dim3(1024), 0, s, x, W, ldw, (int)N, (int)K, sel, R,
                     k, exact, out_idx, out_val);
  return check_launch();
}

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

int rerank_fp8_launch(const uint16_t* x, int64_t M, const uint8_t* W8, int64_t ldw, int64_t N, int64_t K,
                      const float* wscale, const int32_t* sel, int R, float* exact, hipStream_t s) {
  if (!x || !W8 || !wscale || !sel || !exact) return I2H_ERR_ARG;
  if (M < 1 || N < 1 || N > ((int64_t)1 << 31) - 1 || check_k(K) != I2H_OK || ldw < K ||
      M * R > ((int64_t)1 << 32))
    return I2H_ERR_SHAPE;
  if (R < 1 || R > I2H_MAX_R) return I2H_ERR_LIMIT;
  if (!aligned(x, 16) || !aligned(W8, 8) || ldw % 8 != 0 || !aligned(wscale, 4) || !aligned(sel, 4) ||
      !aligned(exact, 4))
    return I2H_ERR_ALIGN;
  const int64_t waves = M * R;
  hipLaunchKernelGGL(rerank_fp8_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, s, x, W8, ldw, (int)N,
                     (int)K, wscale, sel, (int)M, R, exact);
  return check_launch();
}

}  // namespace i2h

extern "C" int i2h_rerank(const uint16_t* x, int64_t M, const uint16_t* W, int64_t ldw, int64_t N,
                          int64_t K, const int32_t* sel, int R, float* exact, void* stream) {
  return i2h::rerank_launch(x, M, W, ldw, N, K, sel, R, exact, (hipStream_t)stream);
}

extern "C" int i2h_rerank_topk(const uint16_t* x, int64_t M, const uint16_t* W, int64_t ldw, int64_t N,
                               int64_t K, const int32_t* sel, int R, int k, float* exact, int32_t* out_idx,
                               float* out_val, void* stream) {
  return i2h::rerank_finalize_launch(x, M, W, ldw, N, K, sel, R, k, exact, out_idx, out_val,
                                     (hipStream_t)stream);
}

extern "C" int i2h_rerank_fp8(const uint16_t* x, int64_t M, const uint8_t* W8, int64_t ldw, int64_t N, int64_t K,
                              const float* wscale, const int32_t* sel, int R, float* exact, void* stream) {
  return i2h::rerank_fp8_launch(x, M, W8, ldw, N, K, wscale, sel, R, exact, (hipStream_t)stream);
}
