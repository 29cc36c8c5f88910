// The drop-in logits row: the coarse bf16 row (or -inf for a top-k caller), the exact scores of
// the reranked tokens written back, the embedding bias and the cast to the head dtype.
//
// radiance_drafthead.py, _apply_head_int2 (the lines after the exact rerank): a top-k caller's
// row is set to -inf; the reranked tokens' entries take their exact scores rounded to bf16; the
// bias is added with torch's type promotion (bf16 + bf16 rounds the fp32 sum back to bf16,
// bf16 + fp16 or fp32 gives fp32) and the row is cast to the head dtype.
//
// One launch: each workgroup writes a chunk of one row (8 entries per thread) and then overwrites
// the reranked tokens that fall in that chunk, with the same finishing arithmetic applied to the
// exact score.
#include <hip/hip_fp16.h>

#include "device_util.h"
#include "host_util.h"

#pragma clang fp contract(off)

namespace i2h {
namespace {

constexpr int kLogitsThreads = 256;

// v (a bf16 value held in fp32, or -inf) at column n, after the bias and the cast, stored at out[i].
template <int BDT, int ODT>
__device__ __forceinline__ void finish(float v, int64_t n, const void* __restrict__ bias, void* __restrict__ out,
                                       int64_t i) {
  float r = v;
  if constexpr (BDT == I2H_DTYPE_BF16) {
    const float b = __uint_as_float((uint32_t)static_cast<const uint16_t*>(bias)[n] << 16);
    r = __uint_as_float(f32_to_bf16_rne(__fadd_rn(v, b)) << 16);  // bf16 + bf16 stays bf16
  } else if constexpr (BDT == I2H_DTYPE_F16) {
    r = __fadd_rn(v, __half2float(static_cast<const __half*>(bias)[n]));
  } else if constexpr (BDT == I2H_DTYPE_F32) {
    r = __fadd_rn(v, static_cast<const float*>(bias)[n]);
  }
  if constexpr (ODT == I2H_DTYPE_BF16) {
    static_cast<uint16_t*>(out)[i] = (uint16_t)f32_to_bf16_rne(r);
  } else if constexpr (ODT == I2H_DTYPE_F16) {
    static_cast<__half*>(out)[i] = __float2half_rn(r);
  } else {
    static_cast<float*>(out)[i] = r;
  }
}

// One workgroup per (row m, chunk of kChunk columns): the row pass over its columns (8 per
// thread), a barrier, then the threads t < R write back the reranked tokens that fall in the
// chunk, so every write-back lands after the row pass wrote the same entry.
constexpr int kChunk = 8 * kLogitsThreads;

template <int BDT, int ODT>
__global__ __launch_bounds__(kLogitsThreads) void logits_kernel(const uint16_t* __restrict__ y, int64_t N,
                                                                const int32_t* __restrict__ sel,
                                                                const float* __restrict__ exact, int R,
                                                                const void* __restrict__ bias, void* __restrict__ out) {
  typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
  const int64_t m = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  const int64_t n0 = c0 + 8 * threadIdx.x;
  const int64_t row = m * N;
  if (n0 < N) {
    uint32_t w[4] = {0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};  // -inf: the top-k caller's row
    if (y != nullptr) {
      if (n0 + 8 <= N && (N & 7) == 0) {  // 16-byte aligned: every row starts on a multiple of 8
        const u32x4 v = *reinterpret_cast<const u32x4*>(y + row + n0);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = v[e];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (n0 + e < N) w[e >> 1] = (w[e >> 1] & ~(0xffffu << (16 * (e & 1)))) | ((uint32_t)y[row + n0 + e] << (16 * (e & 1)));
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (n0 + e < N) finish<BDT, ODT>((e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]), n0 + e, bias, out, row + n0 + e);
  }
  __syncthreads();  // the row pass of this chunk is done (workgroup-scope release/acquire)
  for (int t = threadIdx.x; t < R; t += kLogitsThreads) {
    const int32_t n = sel[m * R + t];
    if (n >= c0 && n < c0 + kChunk && n < N) {
      const float v = __uint_as_float(f32_to_bf16_rne(exact[m * R + t]) << 16);  // the exact score as bf16
      finish<BDT, ODT>(v, n, bias, out, row + n);
    }
  }
}

template <int BDT, int ODT>
int launch_logits(const uint16_t* y, int64_t M, int64_t N, const int32_t* sel, const float* exact, int R,
                  const void* bias, void* out, hipStream_t s) {
  const dim3 grid((unsigned)((N + kChunk - 1) / kChunk), (unsigned)M);
  hipLaunchKernelGGL((logits_kernel<BDT, ODT>), grid, dim3(kLogitsThreads), 0, s, y, N, sel, exact, R, bias, out);
  return check_launch();
}

template <int BDT>
int dispatch_out(int out_dtype, const uint16_t* y, int64_t M, int64_t N, const int32_t* sel, const float* exact,
                 int R, const void* bias, void* out, hipStream_t s) {
  switch (out_dtype) {
    case I2H_DTYPE_BF16: return launch_logits<BDT, I2H_DTYPE_BF16>(y, M, N, sel, exact, R, bias, out, s);
    case I2H_DTYPE_F16: return launch_logits<BDT, I2H_DTYPE_F16>(y, M, N, sel, exact, R, bias, out, s);
    default: return launch_logits<BDT, I2H_DTYPE_F32>(y, M, N, sel, exact, R, bias, out, s);
  }
}

int dtype_bytes(int dt) { return dt == I2H_DTYPE_F32 ? 4 : 2; }

}  // namespace
}  // namespace i2h

extern "C" int i2h_logits(const uint16_t* y, int64_t M, int64_t N, const int32_t* sel, const float* exact, int R,
                          int topk_only, const void* bias, int bias_dtype, void* out, int out_dtype, void* stream) {
  using namespace i2h;
  if (!out || !sel || !exact || (!topk_only && !y)) return I2H_ERR_ARG;
  if (bias_dtype < I2H_DTYPE_NONE || bias_dtype > I2H_DTYPE_F32 || (bias_dtype == I2H_DTYPE_NONE) != (bias == nullptr))
    return I2H_ERR_ARG;
  if (out_dtype < I2H_DTYPE_BF16 || out_dtype > I2H_DTYPE_F32) return I2H_ERR_ARG;
  if (M < 1 || N < 1 || M > 65535 || N > ((int64_t)1 << 40)) return I2H_ERR_SHAPE;
  if (R < 1 || R > I2H_MAX_R) return I2H_ERR_LIMIT;
  if ((y && !aligned(y, 16)) || !aligned(out, 16) || !aligned(sel, 4) || !aligned(exact, 4) ||
      (bias && !aligned(bias, dtype_bytes(bias_dtype))))
    return I2H_ERR_ALIGN;
  const uint16_t* yr = topk_only ? nullptr : y;
  const hipStream_t s = (hipStream_t)stream;
  switch (bias_dtype) {
    case I2H_DTYPE_NONE: return dispatch_out<I2H_DTYPE_NONE>(out_dtype, yr, M, N, sel, exact, R, bias, out, s);
    case I2H_DTYPE_BF16: return dispatch_out<I2H_DTYPE_BF16>(out_dtype, yr, M, N, sel, exact, R, bias, out, s);
    case I2H_DTYPE_F16: return dispatch_out<I2H_DTYPE_F16>(out_dtype, yr, M, N, sel, exact, R, bias, out, s);
    default: return dispatch_out<I2H_DTYPE_F32>(out_dtype, yr, M, N, sel, exact, R, bias, out, s);
  }
}
