// The design alternatives the head is measured against: their packs, group sums, and the entry
// point that runs each of them through the production coarse kernels.
//
// radiance_drafthead.py, module docstring: group 128 against group 64 (twice the scales, and the
// per-group scale and zero work on the accumulator doubles); quarter-split packing against a
// contiguous-4 byte layout (byte j holding k = 4j .. 4j+3); the scale applied to the accumulator
// against dequantising the weight tile (every weight S (1 + v/4) - ZS in fp32, rounded to bf16,
// before the dot).
//
// The coarse alternatives live in the production kernels themselves (coarse.hip one-row kernel,
// coarse_tile.hip 16-row tile, selected by a template parameter, ablation.h), so that each differs
// from the chosen design in one property only and the design member is the production kernel.
//
// Pack kernel (load time): one 256-thread workgroup per (row, span), the page's quantiser with
// IEEE fp32 division (this file is built with correctly rounded division and no contraction),
// bit-exact against the eager fp32 steps.
#include "ablation.h"
#include "dequant.h"
#include "host_util.h"

namespace i2h {
namespace {

constexpr int kQuarter = 0, kContig = 1;
constexpr int kAcc = 0, kTile = 1;
constexpr int kVThreads = 256;

// ---------------------------------------------------------------------------------------------
// pack
// ---------------------------------------------------------------------------------------------
template <int G, int LAYOUT>
__global__ __launch_bounds__(kVThreads) void pack_variant_kernel(const uint16_t* __restrict__ W, int64_t ldw, int K,
                                                                 int nsp, uint8_t* __restrict__ packed,
                                                                 uint16_t* __restrict__ S, uint16_t* __restrict__ ZS) {
  __shared__ float w[4 * G];
  __shared__ float scs[4], zps[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = blockIdx.x / nsp;
  const int sp = blockIdx.x - (int)(n * nsp);
  const int Q = K / 4, KG = K / G;
  // group i of the span starts at k0(i): quarter i's group sp, or the span's i-th group
  auto k0 = [&](int i) { return LAYOUT == kQuarter ? i * Q + G * sp : G * (4 * sp + i); };
  const uint16_t* row = W + n * ldw;
  for (int e = tid; e < 4 * G; e += kVThreads) w[e] = bf16_lo(row[k0(e / G) + e % G]);
  __syncthreads();
  {  // wave i: min / max of group i, then its scale and zero point
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int j = lane; j < G; j += kWave) {
      lo = fminf(lo, w[wave * G + j]);
      hi = fmaxf(hi, w[wave * G + j]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      lo = fminf(lo, __shfl_xor(lo, o));
      hi = fmaxf(hi, __shfl_xor(hi, o));
    }
    if (lane == 0) {
      const float sc = fmaxf((hi - lo) / 3.0f, 1e-8f);
      const float zp = fminf(fmaxf(rintf(-lo / sc), 0.0f), 3.0f);
      scs[wave] = sc;
      zps[wave] = zp;
      const float s4 = 4.0f * sc;
      const int64_t gi = n * KG + k0(wave) / G;
      S[gi] = (uint16_t)f32_to_bf16_rne(s4);
      ZS[gi] = (uint16_t)f32_to_bf16_rne(s4 + zp * sc);
    }
  }
  __syncthreads();
  // G output bytes per span: quarter-split byte b holds element b of each group (field i = group
  // i); contiguous byte b holds span elements 4b .. 4b + 3 (group (4b + f) / G)
  for (int b = tid; b < G; b += kVThreads) {
    uint32_t byte = 0;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const int e = LAYOUT == kQuarter ? f * G + b : 4 * b + f;
      const int i = e / G;
      const float t = w[e] / scs[i] + zps[i];
      const float q = fminf(fmaxf(rintf(t), 0.0f), 3.0f);
      byte |= (uint32_t)q << (2 * f);
    }
    packed[n * Q + G * sp + b] = (uint8_t)byte;
  }
}

// ---------------------------------------------------------------------------------------------
// group sums of x at group G
// ---------------------------------------------------------------------------------------------
template <int G>
__global__ __launch_bounds__(kVThreads) void xsum_group_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                               float* __restrict__ xs) {
  const int KG = K / G, lane = threadIdx.x & 63;
  const int64_t u = (int64_t)blockIdx.x * (kVThreads / kWave) + (threadIdx.x >> 6);
  if (u >= (int64_t)M * KG) return;
  const int64_t m = u / KG;
  const int g = (int)(u - m * KG);
  const uint16_t* p = x + m * K + (int64_t)g * G;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < G / kWave; ++j) s += bf16_lo(p[lane + kWave * j]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) xs[u] = s;
}

bool group_ok(int g) { return g == 64 || g == 128; }

}  // namespace
}  // namespace i2h

extern "C" int i2h_pack_variant(const uint16_t* W, int64_t ldw, int64_t N, int64_t K, int group, int layout,
                                uint8_t* packed, uint16_t* S, uint16_t* ZS, void* stream) {
  using namespace i2h;
  if (!W || !packed || !S || !ZS) return I2H_ERR_ARG;
  if (!group_ok(group) || (layout != kQuarter && layout != kContig)) return I2H_ERR_ARG;
  if (N < 1 || K <= 0 || K % (4 * group) != 0 || K > I2H_MAX_K || ldw < K) return I2H_ERR_SHAPE;
  const int64_t nsp = K / (4 * group);
  if (N * nsp > 0x7fffffff) return I2H_ERR_SHAPE;
  if (!aligned(W, 2) || !aligned(S, 2) || !aligned(ZS, 2)) return I2H_ERR_ALIGN;
  const dim3 grid((unsigned)(N * nsp));
  const hipStream_t s = (hipStream_t)stream;
  if (group == 128) {
    if (layout == kQuarter)
      hipLaunchKernelGGL((pack_variant_kernel<128, kQuarter>), grid, dim3(kVThreads), 0, s, W, ldw, (int)K, (int)nsp,
                         packed, S, ZS);
    else
      hipLaunchKernelGGL((pack_variant_kernel<128, kContig>), grid, dim3(kVThreads), 0, s, W, ldw, (int)K, (int)nsp,
                         packed, S, ZS);
  } else {
    if (layout == kQuarter)
      hipLaunchKernelGGL((pack_variant_kernel<64, kQuarter>), grid, dim3(kVThreads), 0, s, W, ldw, (int)K, (int)nsp,
                         packed, S, ZS);
    else
      hipLaunchKernelGGL((pack_variant_kernel<64, kContig>), grid, dim3(kVThreads), 0, s, W, ldw, (int)K, (int)nsp,
                         packed, S, ZS);
  }
  return check_launch();
}

extern "C" int i2h_xsum_group(const uint16_t* x, int64_t M, int64_t K, int group, float* xs, void* stream) {
  using namespace i2h;
  if (!x || !xs || !group_ok(group)) return I2H_ERR_ARG;
  if (M < 1 || K <= 0 || K % group != 0 || K > I2H_MAX_K || M * (K / group) > ((int64_t)1 << 30)) return I2H_ERR_SHAPE;
  if (!aligned(x, 2) || !aligned(xs, 4)) return I2H_ERR_ALIGN;
  const int64_t units = M * (K / group);
  const dim3 grid((unsigned)((units + 3) / 4));
  if (group == 128)
    hipLaunchKernelGGL(xsum_group_kernel<128>, grid, dim3(kVThreads), 0, (hipStream_t)stream, x, (int)M, (int)K, xs);
  else
    hipLaunchKernelGGL(xsum_group_kernel<64>, grid, dim3(kVThreads), 0, (hipStream_t)stream, x, (int)M, (int)K, xs);
  return check_launch();
}

extern "C" int i2h_coarse_variant_topk(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed,
                                       const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int group,
                                       int layout, int scaling, int kcand, float* cand_score, int32_t* cand_idx,
                                       void* stream) {
  using namespace i2h;
  if (!x || !packed || !S || !ZS || !cand_score || !cand_idx) return I2H_ERR_ARG;
  if (!group_ok(group) || (layout != kQuarter && layout != kContig) || (scaling != kAcc && scaling != kTile))
    return I2H_ERR_ARG;
  // one property changed at a time
  int var;
  if (group == 128 && layout == kQuarter && scaling == kAcc) var = kVarDesign;
  else if (group == 64 && layout == kQuarter && scaling == kAcc) var = kVarG64;
  else if (group == 128 && layout == kContig && scaling == kAcc) var = kVarC4;
  else if (group == 128 && layout == kQuarter && scaling == kTile) var = kVarWTile;
  else return I2H_ERR_ARG;
  if (M < 1 || M > 16 || N < 1 || N > ((int64_t)1 << 30) || (K != 512 && K != 5120)) return I2H_ERR_SHAPE;
  if (kcand < 1 || kcand > I2H_MAX_KCAND) return I2H_ERR_LIMIT;
  if (!aligned(x, 16) || !aligned(packed, 16) || (xs && !aligned(xs, 4)) || !aligned(S, 16) || !aligned(ZS, 16) ||
      !aligned(cand_score, 4) || !aligned(cand_idx, 4))
    return I2H_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  const float* xsv = var == kVarWTile ? nullptr : xs;
  if (M == 1) return small_variant_launch(var, x, xsv, packed, S, ZS, N, K, kcand, cand_score, cand_idx, s);
  return tile_variant_launch(var, x, xsv, M, packed, S, ZS, N, K, kcand, cand_score, cand_idx, s);
}
