// Coarse int2 logits with the fused block top-KCAND emit, and the per-group sums of x.
//
// radiance_drafthead.py, _draft_head_int2 / _emit and the module docstring:
//   * the 2-bit code v of a weight is read as the bf16 value 1 + v/4 straight from its bits
//     (0x3F80 | v << 5), so the dot over a group returns sum x + dot(x, v)/4;
//   * each group g of 128 k then contributes S[n,g] * P - xs[m,g] * ZS[n,g], with the scale
//     and zero applied to the [rows, columns] accumulator, never to the weight tile;
//   * every 64-column block emits its KCAND best columns per row.
//
// Layout on gfx950. A workgroup (4 waves) owns one 64-column block; wave w owns columns
// 64b + 16w .. +15 and every row of x (up to 16*MT rows per launch). The contraction runs on
// v_mfma_f32_16x16x32_bf16: A = 16 rows of x, B = 16 columns of dequantised weights, and lane
// (col = l & 15, h = l >> 4) feeds column col with k-slots 8h .. 8h+7. A lane streams 32
// consecutive packed bytes of its row per 128-byte span (two 16-byte loads); the 8 bytes of
// slice s serve all four quarters t, i.e. the k-slots t*Q + 128 gb + 32h + 8s + (0..7) of four
// different quantisation groups, each with its own MFMA accumulator that is scaled and folded
// into the result once the group is complete. A byte permute puts bytes (0,2,1,3) of each
// dword in place so that the bit-pattern dequant yields bf16 pairs in natural k order, which
// lets the x fragment be one contiguous 16-byte load.
#include "device_util.h"
#include "host_util.h"

namespace i2h {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

constexpr int kCoarseThreads = 256;  // 4 waves x 16 columns = one 64-column block

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Bytes [b0 b1 b2 b3] -> [b0 b2 b1 b3].
__device__ __forceinline__ uint32_t pair_bytes(uint32_t d) { return __builtin_amdgcn_perm(d, d, 0x03010200u); }

// Eight weights of quarter T as bf16 1 + v/4, natural k order; d0/d1 are byte-paired dwords.
template <int T>
__device__ __forceinline__ bf16x8 dequant8(uint32_t d0, uint32_t d1) {
  constexpr uint32_t kMask = 0x00600060u, kOne = 0x3F803F80u;
  u32x4 r;
  if constexpr (T < 3) {
    r[0] = ((d0 << (5 - 2 * T)) & kMask) | kOne;
    r[2] = ((d1 << (5 - 2 * T)) & kMask) | kOne;
  } else {
    r[0] = ((d0 >> 1) & kMask) | kOne;
    r[2] = ((d1 >> 1) & kMask) | kOne;
  }
  r[1] = ((d0 >> (3 + 2 * T)) & kMask) | kOne;
  r[3] = ((d1 >> (3 + 2 * T)) & kMask) | kOne;
  return __builtin_bit_cast(bf16x8, r);
}

// One quarter T of one 128-byte span: 4 MFMAs per m-tile, then the group's scale and zero.
template <int MT, int T>
__device__ __forceinline__ void quarter(f32x4 (&acc)[MT], const uint32_t (&dw)[8], const uint16_t* xq,
                                        int M, int K, int col, float sv, float zv, const float* xsg,
                                        int h) {
  f32x4 p[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) p[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8 b = dequant8<T>(dw[2 * s], dw[2 * s + 1]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = mt * 16 + col;
      u32x4 a = {0u, 0u, 0u, 0u};
      if (m < M) a = ld16(xq + (int64_t)m * K + 8 * s);
      p[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, p[mt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const f32x4 xv = *reinterpret_cast<const f32x4*>(xsg + mt * 16 + 4 * h);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float a = fmaf(sv, p[mt][r], acc[mt][r]);
      acc[mt][r] = fmaf(-xv[r], zv, a);
    }
  }
}

// Descending bitonic sort across the wave of (value, column) pairs; better = larger value,
// then lower column. Afterwards lane r holds the r-th best.
__device__ __forceinline__ void wave_sort_desc(float& v, int& c, int lane) {
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const float ov = __shfl_xor(v, stride);
      const int oc = __shfl_xor(c, stride);
      const bool lower = (lane & stride) == 0;
      const bool desc = (lane & size) == 0;
      const bool other_better = (ov > v) || (ov == v && oc < c);
      if ((lower == desc) == other_better) {
        v = ov;
        c = oc;
      }
    }
  }
}

template <int MT>
__global__ __launch_bounds__(kCoarseThreads) void coarse_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ xs, int M,
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ S,
    const uint16_t* __restrict__ ZS, int N, int K, int kc, int nblk, float* __restrict__ cand_score,
    int32_t* __restrict__ cand_idx, uint16_t* __restrict__ y) {
  constexpr int MR = 16 * MT;
  extern __shared__ float smem[];
  const int Q = K >> 2, NG = Q / kGroup, KG = K / kGroup;
  float* xsT = smem;              // [KG][MR]: xs transposed, zero past row M
  float* cbuf = smem + KG * MR;   // [MR][64]: the block's logits for the emit
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, h = lane >> 4;
  const int b = blockIdx.x;
  const int n = b * kBlockN + wave * 16 + col;
  const bool nvalid = n < N;
  const int nr = nvalid ? n : 0;

  for (int i = tid; i < KG * MR; i += kCoarseThreads) {
    const int g = i / MR, m = i - g * MR;
    xsT[i] = m < M ? xs[(int64_t)m * KG + g] : 0.f;
  }
  __syncthreads();

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint8_t* prow = packed + (int64_t)nr * Q + 32 * h;
  const uint16_t* srow = S + (int64_t)nr * KG;
  const uint16_t* zrow = ZS + (int64_t)nr * KG;
  const uint16_t* xh = x + 32 * h;

  for (int gb = 0; gb < NG; ++gb) {
    u32x4 p0 = {0u, 0u, 0u, 0u}, p1 = {0u, 0u, 0u, 0u};
    if (nvalid) {
      p0 = ld16(prow + gb * kGroup);
      p1 = ld16(prow + gb * kGroup + 16);
    }
    uint32_t dw[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dw[i] = pair_bytes(p0[i]);
      dw[4 + i] = pair_bytes(p1[i]);
    }
    const uint16_t* xg = xh + gb * kGroup;
    quarter<MT, 0>(acc, dw, xg, M, K, col, bf16_lo(srow[gb]), bf16_lo(zrow[gb]), xsT + gb * MR, h);
    quarter<MT, 1>(acc, dw, xg + Q, M, K, col, bf16_lo(srow[NG + gb]), bf16_lo(zrow[NG + gb]),
                   xsT + (NG + gb) * MR, h);
    quarter<MT, 2>(acc, dw, xg + 2 * Q, M, K, col, bf16_lo(srow[2 * NG + gb]),
                   bf16_lo(zrow[2 * NG + gb]), xsT + (2 * NG + gb) * MR, h);
    quarter<MT, 3>(acc, dw, xg + 3 * Q, M, K, col, bf16_lo(srow[3 * NG + gb]),
                   bf16_lo(zrow[3 * NG + gb]), xsT + (3 * NG + gb) * MR, h);
  }

  // acc[mt][r] is c[m = 16 mt + 4 h + r][n]
  if (y != nullptr && nvalid) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = mt * 16 + 4 * h + r;
        if (m < M) y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(acc[mt][r]);
      }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      cbuf[(mt * 16 + 4 * h + r) * kBlockN + wave * 16 + col] = nvalid ? acc[mt][r] : -__builtin_inff();
  __syncthreads();

  const int64_t ld = (int64_t)nblk * kc;
  for (int m = wave; m < M; m += kCoarseThreads / kWave) {
    float v = cbuf[m * kBlockN + lane];
    int c = lane;
    wave_sort_desc(v, c, lane);
    if (lane < kc) {
      const int tok = b * kBlockN + c;
      const bool ok = tok < N;
      const int64_t at = (int64_t)m * ld + (int64_t)b * kc + lane;
      cand_score[at] = ok ? v : -__builtin_inff();
      cand_idx[at] = ok ? tok : -1;
    }
  }
}

__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                   float* __restrict__ xs) {
  const int KG = K / kGroup;
  const int lane = threadIdx.x & 63;
  const int u = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (u >= M * KG) return;
  const int m = u / KG, g = u - m * KG;
  const uint32_t v = *reinterpret_cast<const uint32_t*>(x + (int64_t)m * K + g * kGroup + 2 * lane);
  float s = bf16_lo(v) + bf16_hi(v);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) xs[(int64_t)m * KG + g] = s;
}

template <int MT>
int launch_coarse(const uint16_t* x, const float* xs, int M, const uint8_t* packed, const uint16_t* S,
                  const uint16_t* ZS, int N, int K, int kc, float* cs, int32_t* ci, uint16_t* y,
                  hipStream_t s) {
  const int nblk = (int)nblk_of(N);
  const size_t lds = (size_t)(K / kGroup) * 16 * MT * 4 + (size_t)16 * MT * kBlockN * 4;
  hipLaunchKernelGGL(coarse_kernel<MT>, dim3(nblk), dim3(kCoarseThreads), lds, s, x, xs, M, packed, S,
                     ZS, N, K, kc, nblk, cs, ci, y);
  return check_launch();
}

// Largest m-tile count whose LDS footprint (xs transposed + the block's logits) fits in 64 KiB.
int max_mtiles(int64_t K) {
  int mt = 8;
  while (mt > 1 && ((K / kGroup) * 16 * mt * 4 + 16 * mt * kBlockN * 4) > 65536) mt >>= 1;
  return mt;
}

}  // namespace

int xsum_launch(const uint16_t* x, int64_t M, int64_t K, float* xs, hipStream_t s) {
  if (!x || !xs) return I2H_ERR_ARG;
  if (M < 1 || check_k(K) != I2H_OK || M * (K / kGroup) > (int64_t)1 << 30) return I2H_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(xs, 4)) return I2H_ERR_ALIGN;
  const int64_t units = M * (K / kGroup);
  hipLaunchKernelGGL(xsum_kernel, dim3((unsigned)((units + 3) / 4)), dim3(256), 0, s, x, (int)M, (int)K, xs);
  return check_launch();
}

int coarse_launch(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed,
                  const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int kcand,
                  float* cand_score, int32_t* cand_idx, uint16_t* y, hipStream_t s) {
  if (!x || !xs || !packed || !S || !ZS || !cand_score || !cand_idx) return I2H_ERR_ARG;
  if (M < 1 || N < 1 || N > ((int64_t)1 << 30) || check_k(K) != I2H_OK) return I2H_ERR_SHAPE;
  if (kcand < 1 || kcand > I2H_MAX_KCAND) return I2H_ERR_LIMIT;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(xs, 4) || !aligned(S, 2) || !aligned(ZS, 2) ||
      !aligned(cand_score, 4) || !aligned(cand_idx, 4) || (y && !aligned(y, 2)))
    return I2H_ERR_ALIGN;
  const int64_t ld = nblk_of(N) * kcand;
  const int64_t rows_max = 16 * max_mtiles(K);
  for (int64_t m0 = 0; m0 < M; m0 += rows_max) {
    const int mc = (int)(M - m0 < rows_max ? M - m0 : rows_max);
    const uint16_t* xc = x + m0 * K;
    const float* xsc = xs + m0 * (K / kGroup);
    float* csc = cand_score + m0 * ld;
    int32_t* cic = cand_idx + m0 * ld;
    uint16_t* yc = y ? y + m0 * N : nullptr;
    int st;
    if (mc <= 16)
      st = launch_coarse<1>(xc, xsc, mc, packed, S, ZS, (int)N, (int)K, kcand, csc, cic, yc, s);
    else if (mc <= 32)
      st = launch_coarse<2>(xc, xsc, mc, packed, S, ZS, (int)N, (int)K, kcand, csc, cic, yc, s);
    else if (mc <= 64)
      st = launch_coarse<4>(xc, xsc, mc, packed, S, ZS, (int)N, (int)K, kcand, csc, cic, yc, s);
    else
      st = launch_coarse<8>(xc, xsc, mc, packed, S, ZS, (int)N, (int)K, kcand, csc, cic, yc, s);
    if (st != I2H_OK) return st;
  }
  return I2H_OK;
}

}  // namespace i2h

extern "C" int i2h_xsum(const uint16_t* x, int64_t M, int64_t K, float* xs, void* stream) {
  return i2h::xsum_launch(x, M, K, xs, (hipStream_t)stream);
}

extern "C" int i2h_coarse_topk(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed,
                               const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int kcand,
                               float* cand_score, int32_t* cand_idx, uint16_t* y, void* stream) {
  return i2h::coarse_launch(x, xs, M, packed, S, ZS, N, K, kcand, cand_score, cand_idx, y,
                            (hipStream_t)stream);
}
