// The design alternatives the head is measured against, built as one kernel family so that each
// differs from the chosen design in one property only.
//
// radiance_drafthead.py, module docstring: group 128 against group 64 (the per-group scale and
// zero work on the accumulator doubles at 64); quarter-split packing against a contiguous-4 byte
// layout (byte j holding k = 4j .. 4j+3, so the lanes of a column gather short runs instead of
// streaming one); the scale applied to the accumulator against dequantising the weight tile
// (every weight becomes S (1 + v/4) - ZS in fp32, rounded to bf16, before the dot).
//
// Coarse kernel: one 4-wave workgroup per 64-column block, at most 16 rows of x (one MFMA tile);
// lane (col = l & 15, h = l >> 4). A span is 4 groups: in the quarter-split layout group gb of
// each quarter (the lane's G/4 bytes of the row serve all four), in the contiguous layout 4
// consecutive groups (the lane takes G/16 bytes of each). Every group instance is G/32 MFMAs
// (16x16x32 bf16) over k0 + (G/4) h + 8 s .. + 8, the same k slots in both layouts, so the
// x fragments are addressed alike. The block's S and ZS are staged in LDS once per workgroup (so
// both layouts read a group's scales the same way), and so are up to 4 rows of x, when they fit
// in 64 KiB with the rest (otherwise they are read from L2); the next span's bytes and scales are loaded one span ahead. The emit is
// the int4 kernel's (a wave bitonic sort).
//
// Pack kernel (load time): one 256-thread workgroup per (row, span), the page's quantiser with
// IEEE fp32 division (this file is built with correctly rounded division and no contraction),
// bit-exact against the eager fp32 steps.
#include "dequant.h"
#include "host_util.h"
#include "wave_sort.h"

namespace i2h {
namespace {

constexpr int kQuarter = 0, kContig = 1;
constexpr int kAcc = 0, kTile = 1;
constexpr int kVThreads = 256;

typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

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

// ---------------------------------------------------------------------------------------------
// coarse logits + block emit
// ---------------------------------------------------------------------------------------------
// bf16 1 + v/4 of the 2-bit field at bit `sh` of the low and high half of p: the quarter-split
// form, where the two bytes of a bf16 pair sit at the same place in either half after pairing.
template <int SH>
__device__ __forceinline__ uint32_t pair_field(uint32_t p) {
  const uint32_t a = SH <= 5 ? (p << (5 - SH)) : (p >> (SH - 5));
  return (a & 0x00600060u) | 0x3F803F80u;
}

// Eight weights (slice s) of group instance i in natural k order, as bf16 1 + v/4.
template <int G, int LAYOUT>
__device__ __forceinline__ u32x4 codes8(const uint32_t* d, int i, int s) {
  u32x4 r;
  if constexpr (LAYOUT == kQuarter) {
    // bytes 8s .. 8s + 7 of the lane's run, field i of each
    const uint32_t p0 = __builtin_amdgcn_perm(d[2 * s], d[2 * s], 0x03010200u);  // [b0 b2 b1 b3]
    const uint32_t p1 = __builtin_amdgcn_perm(d[2 * s + 1], d[2 * s + 1], 0x03010200u);
    switch (i) {
      case 0: r = u32x4{pair_field<0>(p0), pair_field<8>(p0), pair_field<0>(p1), pair_field<8>(p1)}; break;
      case 1: r = u32x4{pair_field<2>(p0), pair_field<10>(p0), pair_field<2>(p1), pair_field<10>(p1)}; break;
      case 2: r = u32x4{pair_field<4>(p0), pair_field<12>(p0), pair_field<4>(p1), pair_field<12>(p1)}; break;
      default: r = u32x4{pair_field<6>(p0), pair_field<14>(p0), pair_field<6>(p1), pair_field<14>(p1)}; break;
    }
  } else {
    // bytes 2s, 2s + 1 of the lane's run for group i: 8 consecutive k, two per nibble
    constexpr int RW = G / 64;  // dwords per run (2 for G = 128, 1 for G = 64)
    const uint32_t hw = (d[i * RW + (s >> 1)] >> (16 * (s & 1))) & 0xffffu;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t t = hw >> (4 * j);
      r[j] = ((t << 5) & 0x60u) | ((t << 19) & 0x00600000u) | 0x3F803F80u;
    }
  }
  return r;
}

// The dequantised tile: each weight S (1 + v/4) - ZS in fp32 (the product is exact), rounded to bf16.
__device__ __forceinline__ bf16x8 tile8(const u32x4& c, float sv, float zv) {
  bf16x8 o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    o[2 * j] = (__bf16)__fsub_rn(__fmul_rn(sv, bf16_lo(c[j])), zv);
    o[2 * j + 1] = (__bf16)__fsub_rn(__fmul_rn(sv, bf16_hi(c[j])), zv);
  }
  return o;
}

constexpr int kVXRows = 4;  // rows of x staged in LDS

template <int G, int LAYOUT, int SCALE, bool XL, bool SZL>
__global__ __launch_bounds__(kVThreads) void coarse_variant_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ xs, int M, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ S, const uint16_t* __restrict__ ZS, int N, int K, int kc, int nblk,
    float* __restrict__ cand_score, int32_t* __restrict__ cand_idx) {
  constexpr int LB = G / 4;    // bytes of a row a lane reads per span
  constexpr int NW = LB / 4;   // as dwords
  constexpr int NSL = G / 32;  // MFMAs per group instance
  extern __shared__ float smem[];
  const int KG = K / G, Q = K / 4, nsp = K / (4 * G);
  float* xsT = smem;                                          // [KG][16] (accumulator scaling)
  float* cbuf = smem + (SCALE == kAcc ? KG * 16 : 0);         // [16][64]
  uint32_t* szl = reinterpret_cast<uint32_t*>(cbuf + 16 * kBlockN);  // [KG][64] S | ZS << 16 when SZL
  uint16_t* xl = reinterpret_cast<uint16_t*>(szl + (SZL ? KG * kBlockN : 0));  // [M][K] when XL
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, h = lane >> 4;
  const int b = blockIdx.x;
  const int n = b * kBlockN + wave * 16 + col;
  const bool nvalid = n < N;
  const int nr = nvalid ? n : 0;
  if constexpr (SCALE == kAcc) {
    for (int i = tid; i < KG * 16; i += kVThreads) {
      const int g = i >> 4, m = i & 15;
      xsT[i] = m < M ? xs[(int64_t)m * KG + g] : 0.f;
    }
  }
  if constexpr (XL) {
    for (int i = tid; i < M * K / 8; i += kVThreads)
      *reinterpret_cast<u32x4*>(xl + 8 * i) = ld16(x + 8 * (int64_t)i);
  }
  if constexpr (SZL) {
    for (int i = tid; i < KG * kBlockN; i += kVThreads) {
      const int r = i / KG, g = i - r * KG;
      const int nn = b * kBlockN + r;
      const int64_t at = (int64_t)(nn < N ? nn : 0) * KG + g;
      szl[g * kBlockN + r] = (uint32_t)S[at] | ((uint32_t)ZS[at] << 16);
    }
  }
  if constexpr (SCALE == kAcc || XL || SZL) __syncthreads();
  const uint8_t* prow = packed + (int64_t)nr * Q;
  const uint16_t* srow = S + (int64_t)nr * KG;
  const uint16_t* zrow = ZS + (int64_t)nr * KG;
  // rows past M read row 0, unused
  const uint16_t* xr = (XL ? xl : x) + (int64_t)(col < M ? col : 0) * K + LB * h;

  auto gidx = [&](int sp, int i) { return LAYOUT == kQuarter ? i * nsp + sp : 4 * sp + i; };
  auto fetch = [&](int sp, uint32_t (&d)[NW], float (&sv)[4], float (&zv)[4]) {
    if constexpr (LAYOUT == kQuarter) {
#pragma unroll
      for (int j = 0; j < NW / 4; ++j) {
        const u32x4 v = ld16(prow + G * sp + LB * h + 16 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) d[4 * j + e] = v[e];
      }
    } else if constexpr (G == 128) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x2 v = *reinterpret_cast<const u32x2*>(prow + G * sp + 32 * i + 8 * h);
        d[2 * i] = v[0];
        d[2 * i + 1] = v[1];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = *reinterpret_cast<const uint32_t*>(prow + G * sp + 16 * i + 4 * h);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (SZL) {
        const uint32_t v = szl[gidx(sp, i) * kBlockN + wave * 16 + col];
        sv[i] = bf16_lo(v);
        zv[i] = bf16_hi(v);
      } else {
        sv[i] = bf16_lo(srow[gidx(sp, i)]);
        zv[i] = bf16_lo(zrow[gidx(sp, i)]);
      }
    }
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  uint32_t dc[NW], dn[NW];
  float sc[4], zc[4], sn[4], zn[4];
  fetch(0, dc, sc, zc);
  for (int sp = 0; sp < nsp; ++sp) {
    fetch(sp + 1 < nsp ? sp + 1 : sp, dn, sn, zn);
    u32x4 xa[4][NSL];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = LAYOUT == kQuarter ? i * Q + G * sp : G * (4 * sp + i);
#pragma unroll
      for (int s = 0; s < NSL; ++s) xa[i][s] = ld16(xr + k0 + 8 * s);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (SCALE == kAcc) {
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NSL; ++s)
          p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[i][s]),
                                                      __builtin_bit_cast(bf16x8, codes8<G, LAYOUT>(dc, i, s)), p, 0,
                                                      0, 0);
        const f32x4 xv = *reinterpret_cast<const f32x4*>(xsT + gidx(sp, i) * 16 + 4 * h);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = fmaf(-xv[r], zc[i], fmaf(sc[i], p[r], acc[r]));
      } else {
#pragma unroll
        for (int s = 0; s < NSL; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xa[i][s]),
                                                        tile8(codes8<G, LAYOUT>(dc, i, s), sc[i], zc[i]), acc, 0, 0,
                                                        0);
      }
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) dc[j] = dn[j];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = sn[i];
      zc[i] = zn[i];
    }
  }

  // acc[r] is c[m = 4 h + r][n]
#pragma unroll
  for (int r = 0; r < 4; ++r) cbuf[(4 * h + r) * kBlockN + wave * 16 + col] = nvalid ? acc[r] : -__builtin_inff();
  __syncthreads();
  const int64_t ld = (int64_t)nblk * kc;
  for (int m = wave; m < M; m += kVThreads / kWave) {
    float v = cbuf[m * kBlockN + lane];
    int c = lane;
    wave_sort_vc(v, c, lane);
    if (lane < kc) {
      const int tok = b * kBlockN + c;
      const bool ok = tok < N;
      const int64_t at = (int64_t)m * ld + (int64_t)b * kc + lane;
      cand_score[at] = ok ? v : -__builtin_inff();
      cand_idx[at] = ok ? tok : -1;
    }
  }
}

template <int G, int LAYOUT, int SCALE>
void launch_variant(const uint16_t* x, const float* xs, int M, const uint8_t* packed, const uint16_t* S,
                    const uint16_t* ZS, int N, int K, int kc, int nblk, float* cs, int32_t* ci, hipStream_t s) {
  // what fits in the default 64 KiB of dynamic LDS: the block's scales, then up to 4 rows of x
  size_t lds = ((SCALE == kAcc ? (size_t)(K / G) * 16 : 0) + (size_t)16 * kBlockN) * sizeof(float);
  const size_t szb = (size_t)(K / G) * kBlockN * sizeof(uint32_t), xb = (size_t)M * K * sizeof(uint16_t);
  const bool szl = lds + szb <= 65536;
  if (szl) lds += szb;
  const bool xl = M <= kVXRows && lds + xb <= 65536;
  if (xl) lds += xb;
  const dim3 grid((unsigned)nblk), block(kVThreads);
  if (szl && xl)
    hipLaunchKernelGGL((coarse_variant_kernel<G, LAYOUT, SCALE, true, true>), grid, block, lds, s, x, xs, M, packed,
                       S, ZS, N, K, kc, nblk, cs, ci);
  else if (szl)
    hipLaunchKernelGGL((coarse_variant_kernel<G, LAYOUT, SCALE, false, true>), grid, block, lds, s, x, xs, M, packed,
                       S, ZS, N, K, kc, nblk, cs, ci);
  else if (xl)
    hipLaunchKernelGGL((coarse_variant_kernel<G, LAYOUT, SCALE, true, false>), grid, block, lds, s, x, xs, M, packed,
                       S, ZS, N, K, kc, nblk, cs, ci);
  else
    hipLaunchKernelGGL((coarse_variant_kernel<G, LAYOUT, SCALE, false, false>), grid, block, lds, s, x, xs, M,
                       packed, S, ZS, N, K, kc, nblk, cs, ci);
}

template <int G>
void dispatch_variant(int layout, int scaling, const uint16_t* x, const float* xs, int M, const uint8_t* packed,
                      const uint16_t* S, const uint16_t* ZS, int N, int K, int kc, int nblk, float* cs, int32_t* ci,
                      hipStream_t s) {
  if (layout == kQuarter && scaling == kAcc)
    launch_variant<G, kQuarter, kAcc>(x, xs, M, packed, S, ZS, N, K, kc, nblk, cs, ci, s);
  else if (layout == kQuarter)
    launch_variant<G, kQuarter, kTile>(x, xs, M, packed, S, ZS, N, K, kc, nblk, cs, ci, s);
  else if (scaling == kAcc)
    launch_variant<G, kContig, kAcc>(x, xs, M, packed, S, ZS, N, K, kc, nblk, cs, ci, s);
  else
    launch_variant<G, kContig, kTile>(x, xs, M, packed, S, ZS, N, K, kc, nblk, cs, ci, s);
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
  if (scaling == kAcc && !xs) return I2H_ERR_ARG;
  if (M < 1 || M > 16 || N < 1 || N > ((int64_t)1 << 30) || K <= 0 || K % (4 * group) != 0 || K > I2H_MAX_K)
    return I2H_ERR_SHAPE;
  if (kcand < 1 || kcand > I2H_MAX_KCAND) return I2H_ERR_LIMIT;
  if (!aligned(x, 16) || !aligned(packed, 16) || (xs && !aligned(xs, 16)) || !aligned(S, 2) || !aligned(ZS, 2) ||
      !aligned(cand_score, 4) || !aligned(cand_idx, 4))
    return I2H_ERR_ALIGN;
  const int nblk = (int)nblk_of(N);
  const hipStream_t s = (hipStream_t)stream;
  if (group == 128)
    dispatch_variant<128>(layout, scaling, x, xs, (int)M, packed, S, ZS, (int)N, (int)K, kcand, nblk, cand_score,
                          cand_idx, s);
  else
    dispatch_variant<64>(layout, scaling, x, xs, (int)M, packed, S, ZS, (int)N, (int)K, kcand, nblk, cand_score,
                         cand_idx, s);
  return check_launch();
}
