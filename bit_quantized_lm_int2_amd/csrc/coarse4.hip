// Coarse logits and block candidates of the int4 head.
//
// radiance_drafthead.py (the module docstring's bit-pattern dequant, bias fold and accumulator
// scaling, written for the 4-bit layout of _quantize_head_now): byte j of a packed row [K/2]
// holds the codes of k = j (bits 0-3) and K/2 + j (bits 4-7); the bf16 pattern 0x3F80 | v << 3
// reads as 1 + v/16, and with S = 16 sc, ZS = 16 sc + zp sc each group contributes
// S * sum_k x (1 + v/16) - xs * ZS. The page prints no 4-bit kernel; this is the 2-bit coarse
// kernel's structure with the half-split layout: a 128-byte span of a row feeds group gb of the
// first half and group KG/2 + gb of the second, each through 4 MFMAs (16x16x32 bf16) per m-tile.
//
// One 4-wave workgroup per 64-column block; lane (col = l & 15, h = l >> 4) streams bytes
// 32 h .. 32 h + 31 of each span of its row. When x is small (up to 32 KB: M <= 3 at K = 5120) it
// is staged in LDS once per workgroup and two spans of packed bytes and scales are in flight per
// lane; otherwise one span is, with the lane's x fragments when one m-tile covers the rows (x
// then comes from L2). The emit ranks the block's columns with a wave bitonic sort (any
// kcand <= 64).
#include "dequant.h"
#include "host_util.h"
#include "wave_sort.h"

namespace i2h {
namespace {

constexpr int kC4Threads = 256;
#ifndef I2H_C4_PF
#define I2H_C4_PF 1
#endif
constexpr int kC4Pf = I2H_C4_PF;  // spans of packed bytes (and x) in flight per lane
#ifndef I2H_C4_PF_XL
#define I2H_C4_PF_XL 2
#endif
constexpr int kC4PfXl = I2H_C4_PF_XL;  // spans in flight when x sits in LDS
#ifndef I2H_C4_PF_XL5120
#define I2H_C4_PF_XL5120 3
#endif
// waves per SIMD the launch bound asks for on the unrolled path: 6 (79 VGPRs, 22 KB of LDS: six
// workgroups per CU; 84 VGPRs and five without the bound, 1.1 us slower)
#ifndef I2H_C4_WPE_XL5120
#define I2H_C4_WPE_XL5120 6
#endif
constexpr int kC4PfXl5120 = I2H_C4_PF_XL5120;  // the same, with the span loop unrolled (K = 5120)
#ifndef I2H_C4_XL_BYTES
#define I2H_C4_XL_BYTES 32768
#endif
constexpr size_t kC4XlBytes = I2H_C4_XL_BYTES;  // largest x staged in LDS (M = 3 at K = 5120)

// Bytes [b0 b1 b2 b3] -> [b0 b2 b1 b3], so that one mask takes the nibbles of b0 and b1 (then b2
// and b3) into the two bf16 halves of a dword.
__device__ __forceinline__ uint32_t pair_bytes4(uint32_t d) { return __builtin_amdgcn_perm(d, d, 0x03010200u); }

// Eight weights of half HALF as bf16 1 + v/16 in natural k order; d0/d1 are byte-paired dwords.
template <int HALF>
__device__ __forceinline__ bf16x8 dequant4x8(uint32_t d0, uint32_t d1) {
  constexpr uint32_t kMask = 0x00780078u, kOne = 0x3F803F80u;
  u32x4 r;
  if constexpr (HALF == 0) {
    r[0] = ((d0 << 3) & kMask) | kOne;
    r[1] = ((d0 >> 5) & kMask) | kOne;
    r[2] = ((d1 << 3) & kMask) | kOne;
    r[3] = ((d1 >> 5) & kMask) | kOne;
  } else {
    r[0] = ((d0 >> 1) & kMask) | kOne;
    r[1] = ((d0 >> 9) & kMask) | kOne;
    r[2] = ((d1 >> 1) & kMask) | kOne;
    r[3] = ((d1 >> 9) & kMask) | kOne;
  }
  return __builtin_bit_cast(bf16x8, r);
}

// One half of one span: 4 MFMAs per m-tile, then the group's scale and zero. xa[s] (MT == 1) holds
// the x fragment of slice s already loaded; otherwise x is read here.
template <int MT, int HALF>
__device__ __forceinline__ void half4(f32x4 (&acc)[MT], const uint32_t (&dw)[8], const u32x4* xa,
                                      const uint16_t* xq, int M, int K, int col, float sv, float zv,
                                      const float* xsg, int hrow) {
  f32x4 p[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) p[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const bf16x8 b = dequant4x8<HALF>(dw[2 * s], dw[2 * s + 1]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      u32x4 a;
      if constexpr (MT == 1) {
        a = xa[s];
      } else {
        const int m = mt * 16 + col;
        a = m < M ? ld16(xq + (int64_t)m * K + 8 * s) : u32x4{0u, 0u, 0u, 0u};
      }
      p[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, p[mt], 0, 0, 0);
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const f32x4 xv = *reinterpret_cast<const f32x4*>(xsg + mt * 16 + hrow);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float a = fmaf(sv, p[mt][r], acc[mt][r]);
      acc[mt][r] = fmaf(-xv[r], zv, a);
    }
  }
}

// XL: x (at most kC4XlBytes) is staged in LDS once per workgroup and the fragments are read from
// there, so a ring slot holds only the packed bytes and the scales and PF slots fit in registers.
// NSC > 0: the number of 128-byte spans per half row (K / 256), a compile-time constant, so the
// span loop is unrolled completely and every wait for a span in flight is exact (a run-time loop
// with its loads under a test makes the compiler wait for every load at each iteration).
template <int MT, bool XL, int PF, int NSC = 0>
__global__ __launch_bounds__(kC4Threads, NSC > 0 ? I2H_C4_WPE_XL5120 : 1) void coarse4_kernel(const uint16_t* __restrict__ x, const float* __restrict__ xs,
                                                             int M, const uint8_t* __restrict__ packed,
                                                             const uint16_t* __restrict__ S,
                                                             const uint16_t* __restrict__ ZS, int N, int K, int kc,
                                                             int nblk, float* __restrict__ cand_score,
                                                             int32_t* __restrict__ cand_idx, uint16_t* __restrict__ y) {
  constexpr int MR = 16 * MT;
  // with the span loop unrolled (XL): the block's S | ZS << 16 rows, [64][KG | 1], each wave's 16
  // rows staged by that wave, so the ring holds only packed bytes; there at most 3 rows are real
  // (x in LDS), so the group sums and the emit's logits keep 4 rows, not 16
  constexpr bool kSzL = XL && NSC > 0;
  constexpr int XR = kSzL ? 4 : MR;  // rows per group of xsT, rows of cbuf
  extern __shared__ float smem[];
  const int H = K >> 1, NS = H / kGroup, KG = K / kGroup;
  float* xsT = smem;             // [KG][XR]: xs transposed, zero past row M
  float* cbuf = smem + KG * XR;  // [XR][64]: the block's logits for the emit
  uint16_t* xl = reinterpret_cast<uint16_t*>(cbuf + XR * kBlockN);  // [M][K] when XL
  const int KGP = KG | 1;
  uint32_t* szl = reinterpret_cast<uint32_t*>(xl + (XL ? M * K : 0));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, h = lane >> 4;
  const int b = blockIdx.x;
  const int n = b * kBlockN + wave * 16 + col;
  const bool nvalid = n < N;
  const int nr = nvalid ? n : 0;

  for (int i = tid; i < KG * XR; i += kC4Threads) {
    const int g = i / XR, m = i - g * XR;
    xsT[i] = m < M ? xs[(int64_t)m * KG + g] : 0.f;
  }
  if constexpr (kSzL) {  // this wave's 16 rows (rows past N: zeros, never emitted)
    const int r0 = b * kBlockN + wave * 16;
    for (int e = lane; e < 16 * KG; e += kWave) {
      const int r = e / KG, g = e - r * KG;
      const bool ok = r0 + r < N;
      const uint32_t sb = ok ? S[(int64_t)(r0 + r) * KG + g] : 0u, zb = ok ? ZS[(int64_t)(r0 + r) * KG + g] : 0u;
      szl[(wave * 16 + r) * KGP + g] = sb | (zb << 16);
    }
  }
  if constexpr (XL)
    for (int u = tid; u < M * K / 8; u += kC4Threads)
      *reinterpret_cast<u32x4*>(xl + 8 * u) = ld16(x + 8 * u);
  __syncthreads();

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint8_t* prow = packed + (int64_t)nr * H + 32 * h;
  const uint16_t* srow = S + (int64_t)nr * KG;
  const uint16_t* zrow = ZS + (int64_t)nr * KG;
  const uint16_t* xh = x + 32 * h;
  // a ring of kC4Pf spans in flight: the packed bytes and the two groups' S / ZS (rows past N
  // read row 0, never stored) and, for one m-tile, the lane's x fragments of both halves (rows
  // past M read row 0, unused)
  constexpr int kXF = MT == 1 && !XL ? 8 : 1;
  const int xrow = MT == 1 ? (col < M ? col : 0) : 0;
  struct Slot {
    u32x4 p0, p1;
    u32x4 xa[kXF];
    uint32_t s0, z0, s1, z1;  // the two groups' S and ZS bits
  };
  auto fetch = [&](Slot& sl, int gb) {
    sl.p0 = ld16(prow + gb * kGroup);
    sl.p1 = ld16(prow + gb * kGroup + 16);
    if constexpr (!kSzL) {
      sl.s0 = srow[gb];
      sl.z0 = zrow[gb];
      sl.s1 = srow[KG / 2 + gb];
      sl.z1 = zrow[KG / 2 + gb];
    }
    if constexpr (MT == 1 && !XL) {
      const uint16_t* xq = xh + (int64_t)xrow * K + gb * kGroup;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sl.xa[s] = ld16(xq + 8 * s);
        sl.xa[4 + s] = ld16(xq + H + 8 * s);
      }
    }
  };
  auto body = [&](const Slot& sl, int gb) {
    uint32_t dw[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dw[i] = pair_bytes4(sl.p0[i]);
      dw[4 + i] = pair_bytes4(sl.p1[i]);
    }
    const uint16_t* xg = xh + gb * kGroup;
    const int g0 = gb, g1 = KG / 2 + gb;
    const u32x4* xa = sl.xa;
    u32x4 xv[8];
    if constexpr (XL) {
      // the lane's x fragments of this span, from LDS
      const uint16_t* xq = xl + xrow * K + gb * kGroup + 32 * h;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        xv[s] = *reinterpret_cast<const u32x4*>(xq + 8 * s);
        xv[4 + s] = *reinterpret_cast<const u32x4*>(xq + H + 8 * s);
      }
      xa = xv;
    }
    uint32_t s0, z0, s1, z1;
    if constexpr (kSzL) {
      const uint32_t w0 = szl[(wave * 16 + col) * KGP + g0], w1 = szl[(wave * 16 + col) * KGP + g1];
      s0 = w0 & 0xffffu;
      z0 = w0 >> 16;
      s1 = w1 & 0xffffu;
      z1 = w1 >> 16;
    } else {
      s0 = sl.s0;
      z0 = sl.z0;
      s1 = sl.s1;
      z1 = sl.z1;
    }
    // (with 4 rows per group every lane reads the same four: only those of the real rows count)
    half4<MT, 0>(acc, dw, xa, xg, M, K, col, bf16_lo(s0), bf16_lo(z0), xsT + g0 * XR, XR == MR ? 4 * h : 0);
    half4<MT, 1>(acc, dw, xa + (MT == 1 ? 4 : 0), xg + H, M, K, col, bf16_lo(s1), bf16_lo(z1), xsT + g1 * XR,
                 XR == MR ? 4 * h : 0);
  };
  Slot ring[PF];
#pragma unroll
  for (int q = 0; q < PF; ++q) fetch(ring[q], q < NS ? q : NS - 1);
  if constexpr (NSC > 0) {
#pragma unroll
    for (int gb = 0; gb < NSC; ++gb) {
      body(ring[gb % PF], gb);
      if (gb + PF < NSC) fetch(ring[gb % PF], gb + PF);
    }
  } else {
    for (int gb0 = 0; gb0 < NS; gb0 += PF) {
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        const int gb = gb0 + q;
        if (gb < NS) {
          body(ring[q], gb);
          const int nx = gb + PF;
          fetch(ring[q], nx < NS ? nx : NS - 1);
        }
      }
    }
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
      if (mt * 16 + 4 * h + r < XR)
        cbuf[(mt * 16 + 4 * h + r) * kBlockN + wave * 16 + col] = nvalid ? acc[mt][r] : -__builtin_inff();
  __syncthreads();

  const int64_t ld = (int64_t)nblk * kc;
  for (int m = wave; m < M; m += kC4Threads / kWave) {
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

template <int MT>
void launch4(const uint16_t* x, const float* xs, int M, const uint8_t* packed, const uint16_t* S, const uint16_t* ZS,
             int N, int K, int kc, int nblk, float* cs, int32_t* ci, uint16_t* y, hipStream_t s) {
  const size_t lds = ((size_t)(K / kGroup) * 16 * MT + (size_t)16 * MT * kBlockN) * sizeof(float);
  const size_t xbytes = (size_t)M * K * 2;
  if constexpr (MT == 1) {
    if (xbytes <= kC4XlBytes) {
      if (K == 5120)  // the head's K: the span loop unrolled, S / ZS rows in LDS, 4-row group sums and logits
        hipLaunchKernelGGL((coarse4_kernel<MT, true, kC4PfXl5120, 20>), dim3((unsigned)nblk), dim3(kC4Threads),
                           ((size_t)(K / kGroup) * 4 + (size_t)4 * kBlockN) * sizeof(float) + xbytes +
                               (size_t)64 * ((K / kGroup) | 1) * 4,
                           s, x, xs, M, packed, S, ZS, N, K, kc, nblk, cs, ci, y);
      else
        hipLaunchKernelGGL((coarse4_kernel<MT, true, kC4PfXl>), dim3((unsigned)nblk), dim3(kC4Threads), lds + xbytes,
                           s, x, xs, M, packed, S, ZS, N, K, kc, nblk, cs, ci, y);
      return;
    }
  }
  hipLaunchKernelGGL((coarse4_kernel<MT, false, kC4Pf>), dim3((unsigned)nblk), dim3(kC4Threads), lds, s, x, xs, M,
                     packed, S, ZS, N, K, kc, nblk, cs, ci, y);
}

}  // namespace
}  // namespace i2h

extern "C" int i2h_coarse4_topk(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed,
                                const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int kcand,
                                float* cand_score, int32_t* cand_idx, uint16_t* y, void* stream) {
  using namespace i2h;
  if (!x || !xs || !packed || !S || !ZS || !cand_score || !cand_idx) return I2H_ERR_ARG;
  if (M < 1 || N < 1 || N > ((int64_t)1 << 31) - 64 || K <= 0 || K % (2 * I2H_GROUP) != 0 || K > I2H_MAX_K)
    return I2H_ERR_SHAPE;
  if (kcand < 1 || kcand > I2H_MAX_KCAND) return I2H_ERR_LIMIT;
  if (!aligned(x, 16) || !aligned(xs, 16) || !aligned(packed, 16) || !aligned(S, 2) || !aligned(ZS, 2) ||
      !aligned(cand_score, 4) || !aligned(cand_idx, 4) || (y && !aligned(y, 2)))
    return I2H_ERR_ALIGN;
  const int64_t nblk = nblk_of(N);
  const int64_t KG = K / I2H_GROUP, ld = nblk * kcand;
  const hipStream_t s = (hipStream_t)stream;
  // rows in chunks of at most 64 (one launch each)
  for (int64_t m0 = 0; m0 < M; m0 += 64) {
    const int mc = (int)(M - m0 < 64 ? M - m0 : 64);
    const uint16_t* xm = x + m0 * K;
    const float* xsm = xs + m0 * KG;
    float* csm = cand_score + m0 * ld;
    int32_t* cim = cand_idx + m0 * ld;
    uint16_t* ym = y ? y + m0 * N : nullptr;
    if (mc <= 16)
      launch4<1>(xm, xsm, mc, packed, S, ZS, (int)N, (int)K, kcand, (int)nblk, csm, cim, ym, s);
    else if (mc <= 32)
      launch4<2>(xm, xsm, mc, packed, S, ZS, (int)N, (int)K, kcand, (int)nblk, csm, cim, ym, s);
    else
      launch4<4>(xm, xsm, mc, packed, S, ZS, (int)N, (int)K, kcand, (int)nblk, csm, cim, ym, s);
    const int st = check_launch();
    if (st != I2H_OK) return st;
  }
  return I2H_OK;
}
