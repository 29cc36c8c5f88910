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
// packed bytes of its row per 128-byte span (two 16-byte loads; the M <= 4 kernel takes bytes
// 16h and 64 + 16h, whole 64-byte sectors per load); the 8 bytes of slice s serve all four
// quarters t, i.e. four different quantisation groups, each with its own MFMA accumulator that
// is scaled and folded into the result once the group is complete. A byte permute puts bytes (0,2,1,3) of each
// dword in place so that the bit-pattern dequant yields bf16 pairs in natural k order, which
// lets the x fragment be one contiguous 16-byte load.
#include <type_traits>

#include "ablation.h"
#include "dequant.h"
#include "host_util.h"

namespace i2h {
namespace {

constexpr int kCoarseThreads = 256;  // 4 waves x 16 columns = one 64-column block

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
    int32_t* __restrict__ cand_idx, uint16_t* __restrict__ y, float* __restrict__ bmax) {
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
      if (lane == 0 && bmax != nullptr) bmax[(int64_t)m * nblk + b] = ok ? v : -__builtin_inff();
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Small-M band (M <= 4): one m-tile, HBM-bound. Differences from coarse_kernel:
//   * the block's S and ZS rows (contiguous in memory) and, when it fits, x itself are staged
//     in LDS once per workgroup, so the K loop issues no small scattered loads;
//   * the packed stream is prefetched several 128-byte spans ahead;
//   * quarters 0-2 are dequantised with a mask alone (dequant.h), the high byte of each half
//     brought down by one shift shared by the four quarters: 12 VALU ops per 16 weights;
//   * only the accumulator rows that can hold a real row are scaled.
// In the head it takes one or two rows (one row: at most 80 VGPRs and 21 KB of LDS, six
// workgroups per CU, two spans in flight per lane; two rows: 32 KB of LDS, five workgroups per
// CU; from three rows x in LDS costs occupancy and the tile kernel is faster).
// ---------------------------------------------------------------------------------------------

#ifndef I2H_COARSE_PF
#define I2H_COARSE_PF 2
#endif
constexpr int kPf = I2H_COARSE_PF;
// Packed bytes per lane and span: 1 = aligned 64-byte sectors (lane h takes bytes 16h and
// 64 + 16h, so each load instruction reads whole sectors), 0 = 32 consecutive bytes at 32h.
#ifndef I2H_SMALL_SECTOR
#define I2H_SMALL_SECTOR 1
#endif
constexpr int kLaneOff = I2H_SMALL_SECTOR ? 16 : 32;  // byte offset of lane h's first load
constexpr int kHalfOff = I2H_SMALL_SECTOR ? 64 : 16;  // byte offset of its second load
#ifndef I2H_COARSE_SLICE_FENCE
#define I2H_COARSE_SLICE_FENCE 1
#endif  // 128-byte spans of the packed stream in flight per lane

// Rows of the transposed group-sum table per group: the rows an accumulator lane can hold, 4 when
// at most two rows are real (every lane then reads the same four, and only rows 0 and 1 are used).
__host__ __device__ constexpr int small_xs_rows(int maxr) { return maxr <= 2 ? 4 : 16; }

// LDS footprint of coarse_small_kernel in bytes: S|ZS for the block's rows, xs transposed (G: the
// quantisation group), the block's 64-bit ranking keys for its maxr rows, and x itself when xlds.
__host__ __device__ constexpr size_t small_lds_bytes(int K, int maxr, bool xlds, int G = kGroup) {
  return (size_t)64 * (K / G) * 4 + (size_t)(K / G) * small_xs_rows(maxr) * 4 + (size_t)maxr * kBlockN * 8 +
         (xlds ? (size_t)maxr * K * 2 : 0);
}

// Ranking key of a coarse logit in its block: higher value first, then lower column.
__device__ __forceinline__ uint64_t block_key(float v, int col_in_block) {
  return ((uint64_t)ordered_key(v) << 32) | (uint64_t)(63 - col_in_block);
}

// Block top-kc of M rows whose 64 keys sit in ck[m][64] (unique keys): a key's rank is the number
// of its row's keys that beat it, and a rank below kc is its output slot. Every wave takes 16
// keys of each row, four lanes per key (lane = 4 i + q compares key 16 wave + i with keys
// 16 q .. 16 q + 15), and the four partial counts are summed across the quad.
__device__ __forceinline__ void emit_ranked(const uint64_t* ck, int M, int b, int N, int kc, int64_t ld,
                                            float* __restrict__ cand_score, int32_t* __restrict__ cand_idx,
                                            float* __restrict__ bmax) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane & 3, i = wave * 16 + (lane >> 2);
  for (int m = 0; m < M; ++m) {
    const uint64_t* row = ck + m * kBlockN;
    const uint64_t mine = row[i];
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const uint64_t a = row[16 * q + j], c = row[16 * q + j + 1];
      rank += (a > mine) + (c > mine);
    }
    rank += __shfl_xor(rank, 1);
    rank += __shfl_xor(rank, 2);
    if (q == 0 && rank < kc) {
      const int tok = b * kBlockN + 63 - (int)(mine & 63u);
      const bool ok = tok < N;
      const int64_t at = (int64_t)m * ld + (int64_t)b * kc + rank;
      cand_score[at] = ok ? from_ordered_key((uint32_t)(mine >> 32)) : -__builtin_inff();
      cand_idx[at] = ok ? tok : -1;
      if (rank == 0 && bmax != nullptr)
        bmax[(int64_t)m * (ld / kc) + b] = ok ? from_ordered_key((uint32_t)(mine >> 32)) : -__builtin_inff();
    }
  }
}

// NGC > 0: the number of 128-byte spans per packed row (K / 512) is a compile-time constant and
// the span loop is unrolled completely, so every wait for a prefetched span is exact; NGC = 0
// runs the loop at run time (the compiler then waits for all loads at each loop header).
// VAR (ablation.h): the design, or one alternative (one row, x in LDS, NGC > 0 only): group 64
// splits each quarter's partial sum in two at k = 64 (the lane's second 16-byte load starts
// there); contiguous-4 takes four 8-byte runs per span, 32 consecutive k of each of the span's
// four groups, with x in LDS in natural order; the weight tile feeds the dequantised weights to
// the matrix cores and needs no group sums.
template <int MAXR, bool XLDS, int NGC, int VAR = kVarDesign>
__global__ __launch_bounds__(kCoarseThreads, MAXR == 2 ? 4 : (MAXR == 1 && VAR == kVarDesign ? 6 : 1)) void coarse_small_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ xs, int M,
    const uint8_t* __restrict__ packed, const uint16_t* __restrict__ S,
    const uint16_t* __restrict__ ZS, int N, int K, int kc, int nblk, float* __restrict__ cand_score,
    int32_t* __restrict__ cand_idx, uint16_t* __restrict__ y, float* __restrict__ bmax, int32_t* __restrict__ zc) {
  constexpr int RR = MAXR < 4 ? MAXR : 4;  // accumulator rows per lane that can be real
  static_assert(VAR == kVarDesign || (MAXR == 1 && XLDS && NGC > 0), "alternatives: one row, x in LDS");
  constexpr int GV = VAR == kVarG64 ? 64 : kGroup;  // quantisation group along k
  constexpr bool kSums = VAR != kVarWTile;           // the accumulator form needs the group sums
  // zc (may be null): one int per row, set to 0 (the arrival counters of the head's tail)
  if (zc != nullptr && blockIdx.x == 0 && (int)threadIdx.x < M) zc[threadIdx.x] = 0;
  extern __shared__ __align__(16) uint32_t lds[];
  if constexpr (NGC > 0) K = NGC * 512;
  const int Q = K >> 2, NG = NGC > 0 ? NGC : Q / kGroup, KG = K / GV;
  uint32_t* sz = lds;                                        // [64][KG]: S | ZS << 16
  constexpr int XR = small_xs_rows(MAXR);                   // rows of xsT per group
  float* xsT = reinterpret_cast<float*>(sz + 64 * KG);       // [KG][XR]
  uint64_t* ck = reinterpret_cast<uint64_t*>(xsT + KG * XR);  // [MAXR][64] ranking keys
  uint16_t* xl = reinterpret_cast<uint16_t*>(ck + MAXR * kBlockN);  // [MAXR][K] when XLDS
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, h = lane >> 4;
  const int b = blockIdx.x, n0 = b * kBlockN;
  const int n = n0 + wave * 16 + col;
  const bool nvalid = n < N;

  // Loads complete in issue order as far as the wait counter is concerned, so they are issued in
  // the order their data is needed: x (resident in L2) first, then this wave's S/ZS rows, then
  // the first spans of the packed stream.
  constexpr bool kXReg = XLDS && NGC > 0;  // x staged through registers, group sums reduced there
  constexpr int kXU = kXReg ? (MAXR * NGC * 64 + kCoarseThreads - 1) / kCoarseThreads : 1;
  const int xunits = XLDS ? M * (K / 8) : 0;  // 16-byte units of x
  u32x4 xr[kXU];
  if constexpr (kXReg) {
#pragma unroll
    for (int i = 0; i < kXU; ++i) {
      const int u = tid + i * kCoarseThreads;
      xr[i] = u < xunits ? ld16(x + 8 * u) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // 16-byte S units per lane: 16 rows * KG / 8 / 64 (KG <= 128)
  constexpr int kSzW = NGC > 0 ? (2 * NGC * 4 * (kGroup / GV) + 63) / 64 : 4;
  const int rows_valid = N - n0 < kBlockN ? N - n0 : kBlockN;
  const int tot = rows_valid * KG;                   // valid elements of the block's S
  const int wbase = wave * 16 * KG;                  // this wave's rows start here
  const uint16_t* Sb = S + (int64_t)n0 * KG;
  const uint16_t* Zb = ZS + (int64_t)n0 * KG;
  u32x4 sv[kSzW], zv[kSzW];
#pragma unroll
  for (int i = 0; i < kSzW; ++i) {
    const int e0 = wbase + (lane + i * kWave) * 8;
    sv[i] = u32x4{0u, 0u, 0u, 0u};
    zv[i] = u32x4{0u, 0u, 0u, 0u};
    if ((lane + i * kWave) * 8 < 16 * KG) {
      if (e0 + 8 <= tot) {
        sv[i] = ld16(Sb + e0);
        zv[i] = ld16(Zb + e0);
      } else if (e0 < tot) {
        for (int j = 0; j < 8; ++j)
          if (e0 + j < tot) {
            sv[i][j >> 1] |= (uint32_t)Sb[e0 + j] << (16 * (j & 1));
            zv[i][j >> 1] |= (uint32_t)Zb[e0 + j] << (16 * (j & 1));
          }
      }
    }
  }
  // contiguous-4: lane h reads 8 bytes of each of the span's four groups (at 32 i + 8 h)
  const uint8_t* prow = packed + (int64_t)(nvalid ? n : 0) * Q + (VAR == kVarC4 ? 8 : kLaneOff) * h;
  u32x4 ring[kPf][2];
  auto span_load = [&](int g, u32x4 (&r)[2]) {
    if constexpr (VAR == kVarC4) {
      typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
      u32x2 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = *reinterpret_cast<const u32x2*>(prow + g * kGroup + 32 * i);
      r[0] = u32x4{v[0][0], v[0][1], v[1][0], v[1][1]};
      r[1] = u32x4{v[2][0], v[2][1], v[3][0], v[3][1]};
    } else {
      r[0] = ld16(prow + g * kGroup);
      r[1] = ld16(prow + g * kGroup + kHalfOff);
    }
  };
#pragma unroll
  for (int p = 0; p < kPf; ++p) span_load(p < NG ? p : NG - 1, ring[p]);

  // x rows in LDS, laid out by span: xl[m][gb][t][j] holds x[m][t Q + 128 gb + j], so the four
  // quarters of span gb sit 128 apart and every fragment offset is an immediate; each group of
  // four k is stored as (0, 2, 1, 3), the order in which the mask dequant of a raw packed dword
  // yields its weights, so the packed bytes need no permute
  auto put_x = [&](int u, const u32x4& v) {
    if constexpr (VAR == kVarC4) {  // natural order, the layout of x itself
      *reinterpret_cast<u32x4*>(xl + 8 * u) = v;
      return;
    }
    const u32x4 o = x_pair_order(v);
    const int m = (8 * u) / K, k = 8 * u - m * K;
    const int t = k / Q, r = k - t * Q;
    *reinterpret_cast<u32x4*>(xl + m * K + (r / kGroup) * 512 + t * kGroup + (r % kGroup)) = o;
  };
  if constexpr (kXReg) {
#pragma unroll
    for (int i = 0; i < kXU; ++i) {
      const int u = tid + i * kCoarseThreads;
      if (u < xunits) put_x(u, xr[i]);
      if (kSums && xs == nullptr) {
        // the GV / 8 units of a group sit in consecutive lanes
        float sm = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) sm += bf16_lo(xr[i][e]) + bf16_hi(xr[i][e]);
#pragma unroll
        for (int o = 1; o < GV / 8; o <<= 1) sm += __shfl_xor(sm, o);
        if ((tid & (GV / 8 - 1)) == 0 && u < xunits) {
          const int m = (8 * u) / K, g = (8 * u - m * K) / GV;
          xsT[g * XR + m] = sm;
        }
      }
    }
    if (kSums && xs == nullptr)
      for (int i = tid; i < KG * XR; i += kCoarseThreads)
        if (i % XR >= M) xsT[i] = 0.f;
  } else if constexpr (XLDS) {
    for (int u = tid; u < xunits; u += kCoarseThreads) put_x(u, ld16(x + 8 * u));
  }
  if (kSums && xs != nullptr) {
    for (int i = tid; i < KG * XR; i += kCoarseThreads) {
      const int g = i / XR, m = i % XR;
      xsT[i] = m < M ? xs[(int64_t)m * KG + g] : 0.f;
    }
  }
  __syncthreads();
  if (!kXReg && kSums && xs == nullptr) {
    // group sums from the LDS copy of x (only launched so with x in LDS): one thread per group
    for (int i = tid; i < KG * XR; i += kCoarseThreads) {
      const int g = i / XR, m = i % XR;
      float sm = 0.f;
      if (m < M) {
        const int t = g / NG, gb = g - t * NG;
        const uint16_t* xg = xl + m * K + gb * 512 + t * kGroup;
#pragma unroll
        for (int j = 0; j < kGroup; j += 8) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(xg + j);
#pragma unroll
          for (int e = 0; e < 4; ++e) sm += bf16_lo(v[e]) + bf16_hi(v[e]);
        }
      }
      xsT[i] = sm;
    }
    __syncthreads();
  }
  // this wave's S/ZS rows, interleaved S | ZS << 16; only this wave reads them, so no barrier
#pragma unroll
  for (int i = 0; i < kSzW; ++i) {
    if ((lane + i * kWave) * 8 < 16 * KG) {
      const int e0 = wbase + (lane + i * kWave) * 8;
      u32x4 lo, hi;
      lo[0] = __builtin_amdgcn_perm(zv[i][0], sv[i][0], 0x05040100u);
      lo[1] = __builtin_amdgcn_perm(zv[i][0], sv[i][0], 0x07060302u);
      lo[2] = __builtin_amdgcn_perm(zv[i][1], sv[i][1], 0x05040100u);
      lo[3] = __builtin_amdgcn_perm(zv[i][1], sv[i][1], 0x07060302u);
      hi[0] = __builtin_amdgcn_perm(zv[i][2], sv[i][2], 0x05040100u);
      hi[1] = __builtin_amdgcn_perm(zv[i][2], sv[i][2], 0x07060302u);
      hi[2] = __builtin_amdgcn_perm(zv[i][3], sv[i][3], 0x05040100u);
      hi[3] = __builtin_amdgcn_perm(zv[i][3], sv[i][3], 0x07060302u);
      *reinterpret_cast<u32x4*>(sz + e0) = lo;
      *reinterpret_cast<u32x4*>(sz + e0 + 4) = hi;
    }
  }

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const uint32_t* szr = sz + (wave * 16 + col) * KG;
  // A-operand rows past M repeat row M-1: their accumulator rows are computed and never used
  const int arow = col < M ? col : M - 1;
  const DqConst dqc = dq_const();

  auto body = [&](int gb, const u32x4& c0, const u32x4& c1) {
    if constexpr (VAR == kVarC4) {
      // group i of the span (4 gb + i): run i is dwords 2 i, 2 i + 1 of (c0, c1); slice s reads
      // its bytes 2 s, 2 s + 1 (k = 128 (4 gb + i) + 32 h + 8 s .. + 7)
      const uint32_t rd[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
      f32x4 p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* xa = xl + arow * K + gb * 512 + 32 * h;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16x8 bw = dequant8_c4((rd[2 * i + (s >> 1)] >> (16 * (s & 1))) & 0xffffu);
          const u32x4 a = *reinterpret_cast<const u32x4*>(xa + 128 * i + 8 * s);
          p[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), bw, p[i], 0, 0, 0);
        }
#if I2H_COARSE_SLICE_FENCE
        __builtin_amdgcn_sched_barrier(0);
#endif
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {  // codes read at D = 4: the scale and zero as they are
        const int gi = 4 * gb + i;
        const uint32_t w = szr[gi];
        const f32x4 xv = *reinterpret_cast<const f32x4*>(xsT + gi * XR + (XR == 16 ? 4 * h : 0));
#pragma unroll
        for (int r = 0; r < RR; ++r)
          acc[r] = fmaf(-xv[r], __uint_as_float(w & 0xffff0000u), fmaf(__uint_as_float(w << 16), p[i][r], acc[r]));
      }
      return;
    }
    uint32_t dw[8], hw[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      dw[i] = XLDS ? c0[i] : pair_bytes(c0[i]);
      dw[4 + i] = XLDS ? c1[i] : pair_bytes(c1[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) hw[i] = dw[i] >> 8;
    // group 64: each quarter's group ends at k = 64 (after slice 1) and at k = 128 (after slice 3),
    // and each is scaled and folded into the result where it ends
    constexpr int HV = VAR == kVarG64 ? 2 : 1;
    f32x4 p[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) p[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto fold = [&](int hf) {  // scale and zero of the groups that end here
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int gi = HV * (t * NG + gb) + hf;
        const uint32_t w = szr[gi];
        const float sv = __uint_as_float(w << 16);
        const float zv = __uint_as_float(w & 0xffff0000u);
        const float s2 = kBiasF[t] * sv;
        const float z2 = fmaf(kBiasF[t] - 1.f, sv, zv);
        const f32x4 xv = *reinterpret_cast<const f32x4*>(xsT + gi * XR + (XR == 16 ? 4 * h : 0));
#pragma unroll
        for (int r = 0; r < RR; ++r) {
          const float a = fmaf(s2, p[t][r], acc[r]);
          acc[r] = fmaf(-xv[r], z2, a);
        }
        p[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };
    // weight tile: each quarter's f S and (f - 1) S + ZS, which the dequantised weights take
    float s1[4], z1[4];
    if constexpr (VAR == kVarWTile) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t w = szr[t * NG + gb];
        s1[t] = kBiasF[t] * __uint_as_float(w << 16);
        z1[t] = fmaf(kBiasF[t] - 1.f, __uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
      }
    }
    const uint16_t* xa = XLDS ? xl + arow * K + gb * 512 + kLaneOff * h : x + (int64_t)arow * K + gb * kGroup + kLaneOff * h;
    // k offset of slice s within lane h's part of the group
    auto soff = [](int s_) { return I2H_SMALL_SECTOR ? 8 * (s_ & 1) + 64 * (s_ >> 1) : 8 * s_; };
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bf16x8 bw;
        const uint32_t d0 = dw[2 * s], d1 = dw[2 * s + 1], h0 = hw[2 * s], h1 = hw[2 * s + 1];
        if (t == 0) bw = dequant8_mask<0>(d0, d1, h0, h1, dqc);
        else if (t == 1) bw = dequant8_mask<1>(d0, d1, h0, h1, dqc);
        else if (t == 2) bw = dequant8_mask<2>(d0, d1, h0, h1, dqc);
        else bw = dequant8_mask<3>(d0, d1, h0, h1, dqc);
        u32x4 a;
        if constexpr (XLDS) a = *reinterpret_cast<const u32x4*>(xa + t * kGroup + soff(s));
        else a = ld16(xa + t * Q + soff(s));
        if constexpr (VAR == kVarWTile)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), tile8_fold(bw, s1[t], z1[t]),
                                                        acc, 0, 0, 0);
        else
          p[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), bw, p[t], 0, 0, 0);
      }
#if I2H_COARSE_SLICE_FENCE
      // keep the next slice's x fragments from being hoisted: 4 live fragments instead of 16
      __builtin_amdgcn_sched_barrier(0);
#endif
      if (HV == 2 && s == 1) {
        fold(0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (VAR != kVarWTile) fold(HV - 1);
  };

  // ring of I2H_COARSE_PF spans in flight: slot p is consumed in place, then refilled with the
  // span PF ahead (refilling before the body would make the compiler copy the slot out first,
  // which waits for every load in flight)
  if constexpr (NGC > 0) {
#pragma unroll
    for (int gb = 0; gb < NGC; ++gb) {
      body(gb, ring[gb % kPf][0], ring[gb % kPf][1]);
      if (gb + kPf < NGC) span_load(gb + kPf, ring[gb % kPf]);
    }
  } else {
    for (int gb0 = 0; gb0 < NG; gb0 += kPf) {
#pragma unroll
      for (int p = 0; p < kPf; ++p) {
        const int gb = gb0 + p;
        if (gb < NG) {
          body(gb, ring[p][0], ring[p][1]);
          span_load(gb + kPf < NG ? gb + kPf : NG - 1, ring[p]);
        }
      }
    }
  }

  // acc[r] is c[m = 4 h + r][n]
  if (y != nullptr && nvalid) {
#pragma unroll
    for (int r = 0; r < RR; ++r) {
      const int m = 4 * h + r;
      if (m < M) y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < RR; ++r)  // rows past MAXR (lanes h > 0) hold no row of x
    if (4 * h + r < MAXR)
      ck[(4 * h + r) * kBlockN + wave * 16 + col] = block_key(nvalid ? acc[r] : -__builtin_inff(), wave * 16 + col);
  __syncthreads();
  emit_ranked(ck, M, b, N, kc, (int64_t)nblk * kc, cand_score, cand_idx, bmax);
}

// One wave per row of x: lane l sums elements 8l..8l+7 of each 512-element chunk (one 16-byte
// load; all of a row's loads are issued before any sum), then the 16 lanes of each group of 128
// reduce by butterfly. Rows are independent, so any M takes ceil(M / 4) workgroups.
// zc (may be null): one int per row, set to 0 here (the arrival counters of the head's tail).
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                   float* __restrict__ xs, int32_t* __restrict__ zc) {
  constexpr int kBatch = 10;  // 512-element chunks in flight per lane (K = 5120 in one batch)
  const int KG = K / kGroup;
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  if (zc != nullptr && lane == 0) zc[m] = 0;
  const uint16_t* xr = x + (int64_t)m * K;
  const int nch = (K + 511) / 512;
  for (int c0 = 0; c0 < nch; c0 += kBatch) {
    u32x4 v[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int e = (c0 + j) * 512 + 8 * lane;
      v[j] = c0 + j < nch && e < K ? ld16(xr + e) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      float sm = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) sm += bf16_lo(v[j][e]) + bf16_hi(v[j][e]);
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) sm += __shfl_xor(sm, o);
      const int g = (c0 + j) * 4 + (lane >> 4);
      if ((lane & 15) == 0 && c0 + j < nch && g < KG) xs[(int64_t)m * KG + g] = sm;
    }
  }
}

template <int MT>
int launch_coarse(const uint16_t* x, const float* xs, int M, const uint8_t* packed, const uint16_t* S,
                  const uint16_t* ZS, int N, int K, int kc, float* cs, int32_t* ci, uint16_t* y,
                  float* bmax, hipStream_t s) {
  const int nblk = (int)nblk_of(N);
  const size_t lds = (size_t)(K / kGroup) * 16 * MT * 4 + (size_t)16 * MT * kBlockN * 4;
  hipLaunchKernelGGL(coarse_kernel<MT>, dim3(nblk), dim3(kCoarseThreads), lds, s, x, xs, M, packed, S,
                     ZS, N, K, kc, nblk, cs, ci, y, bmax);
  return check_launch();
}

template <int MAXR, bool XLDS>
int launch_small(const uint16_t* x, const float* xs, int M, const uint8_t* packed, const uint16_t* S,
                 const uint16_t* ZS, int N, int K, int kc, float* cs, int32_t* ci, uint16_t* y, float* bmax,
                 int32_t* zc, hipStream_t s) {
  const int nblk = (int)nblk_of(N);
  const size_t lds = small_lds_bytes(K, MAXR, XLDS);
  // the span loop unrolled for the K of the head's family, a run-time loop otherwise
  auto go = [&](auto ngc) {
    hipLaunchKernelGGL((coarse_small_kernel<MAXR, XLDS, decltype(ngc)::value>), dim3(nblk), dim3(kCoarseThreads), lds,
                       s, x, xs, M, packed, S, ZS, N, K, kc, nblk, cs, ci, y, bmax, zc);
  };
  switch (K) {
    case 5120: go(std::integral_constant<int, 10>{}); break;
    case 4096: go(std::integral_constant<int, 8>{}); break;
    case 3072: go(std::integral_constant<int, 6>{}); break;
    case 2048: go(std::integral_constant<int, 4>{}); break;
    case 1024: go(std::integral_constant<int, 2>{}); break;
    case 512: go(std::integral_constant<int, 1>{}); break;
    default: go(std::integral_constant<int, 0>{}); break;
  }
  return check_launch();
}

// One design alternative (ablation.h) through the one-row kernel, at K = 512 or 5120.
template <int VAR>
int launch_small_variant(const uint16_t* x, const float* xs, const uint8_t* packed, const uint16_t* S,
                         const uint16_t* ZS, int N, int K, int kc, float* cs, int32_t* ci, hipStream_t s) {
  const int nblk = (int)nblk_of(N);
  const size_t lds = small_lds_bytes(K, 1, true, VAR == kVarG64 ? 64 : kGroup);
  auto go = [&](auto ngc) {
    hipLaunchKernelGGL((coarse_small_kernel<1, true, decltype(ngc)::value, VAR>), dim3(nblk), dim3(kCoarseThreads), lds,
                       s, x, xs, 1, packed, S, ZS, N, K, kc, nblk, cs, ci, nullptr, nullptr, nullptr);
  };
  if (K == 5120) go(std::integral_constant<int, 10>{});
  else go(std::integral_constant<int, 1>{});
  return check_launch();
}

// True when the small kernel keeps x in LDS for M rows of K (and then sums the groups itself).
bool small_sums_x(int64_t M, int64_t K) {
  return (M <= 2 && small_lds_bytes((int)K, (int)M, true) <= 65536) || (M <= 4 && small_lds_bytes((int)K, 4, true) <= 65536);
}

}  // namespace

// True when every launch coarse_launch makes for M rows of K sums the groups of x itself: rows
// go in chunks of kTileMaxRows, a one-row chunk runs the small kernel (which sums x when x fits in
// its LDS), a larger chunk the tile kernel where it is built for K (which sums x up to 32 rows),
// else the small kernel up to 4 rows (x in its LDS) or the generic kernel (which needs the sums).
bool coarse_sums_x(int64_t M, int64_t K) {
  if (M < 1 || check_k(K) != I2H_OK) return false;
  auto chunk = [&](int64_t mc) {
    if (mc == 1) return small_sums_x(1, K);
    if (tile_supported(mc, K)) return tile_sums_x(mc, K);
    return mc <= 4 && small_sums_x(mc, K);
  };
  if (M > kTileMaxRows && !chunk(kTileMaxRows)) return false;
  return chunk((M - 1) % kTileMaxRows + 1);
}

namespace {

// M <= 4 rows.
int small_band(const uint16_t* x, const float* xs, int M, const uint8_t* packed, const uint16_t* S,
               const uint16_t* ZS, int N, int K, int kc, float* cs, int32_t* ci, uint16_t* y, float* bmax, int32_t* zc,
               hipStream_t s) {
  if (M == 1 && small_lds_bytes(K, 1, true) <= 65536)
    return launch_small<1, true>(x, xs, M, packed, S, ZS, N, K, kc, cs, ci, y, bmax, zc, s);
  if (M == 2 && small_lds_bytes(K, 2, true) <= 65536)
    return launch_small<2, true>(x, xs, M, packed, S, ZS, N, K, kc, cs, ci, y, bmax, zc, s);
  if (M <= 4 && small_lds_bytes(K, 4, true) <= 65536)
    return launch_small<4, true>(x, xs, M, packed, S, ZS, N, K, kc, cs, ci, y, bmax, zc, s);
  return launch_small<4, false>(x, xs, M, packed, S, ZS, N, K, kc, cs, ci, y, bmax, zc, s);
}

// The generic kernel (global A loads, any K) for up to kTileMaxRows rows; needs xs.
int generic_rows(const uint16_t* x, const float* xs, int M, const uint8_t* packed, const uint16_t* S,
                 const uint16_t* ZS, int N, int K, int kc, float* cs, int32_t* ci, uint16_t* y, float* bmax,
                 hipStream_t s) {
  if (!xs) return I2H_ERR_ARG;
  if (M <= 16) return launch_coarse<1>(x, xs, M, packed, S, ZS, N, K, kc, cs, ci, y, bmax, s);
  if (M <= 32) return launch_coarse<2>(x, xs, M, packed, S, ZS, N, K, kc, cs, ci, y, bmax, s);
  return launch_coarse<4>(x, xs, M, packed, S, ZS, N, K, kc, cs, ci, y, bmax, s);
}

}  // namespace

int small_variant_launch(int var, const uint16_t* x, const float* xs, const uint8_t* packed, const uint16_t* S,
                         const uint16_t* ZS, int64_t N, int64_t K, int kc, float* cs, int32_t* ci, hipStream_t s) {
  if (K != 512 && K != 5120) return I2H_ERR_SHAPE;
  switch (var) {
    case kVarDesign: return coarse_launch(x, xs, 1, packed, S, ZS, N, K, kc, cs, ci, nullptr, s);
    case kVarG64: return launch_small_variant<kVarG64>(x, xs, packed, S, ZS, (int)N, (int)K, kc, cs, ci, s);
    case kVarC4: return launch_small_variant<kVarC4>(x, xs, packed, S, ZS, (int)N, (int)K, kc, cs, ci, s);
    case kVarWTile: return launch_small_variant<kVarWTile>(x, xs, packed, S, ZS, (int)N, (int)K, kc, cs, ci, s);
    default: return I2H_ERR_ARG;
  }
}

int xsum_launch(const uint16_t* x, int64_t M, int64_t K, float* xs, hipStream_t s, int32_t* zero_cnt) {
  if (!x || !xs) return I2H_ERR_ARG;
  // whole groups suffice here (the int4 head allows K a multiple of 256)
  if (M < 1 || K <= 0 || K % kGroup != 0 || K > I2H_MAX_K || M * (K / kGroup) > (int64_t)1 << 30)
    return I2H_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(xs, 4)) return I2H_ERR_ALIGN;
  if (zero_cnt && !aligned(zero_cnt, 4)) return I2H_ERR_ALIGN;
  hipLaunchKernelGGL(xsum_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, x, (int)M, (int)K, xs, zero_cnt);
  return check_launch();
}

int coarse_launch(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed,
                  const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int kcand,
                  float* cand_score, int32_t* cand_idx, uint16_t* y, hipStream_t s, int32_t* zero_cnt,
                  float* bmax) {
  if (!x || !packed || !S || !ZS || !cand_score || !cand_idx) return I2H_ERR_ARG;
  if (!xs && !coarse_sums_x(M, K)) return I2H_ERR_ARG;  // in-kernel group sums need x in LDS
  if (M < 1 || N < 1 || N > ((int64_t)1 << 30) || check_k(K) != I2H_OK) return I2H_ERR_SHAPE;
  if (kcand < 1 || kcand > I2H_MAX_KCAND) return I2H_ERR_LIMIT;
  if (!aligned(x, 16) || !aligned(packed, 16) || !aligned(xs, 4) || !aligned(S, 16) || !aligned(ZS, 16) ||
      !aligned(cand_score, 4) || !aligned(cand_idx, 4) || (y && !aligned(y, 2)))
    return I2H_ERR_ALIGN;
  // only the small kernel zeroes counters: the caller passes them when every row runs there
  if (zero_cnt && (xs || !coarse_sums_x(M, K) || !aligned(zero_cnt, 4))) return I2H_ERR_ARG;
  const int64_t ld = nblk_of(N) * kcand;
  // rows go in chunks of kTileMaxRows; a chunk of one or two rows (x in LDS; from three rows the
  // 16-row tile is faster: x for 3 or 4 rows costs the small kernel occupancy), or of at most 4
  // rows with a K the tile kernel is not built for, runs the small kernel; a larger one the tile
  // kernel where it is built for K, else the generic kernel
  for (int64_t m0 = 0; m0 < M; m0 += kTileMaxRows) {
    const int64_t mc = M - m0 < kTileMaxRows ? M - m0 : kTileMaxRows;
    const uint16_t* xc = x + m0 * K;
    const float* xsc = xs ? xs + m0 * (K / kGroup) : nullptr;
    float* csc = cand_score + m0 * ld;
    int32_t* cic = cand_idx + m0 * ld;
    float* bmc = bmax ? bmax + m0 * nblk_of(N) : nullptr;
    uint16_t* yc = y ? y + m0 * N : nullptr;
    int32_t* zcc = zero_cnt ? zero_cnt + m0 : nullptr;
    const bool tile_ok = tile_supported(mc, K);
    int st;
    if ((mc <= 2 && small_sums_x(mc, K)) || (mc <= 4 && !tile_ok))
      st = xsc || small_sums_x(mc, K)
               ? small_band(xc, xsc, (int)mc, packed, S, ZS, (int)N, (int)K, kcand, csc, cic, yc, bmc, zcc, s)
               : I2H_ERR_ARG;
    else if (tile_ok)
      // every other chunk takes the blocks in reverse order: it starts on the blocks the chunk
      // before it read last, which the memory-side cache may still hold
      st = tile_launch(xc, xsc, mc, packed, S, ZS, N, K, kcand, csc, cic, yc, bmc, zcc, s,
                       (int)((m0 / kTileMaxRows) & 1));
    else if (!xsc)
      st = I2H_ERR_ARG;
    else
      st = generic_rows(xc, xsc, (int)mc, packed, S, ZS, (int)N, (int)K, kcand, csc, cic, yc, bmc, s);
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
