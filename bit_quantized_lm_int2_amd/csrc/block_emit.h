// Block top-KCAND emit from a transposed block of coarse logits (gfx950, wave64).
//
// radiance_drafthead.py, _emit: for every row, the KCAND best of the block's 64 columns, best
// first, ties to the lower column. The block's logits sit in LDS as tw[row][column] (row stride
// kTRow floats, -inf past the vocabulary's end); keys are fp64-coded (value, column) so that a
// compare-exchange is v_max_f64 + v_min_f64.
#pragma once
#include "dequant.h"
#include "device_util.h"

namespace i2h {

constexpr int kTRow = 65;  // floats per row of a transposed block (odd: no bank conflicts)

// fp64 ranking key of (value, column in block): the bits 0x3FF | (ordered_key(v) << 6 | 63 - col)
// placed in the mantissa of a double in [1, 2), so double order is (value desc, column asc).
__device__ __forceinline__ double key_f64(float v, int c) {
  const uint32_t u = ordered_key(v);
  const uint32_t hi = 0x3FF00000u | (u >> 12);
  const uint32_t lo = (u << 20) | ((uint32_t)(63 - c) << 14);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float key_value(double k) {
  const uint64_t b = __builtin_bit_cast(uint64_t, k);
  const uint32_t hi = (uint32_t)(b >> 32), lo = (uint32_t)b;
  return from_ordered_key((hi << 12) | (lo >> 20));
}
__device__ __forceinline__ int key_col(double k) {
  return 63 - (int)(((uint32_t)__builtin_bit_cast(uint64_t, k) >> 14) & 63u);
}

__device__ __forceinline__ void cx(double& a, double& b) {  // a <- larger, b <- smaller
  const double hi = __builtin_fmax(a, b), lo = __builtin_fmin(a, b);
  a = hi;
  b = lo;
}

// Descending sort of 8 keys: a 19-comparator network.
__device__ __forceinline__ void sort8(double* k) {
  cx(k[0], k[2]); cx(k[1], k[3]); cx(k[4], k[6]); cx(k[5], k[7]);
  cx(k[0], k[4]); cx(k[1], k[5]); cx(k[2], k[6]); cx(k[3], k[7]);
  cx(k[0], k[1]); cx(k[2], k[3]); cx(k[4], k[5]); cx(k[6], k[7]);
  cx(k[2], k[4]); cx(k[3], k[5]);
  cx(k[1], k[4]); cx(k[3], k[6]);
  cx(k[1], k[2]); cx(k[3], k[4]); cx(k[5], k[6]);
}

// a <- the 8 largest of two descending lists a, b (descending): the elementwise maximum of a and
// reversed b is a bitonic sequence holding them, then three half-cleaner stages.
__device__ __forceinline__ void merge_top8(double* a, const double* b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = __builtin_fmax(a[i], b[7 - i]);
#pragma unroll
  for (int st = 4; st > 0; st >>= 1)
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i & st) == 0) cx(a[i], a[i + st]);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, 0xF, 0xF, false);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Block top-kc (kc <= 8) of the wave's block for rows < M. tw[m][c] holds the block's logits
// (-inf past column N). P lanes share a row, each ranking 64 / P of its columns; the P partial
// top-8 lists meet through DPP quad permutes. The lists are then staged in the wave's own rows of
// tw ([MR][16]: 8 scores, 8 indices) and stored by 8 consecutive lanes per row, so that each store
// instruction writes one 32-byte run per row: one scattered dword per lane and slot had made the
// stores, not the ranking, most of the emit's time at 32 and 64 rows (8x the memory requests).
template <int MR, int P>
__device__ __forceinline__ void emit_top8(float* tw, int M, int b, int N, int kc, int64_t ld,
                                          float* __restrict__ cand_score, int32_t* __restrict__ cand_idx,
                                          float* __restrict__ bmax) {
  constexpr int V = 64 / P;
  const int lane = threadIdx.x & 63;
  const int row = lane / P, part = lane % P;
  const float* tr = tw + (row < MR ? row : MR - 1) * kTRow + part * V;
  double k[V];
#pragma unroll
  for (int i = 0; i < V; ++i) k[i] = key_f64(tr[i], part * V + i);
#pragma unroll
  for (int g = 0; g < V / 8; ++g) sort8(k + 8 * g);
#pragma unroll
  for (int w = 8; w < V; w <<= 1)
#pragma unroll
    for (int g = 0; g < V; g += 2 * w) merge_top8(k + g, k + g + w);
  if constexpr (P >= 2) {
    double o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = dpp_f64<0xB1>(k[i]);  // quad_perm [1,0,3,2]: lane ^ 1
    merge_top8(k, o);
  }
  if constexpr (P >= 4) {
    double o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = dpp_f64<0x4E>(k[i]);  // quad_perm [2,3,0,1]: lane ^ 2
    merge_top8(k, o);
  }
  // every lane's reads of tw are issued above; LDS operations of one wave complete in order, and
  // this keeps the compiler from moving the staging writes above them
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t* stg = reinterpret_cast<uint32_t*>(tw);  // [MR][16]
  if (part == 0 && row < MR) {
    u32x4 sc[2], ix[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tok = b * kBlockN + key_col(k[i]);
      const bool ok = tok < N;
      sc[i >> 2][i & 3] = __float_as_uint(ok ? key_value(k[i]) : -__builtin_inff());
      ix[i >> 2][i & 3] = (uint32_t)(ok ? tok : -1);
    }
    u32x4* d = reinterpret_cast<u32x4*>(stg + row * 16);
    d[0] = sc[0];
    d[1] = sc[1];
    d[2] = ix[0];
    d[3] = ix[1];
    if (bmax != nullptr && row < M) bmax[(int64_t)row * (ld / kc) + b] = __uint_as_float(sc[0][0]);
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const int sl = lane & 7;
#pragma unroll
  for (int j = 0; j < MR / 8; ++j) {
    const int r = 8 * j + (lane >> 3);
    if (r < M && sl < kc) {
      const int64_t at = (int64_t)r * ld + (int64_t)b * kc + sl;
      cand_score[at] = __uint_as_float(stg[r * 16 + sl]);
      cand_idx[at] = (int32_t)stg[r * 16 + 8 + sl];
    }
  }
}

// Block top-kc for any kc <= 64: lane c counts the columns of its row that rank before it.
template <int MR>
__device__ void emit_counted(const float* tw, int M, int b, int N, int kc, int64_t ld,
                             float* __restrict__ cand_score, int32_t* __restrict__ cand_idx,
                             float* __restrict__ bmax) {
  const int lane = threadIdx.x & 63;
  for (int m = 0; m < M && m < MR; ++m) {
    const float* tr = tw + m * kTRow;
    const float v = tr[lane];
    int rank = 0;
    for (int j = 0; j < kBlockN; ++j) {
      const float o = tr[j];
      rank += (o > v) || (o == v && j < lane);
    }
    if (rank < kc) {
      const int tok = b * kBlockN + lane;
      const bool ok = tok < N;
      const int64_t at = (int64_t)m * ld + (int64_t)b * kc + rank;
      cand_score[at] = ok ? v : -__builtin_inff();
      cand_idx[at] = ok ? tok : -1;
      if (rank == 0 && bmax != nullptr) bmax[(int64_t)m * (ld / kc) + b] = ok ? v : -__builtin_inff();
    }
  }
}

}  // namespace i2h
