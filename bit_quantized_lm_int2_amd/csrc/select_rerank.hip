// Top-R selection, exact rerank and final top-k in one kernel, one workgroup per row.
//
// radiance_drafthead.py, _apply_head_int2 / _rerank_exact: the RERANK best of the row's block
// candidates (score descending, token ascending) are rescored exactly against their bf16 weight
// rows, and the final argmax or top-k is drawn from those exact scores only.
//
// For small M this tail is latency-bound (one row per workgroup, a chain of dependent steps).
// The x row goes to LDS while the best entry of every block is ranked (each thread holds up to 4
// blocks; a block's list is best first, so the R best entries of the row lie in the R best
// blocks), then the entries of the R best blocks are gathered and ranked, and the R weight rows
// are gathered with every load in flight.
// Ranking runs in registers on fp64-coded keys (wave_rank.h); 16 waves meet in a merge tree.
// The exact dot products use the same lane mapping and summation order as rerank.hip, so both
// paths give the same bits.
#include "dequant.h"
#include "host_util.h"
#include "wave_rank.h"

namespace i2h {
namespace {

constexpr int kSrThreads = 1024;
constexpr int kSrWaves = kSrThreads / kWave;  // 16
constexpr int kSrMaxR = 64, kSrMaxKc = 8;
constexpr int kSrChunk = 10;  // 512-k steps of the two weight rows a wave has in flight at once

struct SrLds {
  double lists[kSrWaves][64];
  double top[64];
  int32_t sel[kSrMaxR];
  float ex[kSrMaxR];
};
constexpr size_t kSrLdsHead = (sizeof(SrLds) + 15) / 16 * 16;

// The 64 best of the first NW (a power of two) waves' 64-lists, best first, into L.top. Every
// thread of the block calls it with its lane's entry of its wave's sorted list.
__device__ void merge_waves(SrLds& L, double mine, int NW) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave < NW) L.lists[wave][lane] = mine;
  __syncthreads();
  for (int step = 1; step < NW; step <<= 1) {
    // an active wave reads its list and its partner's (inactive at this step) and rewrites its own
    if ((wave & (2 * step - 1)) == 0 && wave < NW) {
      const double v = wave_merge64_f64(L.lists[wave][lane], L.lists[wave + step]);
      L.lists[wave][lane] = v;
    }
    __syncthreads();
  }
  if (wave == 0) L.top[lane] = L.lists[0][lane];
  __syncthreads();
}

template <int BPT>
__global__ __launch_bounds__(kSrThreads) void select_rerank_kernel(
    const float* __restrict__ cs, const int32_t* __restrict__ ci, int nblk, int kc, int R,
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ W, int64_t ldw, int N, int K, int k,
    int32_t* __restrict__ sel_out, float* __restrict__ ex_out, int32_t* __restrict__ oi,
    float* __restrict__ ov) {
  extern __shared__ __align__(16) uint8_t smem[];
  SrLds& L = *reinterpret_cast<SrLds*>(smem);
  uint16_t* xl = reinterpret_cast<uint16_t*>(smem + kSrLdsHead);
  const int m = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t ld = (int64_t)nblk * kc;
  const float* s = cs + (int64_t)m * ld;
  const int32_t* c = ci + (int64_t)m * ld;

  // --- the best entry of each of this thread's blocks (t + 1024 j), and the x row into LDS
  double srt[BPT];
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    const int b = tid + kSrThreads * j;
    float v = -__builtin_inff();
    int32_t t = -1;
    if (b < nblk) {
      v = s[(int64_t)b * kc];
      t = c[(int64_t)b * kc];
    }
    srt[j] = token_key(v, t);
  }
  const uint16_t* xr = x + (int64_t)m * K;
  for (int u = tid; u < K / 8; u += kSrThreads)
    *reinterpret_cast<u32x4*>(xl + 8 * u) = ld16(xr + 8 * u);

  // --- the R best blocks, by their best entry
  wave_sort_f64<BPT>(srt);
  merge_waves(L, srt[0], kSrWaves);

  // --- every entry of those blocks (thread t: entry t % kc of block rank t / kc), ranked. A
  // block's key holds the token of its best entry, and block b holds tokens 64 b .. 64 b + 63.
  const int nsel = R * kc;
  double ek[1] = {0.0};
  if (tid < nsel) {
    const double bkey = L.top[tid / kc];
    if (bkey > 0.0) {
      const int64_t at = (int64_t)(token_key_token(bkey) / kBlockN) * kc + tid % kc;
      ek[0] = token_key(s[at], c[at]);
    }
  }
  const int nw = nsel <= 64 ? 1 : (nsel <= 128 ? 2 : (nsel <= 256 ? 4 : 8));
  if (wave < nw) wave_sort_f64<1>(ek);
  merge_waves(L, ek[0], nw);  // its first barrier follows every read of L.top above
  if (tid < R) L.sel[tid] = token_key_token(L.top[tid]);
  __syncthreads();

  // --- exact rerank: wave w scores selected tokens w, w + 16, ... two rows at a time, with the
  // loads of both rows (up to kSrChunk 512-k steps each) in flight together
  const int steps = K / 512;
  for (int j0 = wave; j0 < R; j0 += 2 * kSrWaves) {
    const int j1 = j0 + kSrWaves;
    const int n0 = L.sel[j0], n1 = j1 < R ? L.sel[j1] : -1;
    const bool v0 = n0 >= 0 && n0 < N, v1 = n1 >= 0 && n1 < N;
    const uint16_t* w0 = W + (int64_t)(v0 ? n0 : 0) * ldw + 8 * lane;
    const uint16_t* w1 = W + (int64_t)(v1 ? n1 : 0) * ldw + 8 * lane;
    float a00 = 0.f, a01 = 0.f, a10 = 0.f, a11 = 0.f;
    for (int i0 = 0; i0 < steps; i0 += kSrChunk) {
      u32x4 r0[kSrChunk], r1[kSrChunk];
#pragma unroll
      for (int i = 0; i < kSrChunk; ++i) {
        const bool in = i0 + i < steps;
        r0[i] = in && v0 ? ld16(w0 + 512 * (i0 + i)) : u32x4{0u, 0u, 0u, 0u};
        r1[i] = in && v1 ? ld16(w1 + 512 * (i0 + i)) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kSrChunk; ++i) {
        if (i0 + i < steps) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xl + 8 * lane + 512 * (i0 + i));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a00 = fmaf(bf16_lo(xv[e]), bf16_lo(r0[i][e]), a00);
            a01 = fmaf(bf16_hi(xv[e]), bf16_hi(r0[i][e]), a01);
            a10 = fmaf(bf16_lo(xv[e]), bf16_lo(r1[i][e]), a10);
            a11 = fmaf(bf16_hi(xv[e]), bf16_hi(r1[i][e]), a11);
          }
        }
      }
    }
    float d0 = a00 + a01, d1 = a10 + a11;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      d0 += __shfl_xor(d0, o);
      d1 += __shfl_xor(d1, o);
    }
    if (lane == 0) {
      L.ex[j0] = v0 ? d0 : -__builtin_inff();
      if (j1 < R) L.ex[j1] = v1 ? d1 : -__builtin_inff();
    }
  }
  __syncthreads();

  // --- outputs: the selection and its exact scores (optional), the k best by exact score
  if (tid < R) {
    if (sel_out != nullptr) sel_out[(int64_t)m * R + tid] = L.sel[tid];
    if (ex_out != nullptr) ex_out[(int64_t)m * R + tid] = L.ex[tid];
  }
  if (wave == 0) {
    double fk[1] = {lane < R ? token_key(L.ex[lane], L.sel[lane]) : 0.0};
    wave_sort_f64<1>(fk);
    if (lane < k) {
      oi[(int64_t)m * k + lane] = token_key_token(fk[0]);
      ov[(int64_t)m * k + lane] = token_key_score(fk[0]);
    }
  }
}

}  // namespace

bool select_rerank_supported(int64_t nblk, int kc, int R, int64_t N, int64_t K) {
  return nblk >= 1 && nblk <= 4 * kSrThreads && kc >= 1 && kc <= kSrMaxKc && R >= 1 && R <= kSrMaxR &&
         N >= 1 && N <= (int64_t)1 << 19 && check_k(K) == I2H_OK;
}

int select_rerank_launch(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk, int kc, int R,
                         const uint16_t* x, const uint16_t* W, int64_t ldw, int64_t N, int64_t K, int k,
                         int32_t* sel, float* exact, int32_t* out_idx, float* out_val, hipStream_t s) {
  if (!cand_score || !cand_idx || !x || !W || !out_idx || !out_val) return I2H_ERR_ARG;
  if (M < 1 || M > (1 << 30) || nblk != nblk_of(N) || ldw < K) return I2H_ERR_SHAPE;
  if (!select_rerank_supported(nblk, kc, R, N, K)) return I2H_ERR_LIMIT;
  if (k < 1 || k > R) return I2H_ERR_LIMIT;
  if (!aligned(cand_score, 4) || !aligned(cand_idx, 4) || !aligned(x, 16) || !aligned(W, 16) || ldw % 8 != 0 ||
      !aligned(out_idx, 4) || !aligned(out_val, 4) || (sel && !aligned(sel, 4)) || (exact && !aligned(exact, 4)))
    return I2H_ERR_ALIGN;
  const size_t lds = kSrLdsHead + (size_t)K * 2;
  const dim3 grid((unsigned)M), block(kSrThreads);
  if (nblk <= kSrThreads)
    hipLaunchKernelGGL(select_rerank_kernel<1>, grid, block, lds, s, cand_score, cand_idx, (int)nblk, kc, R, x, W,
                       ldw, (int)N, (int)K, k, sel, exact, out_idx, out_val);
  else if (nblk <= 2 * kSrThreads)
    hipLaunchKernelGGL(select_rerank_kernel<2>, grid, block, lds, s, cand_score, cand_idx, (int)nblk, kc, R, x, W,
                       ldw, (int)N, (int)K, k, sel, exact, out_idx, out_val);
  else
    hipLaunchKernelGGL(select_rerank_kernel<4>, grid, block, lds, s, cand_score, cand_idx, (int)nblk, kc, R, x, W,
                       ldw, (int)N, (int)K, k, sel, exact, out_idx, out_val);
  return check_launch();
}

}  // namespace i2h

extern "C" int i2h_select_rerank_topk(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk,
                                      int kcand, int R, const uint16_t* x, const uint16_t* W, int64_t ldw, int64_t N,
                                      int64_t K, int k, int32_t* sel, float* exact, int32_t* out_idx, float* out_val,
                                      void* stream) {
  return i2h::select_rerank_launch(cand_score, cand_idx, M, nblk, kcand, R, x, W, ldw, N, K, k, sel, exact, out_idx,
                                   out_val, (hipStream_t)stream);
}
