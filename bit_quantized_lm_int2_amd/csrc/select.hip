// Top-R selection over the block candidates, and the final argmax / top-k.
//
// radiance_drafthead.py, _apply_head_int2: the RERANK best of a row's block candidates are the
// ones rescored exactly; a top-k caller draws only from the reranked tokens, an argmax caller
// wins on the exact scores (module docstring).
//
// Selection uses the block structure of the candidates: each block's KCAND entries are best
// first, so every member of the row's top R belongs to a block whose best entry is itself in
// the top R of the block maxima (all entries of that block ranked above the member are in the
// top R too, its best entry among them). One workgroup per row therefore ranks the NBLK block
// maxima, keeps the R best blocks, and ranks their R*KCAND entries. Ranking is by a 64-bit key
// (score descending, then token index ascending), sorted bitonically in LDS.
#include "device_util.h"
#include "host_util.h"

namespace i2h {
namespace {

constexpr int kSelectThreads = 1024;
constexpr int kSelectMaxKeys = 8192;   // LDS keys: max(NBLK, R * KCAND) <= 8192 (64 KiB)
constexpr int kPerThread = kSelectMaxKeys / kSelectThreads;

__global__ __launch_bounds__(kSelectThreads) void select_kernel(const float* __restrict__ cs,
                                                               const int32_t* __restrict__ ci,
                                                               int nblk, int kc, int R,
                                                               int32_t* __restrict__ sel) {
  extern __shared__ uint64_t keys[];
  const int m = blockIdx.x;
  const int64_t ld = (int64_t)nblk * kc;
  const float* s = cs + m * ld;
  const int32_t* c = ci + m * ld;

  // Stage 1: block maxima. Equal maxima rank by block position, which orders them by token
  // index because block b holds tokens 64b .. 64b+63.
  const int n1 = pow2_at_least(nblk);
  for (int b = threadIdx.x; b < n1; b += kSelectThreads) {
    uint64_t k = 0ull;
    if (b < nblk && c[(int64_t)b * kc] >= 0)
      k = ((uint64_t)ordered_key(s[(int64_t)b * kc]) << 32) | (uint64_t)(~(uint32_t)b);
    keys[b] = k;
  }
  __syncthreads();
  block_sort_desc(keys, n1);

  // Stage 2: every entry of the best min(R, nblk) blocks.
  const int nb = R < nblk ? R : nblk;
  const int n2 = pow2_at_least(nb * kc);
  uint64_t mine[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int t = threadIdx.x + i * kSelectThreads;
    uint64_t k = 0ull;
    if (t < nb * kc) {
      const uint64_t bk = keys[t / kc];
      if (bk != 0ull) {
        const int64_t at = (int64_t)(~(uint32_t)bk) * kc + (t % kc);
        k = rank_key(s[at], c[at]);
      }
    }
    mine[i] = k;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int t = threadIdx.x + i * kSelectThreads;
    if (t < n2) keys[t] = mine[i];
  }
  __syncthreads();
  block_sort_desc(keys, n2);
  for (int j = threadIdx.x; j < R; j += kSelectThreads)
    sel[(int64_t)m * R + j] = j < n2 ? rank_key_idx(keys[j]) : -1;
}

// ---------------------------------------------------------------------------------------------
// Fast path for R <= 64 and R * KCAND <= 1024, with five barriers per ranking. Each of the 16
// waves sorts its share of the keys in registers (a bitonic network over shuffles) and keeps
// its best R' (R' = the power of two >= R). The 16 sorted lists are then merged pairwise in a
// tree: for sorted lists A and B, max(A[i], B[R'-1-i]) is a bitonic sequence that holds the R'
// best of both, and one bitonic clean (log2 R' shuffle stages) sorts it.
// ---------------------------------------------------------------------------------------------
constexpr int kFastWaves = kSelectThreads / kWave;  // 16

struct FastLds {
  uint64_t lists[kFastWaves][64];
  uint64_t top[64];
};

// Top R (R <= 64) of the keys the waves hold (KPL per lane, 0 = empty), best first, into
// L.top[0 .. R). Every thread of the block must call it.
template <int KPL>
__device__ void block_top_r(uint64_t (&k)[KPL], int R, FastLds& L) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int Rp = pow2_at_least(R);
  wave_sort_keys<KPL>(k, lane);
  if (lane < Rp) L.lists[wave][lane] = k[0];
  __syncthreads();
  for (int step = 1; step < kFastWaves; step <<= 1) {
    if ((wave & (2 * step - 1)) == 0) {
      const uint64_t a = lane < Rp ? L.lists[wave][lane] : 0ull;
      const uint64_t b = lane < Rp ? L.lists[wave + step][Rp - 1 - lane] : 0ull;
      uint64_t v = a > b ? a : b;
      for (int stride = Rp >> 1; stride > 0; stride >>= 1) {
        const uint64_t o = shfl_xor_u64(v, stride);
        const bool lower = (lane & stride) == 0;
        v = (lower == (o > v)) ? o : v;
      }
      if (lane < Rp) L.lists[wave][lane] = v;
    }
    __syncthreads();
  }
  if (threadIdx.x < R) L.top[threadIdx.x] = L.lists[0][threadIdx.x];
  __syncthreads();
}

template <int KPL>
__global__ __launch_bounds__(kSelectThreads) void select_fast_kernel(const float* __restrict__ cs,
                                                                    const int32_t* __restrict__ ci,
                                                                    int nblk, int kc, int R,
                                                                    int32_t* __restrict__ sel) {
  __shared__ FastLds L;
  const int m = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ld = (int64_t)nblk * kc;
  const float* s = cs + m * ld;
  const int32_t* c = ci + m * ld;
  // stage 1: block maxima, wave w holds blocks w*64*KPL + e*64 + lane
  uint64_t k1[KPL];
#pragma unroll
  for (int e = 0; e < KPL; ++e) {
    const int b = wave * 64 * KPL + e * 64 + lane;
    uint64_t key = 0ull;
    if (b < nblk && c[(int64_t)b * kc] >= 0)
      key = ((uint64_t)ordered_key(s[(int64_t)b * kc]) << 32) | (uint64_t)(~(uint32_t)b);
    k1[e] = key;
  }
  block_top_r<KPL>(k1, R, L);
  // stage 2: every entry of the chosen blocks, one per thread
  const int nb = R < nblk ? R : nblk;
  const int t = threadIdx.x;
  uint64_t k2[1] = {0ull};
  if (t < nb * kc) {
    const uint64_t bk = L.top[t / kc];
    if (bk != 0ull) {
      const int64_t at = (int64_t)(~(uint32_t)bk) * kc + (t % kc);
      k2[0] = rank_key(s[at], c[at]);
    }
  }
  __syncthreads();  // L.lists and L.top are rewritten below
  block_top_r<1>(k2, R, L);
  if (t < R) sel[(int64_t)m * R + t] = rank_key_idx(L.top[t]);
}

__global__ __launch_bounds__(256) void finalize_kernel(const float* __restrict__ ex,
                                                       const int32_t* __restrict__ sel, int R, int k,
                                                       int32_t* __restrict__ oi, float* __restrict__ ov) {
  extern __shared__ uint64_t keys[];
  const int m = blockIdx.x;
  const int n = pow2_at_least(R);
  for (int j = threadIdx.x; j < n; j += blockDim.x)
    keys[j] = j < R ? rank_key(ex[(int64_t)m * R + j], sel[(int64_t)m * R + j]) : 0ull;
  __syncthreads();
  block_sort_desc(keys, n);
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    oi[(int64_t)m * k + j] = rank_key_idx(keys[j]);
    ov[(int64_t)m * k + j] = rank_key_score(keys[j]);
  }
}

int host_pow2(int64_t n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

}  // namespace

int select_launch(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk,
                  int kcand, int R, int32_t* sel, hipStream_t s) {
  if (!cand_score || !cand_idx || !sel) return I2H_ERR_ARG;
  if (M < 1 || M > (1 << 30) || nblk < 1 || nblk > I2H_MAX_NBLK) return I2H_ERR_SHAPE;
  if (kcand < 1 || kcand > I2H_MAX_KCAND || R < 1 || R > I2H_MAX_R ||
      (int64_t)R * kcand > kSelectMaxKeys)
    return I2H_ERR_LIMIT;
  if (!aligned(cand_score, 4) || !aligned(cand_idx, 4) || !aligned(sel, 4)) return I2H_ERR_ALIGN;
  const int64_t nb = R < nblk ? R : nblk;
  if (R <= 64 && (int64_t)R * kcand <= kSelectThreads) {
    if (nblk <= 1024)
      hipLaunchKernelGGL(select_fast_kernel<1>, dim3((unsigned)M), dim3(kSelectThreads), 0, s, cand_score, cand_idx,
                         (int)nblk, kcand, R, sel);
    else if (nblk <= 2048)
      hipLaunchKernelGGL(select_fast_kernel<2>, dim3((unsigned)M), dim3(kSelectThreads), 0, s, cand_score, cand_idx,
                         (int)nblk, kcand, R, sel);
    else if (nblk <= 4096)
      hipLaunchKernelGGL(select_fast_kernel<4>, dim3((unsigned)M), dim3(kSelectThreads), 0, s, cand_score, cand_idx,
                         (int)nblk, kcand, R, sel);
    else
      hipLaunchKernelGGL(select_fast_kernel<8>, dim3((unsigned)M), dim3(kSelectThreads), 0, s, cand_score, cand_idx,
                         (int)nblk, kcand, R, sel);
    return check_launch();
  }
  const int keys = host_pow2(nblk > nb * kcand ? nblk : nb * kcand);
  hipLaunchKernelGGL(select_kernel, dim3((unsigned)M), dim3(kSelectThreads), (size_t)keys * 8, s,
                     cand_score, cand_idx, (int)nblk, kcand, R, sel);
  return check_launch();
}

int finalize_launch(const float* exact, const int32_t* sel, int64_t M, int R, int k, int32_t* out_idx,
                    float* out_val, hipStream_t s) {
  if (!exact || !sel || !out_idx || !out_val) return I2H_ERR_ARG;
  if (M < 1 || M > (1 << 30)) return I2H_ERR_SHAPE;
  if (R < 1 || R > I2H_MAX_R || k < 1 || k > R) return I2H_ERR_LIMIT;
  if (!aligned(exact, 4) || !aligned(sel, 4) || !aligned(out_idx, 4) || !aligned(out_val, 4))
    return I2H_ERR_ALIGN;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)M), dim3(256), (size_t)host_pow2(R) * 8, s, exact,
                     sel, R, k, out_idx, out_val);
  return check_launch();
}

}  // namespace i2h

extern "C" int i2h_select(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk,
                          int kcand, int R, int32_t* sel, void* stream) {
  return i2h::select_launch(cand_score, cand_idx, M, nblk, kcand, R, sel, (hipStream_t)stream);
}

extern "C" int i2h_finalize(const float* exact, const int32_t* sel, int64_t M, int R, int k,
                            int32_t* out_idx, float* out_val, void* stream) {
  return i2h::finalize_launch(exact, sel, M, R, k, out_idx, out_val, (hipStream_t)stream);
}
