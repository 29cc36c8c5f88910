// Host-side helpers shared by the entry points of libi2h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "i2h.h"

namespace i2h {

// Records a failed HIP call for i2h_last_hip_error() and returns I2H_ERR_HIP.
int record_hip_error(hipError_t e);

// Checks the launch that was just enqueued.
inline int check_launch() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? I2H_OK : record_hip_error(e);
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline int check_k(int64_t K) {
  return (K > 0 && K <= I2H_MAX_K && K % (4 * I2H_GROUP) == 0) ? I2H_OK : I2H_ERR_SHAPE;
}

inline int64_t nblk_of(int64_t N) { return (N + I2H_BLOCK_N - 1) / I2H_BLOCK_N; }

// True when the coarse kernel for M rows of K keeps x in LDS and sums its groups itself, so the
// head needs no separate group-sum launch (coarse_launch then accepts xs == nullptr).
bool coarse_sums_x(int64_t M, int64_t K);

// The many-row coarse kernel (coarse_tile.hip): up to kTileMaxRows rows of x per launch, for the
// K it is built for; it takes the group sums xs from i2h_xsum, or sums x itself when xs is null
// and tile_sums_x (up to 32 rows). zc (may be null): M ints the launch sets to 0. bmax (may be
// null): [M, nblk] floats, each block's best score per row (the first slot of its list). rev:
// the blocks are taken in reverse order (for a second launch over the same weights).
constexpr int64_t kTileMaxRows = 64;
bool tile_supported(int64_t M, int64_t K);
bool tile_sums_x(int64_t M, int64_t K);
int tile_launch(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed, const uint16_t* S,
                const uint16_t* ZS, int64_t N, int64_t K, int kc, float* cs, int32_t* ci, uint16_t* y, float* bmax,
                int32_t* zc, hipStream_t s, int rev = 0);

// The design alternatives (ablation.h: var) through the production kernels, for the checks of
// i2h_coarse_variant_topk: one row through the one-row kernel, 1..16 rows through the 16-row
// tile, K = 512 or 5120; var = design runs the production entry point itself.
int small_variant_launch(int var, const uint16_t* x, const float* xs, const uint8_t* packed, const uint16_t* S,
                         const uint16_t* ZS, int64_t N, int64_t K, int kc, float* cs, int32_t* ci, hipStream_t s);
int tile_variant_launch(int var, const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed,
                        const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int kc, float* cs, int32_t* ci,
                        hipStream_t s);

// The fused selection + exact rerank + top-k kernel (select_rerank.hip) and its limits.
bool select_rerank_supported(int64_t nblk, int kc, int R, int64_t N, int64_t K);
// G > 1 workgroups per row split the exact rerank: each publishes its scores to exw [M, R] and
// the last to arrive (counted in cnt [M], which must be 0 at launch and is left at G) ranks them.
// G = 1 needs neither. select_rerank_split gives the G the head uses for M rows. bmax (may be
// null): [M, nblk], each block's best score (cand_score's first slot per block), read in place of
// the strided first slots.
int select_rerank_split(int64_t M, int R);
int select_rerank_launch(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk, int kc, int R,
                         const uint16_t* x, const uint16_t* W, int64_t ldw, int64_t N, int64_t K, int k,
                         int32_t* sel, float* exact, int32_t* out_idx, float* out_val, hipStream_t s, int G = 1,
                         int32_t* cnt = nullptr, float* exw = nullptr, const float* bmax = nullptr);

// Entry points used by i2h_head (same checks and kernels as the exported calls). zero_cnt (may be
// null): M ints the launch sets to 0; coarse_launch takes it only with xs null. bmax (may be
// null): [M, nblk] floats that coarse_launch fills with each block's best score per row.
int xsum_launch(const uint16_t* x, int64_t M, int64_t K, float* xs, hipStream_t s, int32_t* zero_cnt = nullptr);
int coarse_launch(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed,
                  const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int kcand,
                  float* cand_score, int32_t* cand_idx, uint16_t* y, hipStream_t s,
                  int32_t* zero_cnt = nullptr, float* bmax = nullptr);
int select_launch(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk,
                  int kcand, int R, int32_t* sel, hipStream_t s);
int rerank_launch(const uint16_t* x, int64_t M, const uint16_t* W, int64_t ldw, int64_t N,
                  int64_t K, const int32_t* sel, int R, float* exact, hipStream_t s);
int rerank_finalize_launch(const uint16_t* x, int64_t M, const uint16_t* W, int64_t ldw, int64_t N,
                           int64_t K, const int32_t* sel, int R, int k, float* exact, int32_t* out_idx,
                           float* out_val, hipStream_t s);
int finalize_launch(const float* exact, const int32_t* sel, int64_t M, int R, int k,
                    int32_t* out_idx, float* out_val, hipStream_t s);

}  // namespace i2h
