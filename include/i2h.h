/*
 * i2h: the 2-bit speculative-draft LM head on MI355X (gfx950).
 *
 * The head computes logits = x[M, K] @ W[K, N] from a weight stored as int2 codes with an
 * asymmetric scale and zero point per (vocab row, group of 128 consecutive k), packed quarter-
 * split, then keeps the best KCAND columns of every 64-column vocab block, reranks the best R of
 * those exactly against the bf16 weight rows, and returns the argmax or the top-k of the
 * reranked tokens. Source: the page "radiance_drafthead.py" (2-bit MTP draft head with an exact
 * rerank); each entry point below names the part of it that defines the operation.
 *
 * Conventions for every call:
 *   - Pointers are device pointers allocated by the caller; the library allocates, frees and
 *     synchronises nothing and keeps no state between calls. Each call enqueues its kernels on
 *     `stream` (a hipStream_t; NULL is the legacy default stream) and returns at once.
 *   - bf16 values are passed as uint16_t bit patterns. Matrices are row-major; `ld*` arguments
 *     are row strides in elements.
 *   - Arguments are checked before anything is enqueued. On an error nothing is enqueued and a
 *     negative I2H_ERR_* code is returned. I2H_ERR_HIP means a HIP launch failed; the HIP error
 *     code is then available from i2h_last_hip_error() on the calling thread.
 *   - Shapes: G = 128 (quantisation group), BLOCK_N = 64 (candidate block), K a positive
 *     multiple of 512 (four quarters of whole groups) and at most 16384, NBLK = ceil(N / 64).
 *   - Alignment: x, W, packed, S and ZS must be 16-byte aligned, W's row stride a multiple of
 *     8 elements; fp32/int32 arrays 4-byte aligned, y 2-byte aligned.
 *   - Inputs must be finite (no NaN or inf in x or W).
 */
#ifndef I2H_H_
#define I2H_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define I2H_API __attribute__((visibility("default")))

#define I2H_OK 0
#define I2H_ERR_ARG (-1)        /* null pointer or invalid non-shape argument */
#define I2H_ERR_SHAPE (-2)      /* M, N or K outside the supported shapes */
#define I2H_ERR_ALIGN (-3)      /* pointer or stride alignment not met */
#define I2H_ERR_LIMIT (-4)      /* kcand, R or k outside their limits */
#define I2H_ERR_WORKSPACE (-5)  /* workspace missing or smaller than i2h_workspace_bytes() */
#define I2H_ERR_HIP (-6)        /* a HIP launch failed; see i2h_last_hip_error() */
#define I2H_ERR_UNIMPLEMENTED (-7) /* reserved: every operation declared here is implemented, and
                                      no call returns this code */
#define I2H_ERR_SCRATCH (-8)    /* i2h_head_noalloc: the call needs more than its device scratch */

#define I2H_GROUP 128
#define I2H_BLOCK_N 64
#define I2H_MAX_K 16384
#define I2H_MAX_KCAND 64
#define I2H_MAX_R 1024
#define I2H_MAX_NBLK 8192       /* N <= 524288 for the candidate selection */
#define I2H_NOALLOC_SCRATCH_BYTES (26 << 20) /* device scratch of i2h_head_noalloc, per GPU */

/* Element types of the drop-in logits row (i2h_logits). */
#define I2H_DTYPE_NONE 0        /* no embedding bias */
#define I2H_DTYPE_BF16 1
#define I2H_DTYPE_F16 2
#define I2H_DTYPE_F32 3

/* Library version (major * 10000 + minor * 100 + patch). */
I2H_API int i2h_version(void);

/* Text for a status code; never NULL. */
I2H_API const char* i2h_strerror(int status);

/* hipError_t of the last I2H_ERR_HIP returned on the calling thread (0 if none). */
I2H_API int i2h_last_hip_error(void);

/*
 * Sizes of the stored head for an [N, K] weight: packed bytes (N * K / 4) and the element count
 * of each of S and ZS (N * K / 128). Host only.
 */
I2H_API int i2h_sizes(int64_t N, int64_t K, int64_t* packed_bytes, int64_t* scale_elems);

/*
 * Quantise and pack a bf16 head (radiance_drafthead.py, _quantize_head_now: asymmetric min/max
 * at 2 bits per group; quarter-split packing; scale and zero premultiplied by the dequant bias).
 *   W       bf16 [N, K], row stride ldw (>= K, multiple of 8); row n is vocab token n.
 *   packed  u8 [N, K/4] (row stride K/4): byte j of a row holds the codes of k = j, Q+j, 2Q+j
 *           and 3Q+j (Q = K/4) in bits 0-1, 2-3, 4-5 and 6-7.
 *   S, ZS   bf16 [N, K/128] (row stride K/128): S = bf16(4 sc), ZS = bf16(4 sc + zp sc).
 * Per group of 128 consecutive k: sc = max((hi - lo) / 3, 1e-8), zp = clamp(round(-lo / sc),
 * 0, 3), q = clamp(round(w / sc + zp), 0, 3), all in IEEE fp32 with round-half-even and no
 * fused multiply-add, so the result is bit-exact against an eager fp32 evaluation.
 * W must be finite. Limits: N * K / 512 <= 2^30.
 */
I2H_API int i2h_pack(const uint16_t* W, int64_t ldw, int64_t N, int64_t K, uint8_t* packed,
                     uint16_t* S, uint16_t* ZS, void* stream);

/*
 * i2h_pack for an FP8 head (radiance_drafthead.py, _quantize_head_now with a compressed-tensors
 * per-channel FP8 lm_head): the weight is w[n, k] = decode(W8[n, k]) * wscale[n] in fp32, decode
 * being the e4m3 bit formula of _rerank_exact (sign bit 7; exponent field e = bits 3-6, mantissa
 * m = bits 0-2; m * 2^-9 when e = 0, else (1 + m/8) * 2^(e - 7)), and the rest is i2h_pack's
 * quantiser on those fp32 rows, bit-exact against eager fp32 ops.
 *   W8      uint8 e4m3 codes [N, K], row stride ldw bytes (>= K, multiple of 8), 8-byte aligned.
 *   wscale  fp32 [N] per-row scale.
 *   packed, S, ZS as in i2h_pack. Limits as in i2h_pack.
 */
I2H_API int i2h_pack_fp8(const uint8_t* W8, const float* wscale, int64_t ldw, int64_t N, int64_t K,
                         uint8_t* packed, uint16_t* S, uint16_t* ZS, void* stream);

/*
 * Per-group sums of x (radiance_drafthead.py, _apply_head_int2: the fp32 group sums the coarse
 * kernel uses for the zero point and the dequant bias).
 *   x   bf16 [M, K] (row stride K);  xs  fp32 [M, K/128]: xs[m, g] = sum of x[m, 128g .. 128g+127].
 * K a multiple of 128 up to I2H_MAX_K.
 */
I2H_API int i2h_xsum(const uint16_t* x, int64_t M, int64_t K, float* xs, void* stream);

/*
 * Coarse int2 logits and block candidates (radiance_drafthead.py, _draft_head_int2 and _emit):
 *   c[m, n] = sum over groups g of S[n,g] * sum_{k in g} x[m,k] (1 + v[n,k]/4) - xs[m,g] ZS[n,g]
 * with v the 2-bit code, accumulated in fp32. For every row m and block b of 64 columns, the
 * kcand best columns (score descending, lower column first on equal scores) are written, best
 * first, to slots b*kcand .. b*kcand+kcand-1 of
 *   cand_score fp32 [M, NBLK*kcand] and cand_idx int32 [M, NBLK*kcand] (token index n);
 * slots past a tail block's real columns get (-inf, -1).
 *   x bf16 [M, K]; xs fp32 [M, K/128] from i2h_xsum; packed/S/ZS from i2h_pack. xs may be NULL
 *   when i2h_coarse_sums_x(M, K) is true: the kernels then sum the groups of x themselves;
 *   otherwise a NULL xs is I2H_ERR_ARG. Results with xs given and with the kernels' own sums agree
 *   to fp32 summation order.
 *   y   optional bf16 [M, N] (row stride N): the coarse logits rounded to nearest-even; NULL to skip.
 * Limits: M >= 1 (any size; rows are processed in chunks), 1 <= kcand <= 64.
 */
I2H_API int i2h_coarse_topk(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed,
                            const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int kcand,
                            float* cand_score, int32_t* cand_idx, uint16_t* y, void* stream);

/*
 * Top-R selection over the block candidates (radiance_drafthead.py, _apply_head_int2: the
 * RERANK best block candidates of each row are the ones rescored exactly).
 *   cand_score/cand_idx as written by i2h_coarse_topk: [M, nblk*kcand], each block's kcand
 *   entries best first. sel int32 [M, R] receives, best first, the R best candidates by score
 *   descending then token index ascending; entries with index < 0 never count, and if a row
 *   has fewer than R valid candidates the remaining sel entries are -1.
 * Limits: 1 <= nblk <= 8192, 1 <= kcand <= 64, 1 <= R <= 1024.
 */
I2H_API int i2h_select(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk,
                       int kcand, int R, int32_t* sel, void* stream);

/*
 * Exact rerank (radiance_drafthead.py, _rerank_exact): exact[m, j] = sum_k x[m,k] W[sel[m,j], k]
 * over the bf16 weight row of the selected token, accumulated in fp32.
 *   x bf16 [M, K]; W bf16 [N, K] (row stride ldw); sel int32 [M, R]; exact fp32 [M, R].
 * A sel entry outside [0, N) gives -inf.
 */
I2H_API int i2h_rerank(const uint16_t* x, int64_t M, const uint16_t* W, int64_t ldw, int64_t N,
                       int64_t K, const int32_t* sel, int R, float* exact, void* stream);

/*
 * Final choice among the reranked tokens (radiance_drafthead.py, module docstring: the argmax
 * caller wins on the exact scores; _apply_head_int2: a top-k caller draws only from the
 * reranked tokens). out_idx int32 [M, k] and out_val fp32 [M, k] receive the k best (exact
 * score descending, token index ascending); k = 1 is the argmax. Entries with sel < 0 never
 * count; missing places get (-1, -inf). Limits: 1 <= R <= 1024, 1 <= k <= R.
 */
I2H_API int i2h_finalize(const float* exact, const int32_t* sel, int64_t M, int R, int k,
                         int32_t* out_idx, float* out_val, void* stream);

/* 1 if i2h_coarse_topk sums the groups of x itself for these sizes (xs may be NULL), else 0.
 * Rows go in chunks of 64; it is 1 when every chunk sums x itself: a one-row chunk when x fits in
 * the one-row kernel's LDS (K up to 16384), a chunk of 2 to 32 rows at a K the many-row kernel is
 * built for (512, 1024, 2048, 3072, 4096, 5120), and a chunk of 2 to 4 rows at another K when x
 * fits in LDS. Chunks of 33 to 64 rows take xs from i2h_xsum. */
I2H_API int i2h_coarse_sums_x(int64_t M, int64_t K);

/*
 * i2h_rerank followed by i2h_finalize, in one kernel when R <= 64 (one workgroup per row; the
 * exact scores also go to `exact` if it is not NULL). For R > 64 `exact` is required and the two
 * steps run as separate kernels. Limits as in those calls.
 */
I2H_API int i2h_rerank_topk(const uint16_t* x, int64_t M, const uint16_t* W, int64_t ldw, int64_t N,
                            int64_t K, const int32_t* sel, int R, int k, float* exact, int32_t* out_idx,
                            float* out_val, void* stream);

/*
 * i2h_rerank against an FP8 head (radiance_drafthead.py, _rerank_exact, FP8 branch):
 *   exact[m, j] = sum_k x[m,k] * fl32(decode(W8[sel[m,j], k]) * wscale[sel[m,j]])
 * accumulated in fp32 (decode as in i2h_pack_fp8). W8 uint8 [N, K] with row stride ldw bytes
 * (multiple of 8), 8-byte aligned; wscale fp32 [N]. A sel entry outside [0, N) gives -inf.
 */
I2H_API int i2h_rerank_fp8(const uint16_t* x, int64_t M, const uint8_t* W8, int64_t ldw, int64_t N, int64_t K,
                           const float* wscale, const int32_t* sel, int R, float* exact, void* stream);

/*
 * i2h_select, i2h_rerank and i2h_finalize in one kernel, one workgroup per row
 * (radiance_drafthead.py, _apply_head_int2 and _rerank_exact): the R best block candidates of each
 * row, their exact scores against the bf16 weight rows, and the k best of those. Same arguments,
 * layouts and results as the three calls (bit for bit): cand_score/cand_idx [M, nblk*kcand] with
 * nblk = ceil(N/64); x bf16 [M, K]; W bf16 rows with leading dimension ldw; sel int32 [M, R] and
 * exact fp32 [M, R] receive the selection and its exact scores when not NULL; out_idx/out_val
 * [M, k]. Limits: 1 <= kcand <= 8, 1 <= R <= 64, 1 <= k <= R, N <= 262144 (nblk <= 4096), K a
 * multiple of 512 up to I2H_MAX_K; outside them I2H_ERR_LIMIT (use the three calls).
 * Alignment: x and W 16 bytes, ldw a multiple of 8, the rest 4 bytes.
 */
I2H_API int i2h_select_rerank_topk(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk,
                                   int kcand, int R, const uint16_t* x, const uint16_t* W, int64_t ldw,
                                   int64_t N, int64_t K, int k, int32_t* sel, float* exact, int32_t* out_idx,
                                   float* out_val, void* stream);

/*
 * i2h_select_rerank_topk with the exact scores against an FP8 head (as i2h_rerank_fp8): same
 * arguments, with W8/wscale in place of W; bit-identical to i2h_select + i2h_rerank_fp8 +
 * i2h_finalize. Same limits.
 */
I2H_API int i2h_select_rerank_topk_fp8(const float* cand_score, const int32_t* cand_idx, int64_t M, int64_t nblk,
                                       int kcand, int R, const uint16_t* x, const uint8_t* W8, const float* wscale,
                                       int64_t ldw, int64_t N, int64_t K, int k, int32_t* sel, float* exact,
                                       int32_t* out_idx, float* out_val, void* stream);

/*
 * The int4 head (radiance_drafthead.py, _quantize_head_now with BITS = 4, the page's comparison
 * point, used with kcand = 1): codes 0..15 from the same asymmetric min/max quantiser per group of
 * 128 k (sc = max((hi - lo)/15, 1e-8), zp = clamp(round(-lo/sc), 0, 15), q = clamp(round(w/sc +
 * zp), 0, 15), IEEE fp32, bit-exact against eager fp32 ops);
 *   packed4 u8 [N, K/2]: byte j holds q[j] (bits 0-3) and q[K/2 + j] (bits 4-7);
 *   S, ZS   bf16 [N, K/128]: S = bf16(16 sc), ZS = bf16(16 sc + zp sc).
 * W bf16 [N, K], row stride ldw (>= K, multiple of 4), 8-byte aligned; packed4 16-byte aligned.
 * Limits: K a multiple of 256 up to I2H_MAX_K (the exact rerank after it needs a multiple of 512).
 */
I2H_API int i2h_pack4(const uint16_t* W, int64_t ldw, int64_t N, int64_t K, uint8_t* packed4, uint16_t* S,
                      uint16_t* ZS, void* stream);

/*
 * Coarse logits and block candidates of the int4 head (the fold of the page's bit-pattern
 * dequant at bias 16): c[m, n] = sum over groups g of S[n,g] * sum_{k in g} x[m,k] (1 + v/16)
 * - xs[m,g] ZS[n,g], accumulated in fp32; the block top-kcand, y and the layouts as in
 * i2h_coarse_topk. xs from i2h_xsum is required. Limits: M >= 1, 1 <= kcand <= 64, K a
 * multiple of 256. Not tuned for bandwidth (x is read from L2 per block).
 */
I2H_API int i2h_coarse4_topk(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed4,
                             const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int kcand,
                             float* cand_score, int32_t* cand_idx, uint16_t* y, void* stream);

/*
 * Token-level selection over the coarse row (the alternative to block candidates that the page
 * measures; radiance_drafthead.py, _emit docstring and the module docstring's note on
 * selection): sel [M, R] int32 = for each row of y [M, N] bf16 (row-major, row stride N), the
 * indices of its R largest entries, value descending, lower index first on ties, -0.0 equal to
 * +0.0; -1 in slots past N. Feed sel to i2h_rerank or i2h_rerank_topk. y finite. With a
 * workspace of i2h_select_tokens_workspace_bytes() (caller-owned, 8-byte aligned, contents
 * undefined afterwards) a long row is split over workgroups of 16384 entries whose winners are
 * merged; with workspace NULL (or a size of 0 bytes returned) one workgroup takes each row. Both
 * give the same sel. Limits: 1 <= M <= 65535, 1 <= N <= 2^31 - 1, 1 <= R <= I2H_MAX_R; y 2-byte
 * and sel 4-byte aligned; a workspace smaller than needed is I2H_ERR_WORKSPACE.
 */
I2H_API int64_t i2h_select_tokens_workspace_bytes(int64_t M, int64_t N, int R);
I2H_API int i2h_select_tokens(const uint16_t* y, int64_t M, int64_t N, int R, int32_t* sel, void* workspace,
                              int64_t workspace_bytes, void* stream);

/*
 * The design alternatives the head is measured against (radiance_drafthead.py, module
 * docstring: group 128 against 64, quarter-split against contiguous-4 bytes, the scale applied to
 * the accumulator against a dequantised weight tile). Measurement variants, not the per-call path.
 */
#define I2H_LAYOUT_QUARTER 0 /* byte j of a row holds k = j, K/4 + j, K/2 + j, 3K/4 + j */
#define I2H_LAYOUT_CONTIG 1  /* byte j of a row holds k = 4j .. 4j + 3 (bits 0-1 .. 6-7) */
#define I2H_SCALE_ACC 0      /* per group S * sum x (1 + v/4) - xs * ZS on the fp32 accumulator */
#define I2H_SCALE_TILE 1     /* each weight bf16(fl32(S (1 + v/4)) - ZS), then the bf16 dot */

/*
 * i2h_pack at group `group` (64 or 128) in layout I2H_LAYOUT_*: the same quantiser and
 * premultiplied scales; packed [N, K/4], S and ZS [N, K/group]. Bit-exact. Limits: K a multiple
 * of 4 * group up to I2H_MAX_K, ldw >= K, N * K / (4 * group) < 2^31.
 */
I2H_API int i2h_pack_variant(const uint16_t* W, int64_t ldw, int64_t N, int64_t K, int group, int layout,
                             uint8_t* packed, uint16_t* S, uint16_t* ZS, void* stream);

/* i2h_xsum at group `group` (64 or 128): xs [M, K/group] fp32; K a multiple of group. */
I2H_API int i2h_xsum_group(const uint16_t* x, int64_t M, int64_t K, int group, float* xs, void* stream);

/*
 * Coarse logits and block candidates of a head packed by i2h_pack_variant with the same group
 * and layout, scaled per I2H_SCALE_*: c[m, n] = sum_g S * sum_{k in g} x (1 + v/4) - xs ZS
 * (accumulator) or sum_k x[m, k] w~[n, k] with the rounded tile w~ (xs unused); fp32
 * accumulation; the block top-kcand as in i2h_coarse_topk. Each alternative runs through the
 * production kernels (one row: the one-row kernel; 2..16 rows: the 16-row tile) with one property
 * changed: (group, layout, scaling) is one of (128, QUARTER, ACC) (the design itself, the
 * i2h_coarse_topk path), (64, QUARTER, ACC), (128, CONTIG, ACC) or (128, QUARTER, TILE); any
 * other combination is I2H_ERR_ARG. xs (accumulator): the sums from i2h_xsum_group, or NULL for
 * sums taken in the kernel. Limits: 1 <= M <= 16, K = 512 or 5120 (else I2H_ERR_SHAPE),
 * 1 <= kcand <= 64, N <= 2^30; x, packed, S, ZS 16-byte aligned.
 */
I2H_API int i2h_coarse_variant_topk(const uint16_t* x, const float* xs, int64_t M, const uint8_t* packed,
                                    const uint16_t* S, const uint16_t* ZS, int64_t N, int64_t K, int group,
                                    int layout, int scaling, int kcand, float* cand_score, int32_t* cand_idx,
                                    void* stream);

/* Workspace bytes i2h_head needs for these sizes (negative I2H_ERR_* on invalid sizes). */
I2H_API int64_t i2h_workspace_bytes(int64_t M, int64_t N, int64_t K, int kcand, int R);

/*
 * One call of the head: i2h_xsum (skipped when i2h_coarse_sums_x), i2h_coarse_topk, then
 * i2h_select_rerank_topk within its limits, else i2h_select and i2h_rerank_topk, in stream
 * order, with the intermediates in `workspace` (at least i2h_workspace_bytes(), 256-byte
 * aligned, caller-owned, contents undefined on entry and afterwards). Arguments as in those
 * calls; y may be NULL. The limits of every step apply. Up to 16 rows the fused tail runs
 * several workgroups per row, which count their arrivals in the workspace; the call's first
 * kernel zeroes those counters, so results equal i2h_select_rerank_topk's bit for bit and two
 * calls must not share a workspace while both are in flight (as for every intermediate).
 */
I2H_API int i2h_head(const uint16_t* x, int64_t M, const uint8_t* packed, const uint16_t* S,
                     const uint16_t* ZS, const uint16_t* W, int64_t ldw, int64_t N, int64_t K,
                     int kcand, int R, int k, int32_t* out_idx, float* out_val, uint16_t* y,
                     void* workspace, int64_t ws_bytes, void* stream);

/*
 * i2h_head for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): the same arguments without the workspace,
 * the same kernels and results bit for bit. The intermediates live in a device array of
 * I2H_NOALLOC_SCRATCH_BYTES (26 MiB) that the library holds on each GPU it runs on until the
 * process ends; its address is looked up on the first call on a device (the GPU of `stream`),
 * so make that first call outside graph capture. The call allocates nothing: no hipMalloc,
 * hipFree or allocating library routine. A call whose i2h_workspace_bytes() exceeds the scratch
 * returns I2H_ERR_SCRATCH before anything is enqueued (the 124160-row slice at up to 128 rows, or
 * the 248320-row vocabulary at up to 96 rows, fit at kcand = 8, R = 32). Every call on one GPU
 * shares that GPU's scratch, and the scratch keeps the last call's contents (the call's first
 * kernel zeroes the tail's arrival counters, so nothing needs clearing): calls that overlap on one
 * GPU, on different streams or threads, race and must be ordered by the caller.
 */
I2H_API int i2h_head_noalloc(const uint16_t* x, int64_t M, const uint8_t* packed, const uint16_t* S,
                             const uint16_t* ZS, const uint16_t* W, int64_t ldw, int64_t N, int64_t K,
                             int kcand, int R, int k, int32_t* out_idx, float* out_val, uint16_t* y,
                             void* stream);

/*
 * The drop-in logits row (radiance_drafthead.py, _apply_head_int2, after the exact rerank):
 *   row     = topk_only ? -inf : y[m, :]            (y: the coarse bf16 row from i2h_coarse_topk)
 *   row[sel[m, j]] = bf16(exact[m, j])               for every sel[m, j] >= 0
 *   out[m, :] = cast_out(row + bias)                 with torch's type promotion: a bf16 bias
 *             rounds the fp32 sum back to bf16; an fp16 or fp32 bias gives the fp32 sum; no bias
 *             keeps the bf16 row; the cast to out_dtype rounds to nearest-even.
 *   y       bf16 [M, N] (row stride N), 16-byte aligned; may be NULL when topk_only.
 *   sel     int32 [M, R], exact fp32 [M, R] (from i2h_select_rerank_topk or i2h_select +
 *           i2h_rerank); each entry is -1 (no token) or a token in [0, N), and a row's tokens
 *           are distinct (as those calls give them). Any other entry is outside the contract
 *           (the page's scatter would reject it); the kernel ignores it, so nothing outside the
 *           row is ever written.
 *   bias    [N] of bias_dtype (I2H_DTYPE_NONE with bias NULL for none), naturally aligned.
 *   out     [M, N] of out_dtype (BF16 / F16: uint16 bits; F32), 16-byte aligned. out may be y
 *           itself when out_dtype is I2H_DTYPE_BF16 (each entry is read before it is written,
 *           and the write-back of a token follows the row pass over it).
 * One kernel launch on `stream`. Limits: 1 <= M <= 65535, 1 <= R <= 1024.
 */
I2H_API int i2h_logits(const uint16_t* y, int64_t M, int64_t N, const int32_t* sel, const float* exact, int R,
                       int topk_only, const void* bias, int bias_dtype, void* out, int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* I2H_H_ */
