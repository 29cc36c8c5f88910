"""Oracle for the int2 draft LM head. TEST INFRASTRUCTURE ONLY.

A plain, slow, CPU (numpy) statement of what the head computes, written from the page
"radiance_drafthead.py" (the 2-bit MTP draft head with an exact rerank). Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it. The HIP library never
does, and the two share no code: no kernels, headers, helpers, tables or constants.

Precision. The page quantises with eager PyTorch fp32 ops, one kernel per op, so the oracle's
quantiser and scale/zero premultiply run in IEEE fp32, one operation at a time, rounding to
nearest-even, with no fused multiply-add. Everything else is fp64. The dequantised weight
S*(1 + v/4) - ZS is exact in fp64 (and in fp32), so the coarse logits below are the exact
dot products of x with the stored int2 head, up to fp64 rounding of the sums.

Order of the steps (names follow the page):
  quantize      per (row n, group of G consecutive k): min/max, sc, zp, q       (_quantize_head_now)
  pack          quarter split: byte j holds k = j, Q+j, 2Q+j, 3Q+j, Q = K/4     (_quantize_head_now)
  scales        S = bf16(4 sc), ZS = bf16(4 sc + zp sc)                          (_quantize_head_now)
  group_sums    xs[m, g] = sum of x over group g                                  (_apply_head_int2)
  coarse        c[m, n] = sum_k x[m, k] * (S (1 + v/4) - ZS)                      (_draft_head_int2)
  block_emit    per 64-column block, its KCAND best columns, best first           (_emit)
  select        per row, the RERANK best candidates                               (_apply_head_int2)
  rerank        exact dot of x with the selected bf16 weight rows                 (_rerank_exact)
  finalize      argmax, or the top-k of the reranked tokens                       (module docstring;
                                                                                   _apply_head_int2)
  logits_row    the drop-in row: coarse bf16 row (or -inf), exact scores written
                back, embedding bias, head dtype                                  (_apply_head_int2)
Readings of points the page leaves open (each is also listed with the design notes):
  * ties in the block emit go to the lower column; selection and top-k order by score
    descending, then token index ascending; the final argmax takes the lower token index;
  * argmax is taken over the R exact scores;
  * a block with fewer than KCAND real columns (vocab tail) pads with (-inf, -1), and such
    entries are never selected;
  * K must be a multiple of 4 * G, so that every quarter holds whole groups;
  * the exact scores are written back into the row for an argmax caller as well as for a top-k
    caller (whose row is -inf elsewhere).
"""
from __future__ import annotations

import concurrent.futures as _cf
import os

import numpy as np

GROUP = 128     # quantisation group along k
BLOCK_N = 64    # vocab columns per candidate block
_CHUNK = 4096   # rows of W handled at once by the chunked steps (memory bound only)


# ----------------------------------------------------------------------------------------------
# bf16 <-> fp32, written from the IEEE-754 binary32 layout (bf16 is its upper 16 bits)
# ----------------------------------------------------------------------------------------------
def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16, nearest-even (the rounding of torch's .to(torch.bfloat16))."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    if nan.any():
        r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040)), r)
    return r


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _map_chunks(fn, n_rows: int, chunk: int = _CHUNK):
    """Apply fn(a, b) to row ranges [a, b); independent chunks may run on several threads."""
    ranges = [(a, min(n_rows, a + chunk)) for a in range(0, n_rows, chunk)]
    if len(ranges) <= 1:
        return [fn(a, b) for a, b in ranges]
    with _cf.ThreadPoolExecutor(_threads()) as ex:
        return list(ex.map(lambda r: fn(*r), ranges))


def check_shape(K: int, G: int = GROUP) -> None:
    """K must split into four quarters of whole groups (see the readings in the header)."""
    if K <= 0 or K % (4 * G) != 0:
        raise ValueError(f"K={K} is not a positive multiple of 4*G={4 * G}")


# ----------------------------------------------------------------------------------------------
# a1/a2: quantise, pack, premultiplied scales
# radiance_drafthead.py, _quantize_head_now: asymmetric min/max quantisation at 2 bits per group
# of 128 consecutive k of one weight row, quarter-split packing, and the scale and zero arrays
# premultiplied by the bias of the bit-pattern dequant (4 for 2 bits).
# ----------------------------------------------------------------------------------------------
def quantize(W_bits: np.ndarray, G: int = GROUP):
    """Quantise bf16 rows W [N, K] (given as uint16 bits) per group of G consecutive k.

    Returns q uint8 [N, K] in {0..3}, sc fp32 [N, K/G], zp fp32 [N, K/G]:
      lo, hi = min, max of the group (exact);
      sc = max((hi - lo) / 3, 1e-8)           fp32 divide, then clamp
      zp = clamp(round(-lo / sc), 0, 3)       round half to even
      q  = clamp(round(w / sc + zp), 0, 3)    fp32 divide, fp32 add, round half to even
    """
    return _quantize_rows(lambda a, b: bf16_to_f32(W_bits[a:b]), W_bits.shape, G)


def _quantize_rows(rows, shape, G: int = GROUP, levels: int = 3):
    """The quantiser of quantize() over fp32 rows [a, b) that rows(a, b) returns, with codes
    0..levels (3 for 2 bits, 15 for 4 bits)."""
    N, K = shape
    if K % G:
        raise ValueError("K must be a multiple of G")
    q = np.empty((N, K), dtype=np.uint8)
    sc_all = np.empty((N, K // G), dtype=np.float32)
    zp_all = np.empty((N, K // G), dtype=np.float32)
    three = np.float32(levels)
    floor = np.float32(1e-8)

    def run(a: int, b: int) -> None:
        w = rows(a, b).astype(np.float32).reshape(b - a, K // G, G)
        lo = w.min(axis=2)
        hi = w.max(axis=2)
        sc = (hi - lo) / three
        sc = np.maximum(sc, floor)
        zp = np.clip(np.rint(-lo / sc), np.float32(0), three)
        t = w / sc[:, :, None]
        t = t + zp[:, :, None]
        qq = np.clip(np.rint(t), np.float32(0), three)
        q[a:b] = qq.reshape(b - a, K).astype(np.uint8)
        sc_all[a:b] = sc
        zp_all[a:b] = zp

    _map_chunks(run, N)
    return q, sc_all, zp_all


def premultiplied_scales(sc: np.ndarray, zp: np.ndarray):
    """S = bf16(4 sc), ZS = bf16(4 sc + zp sc), each product and the sum rounded in fp32 first.

    The 4 is the bias of the 2-bit bit-pattern dequant (the bf16 weight read is 1 + v/4), which
    the page folds into the stored scales.
    """
    four = np.float32(4.0)
    s4 = (four * sc).astype(np.float32)
    zsc = (zp * sc).astype(np.float32)
    zs = (s4 + zsc).astype(np.float32)
    return f32_to_bf16(s4), f32_to_bf16(zs)


def pack_quarter_split(q: np.ndarray) -> np.ndarray:
    """uint8 [N, K/4]: byte j = q[j] | q[Q+j] << 2 | q[2Q+j] << 4 | q[3Q+j] << 6, Q = K/4."""
    N, K = q.shape
    Q = K // 4
    q = q.astype(np.uint8)
    return (q[:, 0:Q] | (q[:, Q:2 * Q] << 2) | (q[:, 2 * Q:3 * Q] << 4)
            | (q[:, 3 * Q:4 * Q] << 6)).astype(np.uint8)


def unpack_quarter_split(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_quarter_split: v uint8 [N, K] with v[n, t*Q + j] = (byte j >> 2t) & 3."""
    N, Q = packed.shape
    v = np.empty((N, 4 * Q), dtype=np.uint8)
    for t in range(4):
        v[:, t * Q:(t + 1) * Q] = (packed >> np.uint8(2 * t)) & np.uint8(3)
    return v


def pack(W_bits: np.ndarray, G: int = GROUP):
    """The stored head: (packed uint8 [N, K/4], S bf16 bits [N, K/G], ZS bf16 bits [N, K/G])."""
    check_shape(W_bits.shape[1], G)
    q, sc, zp = quantize(W_bits, G)
    S, ZS = premultiplied_scales(sc, zp)
    return pack_quarter_split(q), S, ZS


# ----------------------------------------------------------------------------------------------
# a3: per-group sums of x
# radiance_drafthead.py, _apply_head_int2: the fp32 sum of x over each group of 128 k, the
# term that carries both the zero point and the 1.0 bias of the dequant.
# ----------------------------------------------------------------------------------------------
def group_sums(x_bits: np.ndarray, G: int = GROUP) -> np.ndarray:
    """xs fp64 [M, K/G] = sum over each group of G consecutive k of x."""
    M, K = x_bits.shape
    return bf16_to_f32(x_bits).astype(np.float64).reshape(M, K // G, G).sum(axis=2)


# ----------------------------------------------------------------------------------------------
# a4/a6: coarse logits
# radiance_drafthead.py, module docstring (bit-pattern dequant; bias fold) and _draft_head_int2:
# each group contributes S * sum_k x (1 + v/4) - ZS * sum_k x, which is the same as the dot of
# x with the per-weight dequantised row S (1 + v/4) - ZS. The oracle evaluates that form.
# ----------------------------------------------------------------------------------------------
def dequantize(packed: np.ndarray, S_bits: np.ndarray, ZS_bits: np.ndarray,
               G: int = GROUP) -> np.ndarray:
    """fp64 [N, K]: w'[n, k] = S[n, k/G] * (1 + v[n, k] / 4) - ZS[n, k/G] (exact)."""
    v = unpack_quarter_split(packed).astype(np.float64)
    N, K = v.shape
    s = np.repeat(bf16_to_f32(S_bits).astype(np.float64), G, axis=1)
    zs = np.repeat(bf16_to_f32(ZS_bits).astype(np.float64), G, axis=1)
    return s * (1.0 + v / 4.0) - zs


def coarse_logits(x_bits: np.ndarray, packed: np.ndarray, S_bits: np.ndarray,
                  ZS_bits: np.ndarray, G: int = GROUP) -> np.ndarray:
    """c fp64 [M, N] = x @ dequantize(...)^T."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    N = packed.shape[0]
    c = np.empty((x.shape[0], N), dtype=np.float64)

    def run(a: int, b: int) -> None:
        c[:, a:b] = x @ dequantize(packed[a:b], S_bits[a:b], ZS_bits[a:b], G).T

    _map_chunks(run, N)
    return c


# ----------------------------------------------------------------------------------------------
# a5: block top-KCAND
# radiance_drafthead.py, _emit: KCAND rounds of (max, argmax, mask) over the block's 64
# fp32 accumulator columns; a column past N is -inf. Reading: ties go to the lower column.
# ----------------------------------------------------------------------------------------------
def block_emit(c: np.ndarray, kcand: int, block_n: int = BLOCK_N):
    """(score fp64 [M, NBLK*kcand], idx int32 [M, NBLK*kcand]); block b owns slots b*kcand...

    Within a block the entries are best first (score descending, column ascending on ties).
    Slots beyond the block's real columns hold (-inf, -1).
    """
    M, N = c.shape
    nblk = (N + block_n - 1) // block_n
    padded = np.full((M, nblk * block_n), -np.inf)
    padded[:, :N] = c
    padded = padded.reshape(M, nblk, block_n)
    # a stable sort of -score keeps equal scores in column order, so ties go to the lower column
    order = np.argsort(-padded, axis=2, kind="stable")[:, :, :kcand]
    score = np.take_along_axis(padded, order, axis=2)
    col = (np.arange(nblk)[None, :, None] * block_n + order).astype(np.int64)
    real = col < N
    score = np.where(real, score, -np.inf)
    idx = np.where(real, col, -1).astype(np.int32)
    return score.reshape(M, nblk * kcand), idx.reshape(M, nblk * kcand)


# ----------------------------------------------------------------------------------------------
# a7: top-R selection
# radiance_drafthead.py, _apply_head_int2: the R best of the row's block candidates, by score.
# Reading: order by score descending, then token index ascending; (-inf, -1) entries never count.
# ----------------------------------------------------------------------------------------------
def _rank_order(score: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Positions of one row's valid entries, best first (score desc, index asc)."""
    pos = np.nonzero(idx >= 0)[0]
    o = np.lexsort((idx[pos], -score[pos]))
    return pos[o]


def select_top_r(score: np.ndarray, idx: np.ndarray, R: int) -> np.ndarray:
    """sel int32 [M, R], best first; -1 where a row has fewer than R valid candidates."""
    M = score.shape[0]
    sel = np.full((M, R), -1, dtype=np.int32)
    for m in range(M):
        o = _rank_order(score[m], idx[m])[:R]
        sel[m, :len(o)] = idx[m][o]
    return sel


# ----------------------------------------------------------------------------------------------
# a8: exact rerank
# radiance_drafthead.py, _rerank_exact: the exact logit of each selected token, the dot of x
# with that token's bf16 weight row. Products of two bf16 values are exact in fp64.
# ----------------------------------------------------------------------------------------------
def rerank_exact(x_bits: np.ndarray, W_bits: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """e fp64 [M, R]; -inf where sel is -1."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    M, R = sel.shape
    e = np.full((M, R), -np.inf)
    for m in range(M):
        ok = sel[m] >= 0
        rows = bf16_to_f32(W_bits[sel[m][ok]]).astype(np.float64)
        e[m, ok] = rows @ x[m]
    return e


# ----------------------------------------------------------------------------------------------
# a9: finalize
# radiance_drafthead.py, module docstring (reranked scores are what the argmax caller wins on)
# and _apply_head_int2 (a top-k caller may draw only from the reranked tokens).
# ----------------------------------------------------------------------------------------------
def finalize(e: np.ndarray, sel: np.ndarray, k: int):
    """(idx int32 [M, k], val fp64 [M, k]): the k best reranked tokens, best first.

    Order: exact score descending, then token index ascending. k = 1 is the argmax.
    """
    M = e.shape[0]
    out_i = np.full((M, k), -1, dtype=np.int32)
    out_v = np.full((M, k), -np.inf)
    for m in range(M):
        o = _rank_order(e[m], sel[m])[:k]
        out_i[m, :len(o)] = sel[m][o]
        out_v[m, :len(o)] = e[m][o]
    return out_i, out_v


def head(x_bits: np.ndarray, W_bits: np.ndarray, packed: np.ndarray, S_bits: np.ndarray,
         ZS_bits: np.ndarray, kcand: int = 8, R: int = 32, k: int = 1, G: int = GROUP,
         block_n: int = BLOCK_N, coarse: np.ndarray | None = None) -> dict:
    """One call of the head for the rows of x; every intermediate is returned.

    `coarse` may carry precomputed oracle coarse logits for these rows (the same values
    coarse_logits would return), so several calls can share one pass over W.
    """
    c = coarse_logits(x_bits, packed, S_bits, ZS_bits, G) if coarse is None else coarse
    cs, ci = block_emit(c, kcand, block_n)
    sel = select_top_r(cs, ci, R)
    e = rerank_exact(x_bits, W_bits, sel)
    oi, ov = finalize(e, sel, k)
    return dict(coarse=c, cand_score=cs, cand_idx=ci, sel=sel, exact=e, idx=oi, val=ov)


# ----------------------------------------------------------------------------------------------
# The dense bf16 head the int2 head stands in for (the stock head the page replaces).
# ----------------------------------------------------------------------------------------------
def exact_logits(x_bits: np.ndarray, W_bits: np.ndarray) -> np.ndarray:
    """fp64 [M, N] = x @ W^T over the bf16 rows."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    N = W_bits.shape[0]
    out = np.empty((x.shape[0], N))

    def run(a: int, b: int) -> None:
        out[:, a:b] = x @ bf16_to_f32(W_bits[a:b]).astype(np.float64).T

    _map_chunks(run, N)
    return out


def storage_bytes(N: int, K: int, G: int = GROUP) -> dict:
    """Bytes of the stored head: packed int2, S and ZS (bf16 each), and the bf16 weight."""
    packed = N * K // 4
    scales = N * (K // G) * 2
    return dict(packed=packed, S=scales, ZS=scales, int2_total=packed + 2 * scales,
                bf16_weight=N * K * 2)


# ----------------------------------------------------------------------------------------------
# NEXT f1: the drop-in logits row
# radiance_drafthead.py, _apply_head_int2: the coarse logits are a bf16 row Y [M, N]. A top-k
# caller's row is first set to -inf everywhere; the R reranked tokens' entries are then
# overwritten by their exact scores rounded to bf16 (for both callers: the reading that the
# write-back belongs to every caller with an exact weight). The embedding bias is added next, with
# torch's type promotion (bf16 + bf16 stays bf16, bf16 + fp16 or fp32 becomes fp32), and the row
# is cast to the head dtype.
# ----------------------------------------------------------------------------------------------
LOGIT_DTYPES = ("bf16", "fp16", "fp32")


def logits_row(y_bits: np.ndarray, sel: np.ndarray, exact: np.ndarray, topk_only: bool,
               bias: np.ndarray | None = None, bias_dtype: str | None = None,
               out_dtype: str = "bf16") -> np.ndarray:
    """The drop-in output [M, N]: uint16 bits for bf16/fp16 heads, float32 for fp32 heads.

    y_bits bf16 bits [M, N]; sel int32 [M, R] (distinct tokens per row, -1 = none); exact
    float32 [M, R]; bias [N] given as uint16 bits (bf16), float16 or float32 per bias_dtype.
    A token outside [0, N) other than -1 raises ValueError: the page writes the exact scores
    back with a scatter over the row, which rejects an index past the row's end.
    """
    assert out_dtype in LOGIT_DTYPES and (bias is None) == (bias_dtype is None)
    M, N = y_bits.shape
    sel = np.asarray(sel)
    if ((sel < -1) | (sel >= N)).any():
        raise ValueError("sel holds a token outside [0, N) that is not -1 (none)")
    # the row before the bias: coarse bf16 values, or -inf for a top-k caller
    y = np.full((M, N), -np.inf, dtype=np.float32) if topk_only else bf16_to_f32(y_bits)
    e = bf16_to_f32(f32_to_bf16(np.asarray(exact, dtype=np.float32)))  # ex.to(bfloat16)
    for m in range(M):
        for j in range(sel.shape[1]):
            if sel[m, j] >= 0:  # -1: no token in this slot
                y[m, sel[m, j]] = e[m, j]
    # the bias, then the row's dtype after promotion
    if bias is None:
        r, rtype = y, "bf16"
    elif bias_dtype == "bf16":
        r, rtype = bf16_to_f32(f32_to_bf16((y + bf16_to_f32(bias)[None, :]).astype(np.float32))), "bf16"
    elif bias_dtype == "fp16":
        r, rtype = (y + np.asarray(bias, dtype=np.float16).astype(np.float32)[None, :]).astype(np.float32), "fp32"
    else:
        assert bias_dtype == "fp32"
        r, rtype = (y + np.asarray(bias, dtype=np.float32)[None, :]).astype(np.float32), "fp32"
    # the cast to the head dtype (a no-op when the dtypes agree)
    if out_dtype == "fp32":
        return r.astype(np.float32)
    if out_dtype == "bf16":
        return f32_to_bf16(r)  # exact when the row already holds bf16 values
    return r.astype(np.float16).view(np.uint16)



# ----------------------------------------------------------------------------------------------
# NEXT f4: an FP8 e4m3 head with a per-row fp32 scale as the weight source
# radiance_drafthead.py, _rerank_exact (FP8 branch): a byte b decodes by bit arithmetic as
# sign (bit 7), exponent field e = bits 3-6, mantissa m = bits 0-2: m * 2^-9 when e = 0, else
# (1 + m/8) * 2^(e - 7); the weight is that value times the row's fp32 scale, an fp32 product.
# _quantize_head_now: the int2 head of such a weight quantises the same fp32 rows.
# ----------------------------------------------------------------------------------------------
def fp8_e4m3_decode(b: np.ndarray) -> np.ndarray:
    """fp64 values of e4m3 bytes by the page's bit formula (exact; 0x7F decodes to 480)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    e = (b >> 3) & 15
    m = (b & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    return np.where((b & 128) != 0, -mag, mag)


def fp8_rows_f32(W8: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp32 [rows, K]: decode(W8) * scale[row], one fp32 multiply (the decode is exact in fp32)."""
    return (fp8_e4m3_decode(W8).astype(np.float32) * np.asarray(scale, np.float32)[:, None]).astype(np.float32)


def quantize_fp8(W8: np.ndarray, scale: np.ndarray, G: int = GROUP):
    """quantize() over the fp32 rows of an FP8 head (W8 uint8 [N, K], scale fp32 [N])."""
    return _quantize_rows(lambda a, b: fp8_rows_f32(W8[a:b], scale[a:b]), W8.shape, G)


def pack_fp8(W8: np.ndarray, scale: np.ndarray, G: int = GROUP):
    """The stored int2 head of an FP8 head: (packed uint8 [N, K/4], S bits, ZS bits)."""
    check_shape(W8.shape[1], G)
    q, sc, zp = quantize_fp8(W8, scale, G)
    S, ZS = premultiplied_scales(sc, zp)
    return pack_quarter_split(q), S, ZS


def rerank_exact_fp8(x_bits: np.ndarray, W8: np.ndarray, scale: np.ndarray, sel: np.ndarray) -> np.ndarray:
    """e fp64 [M, R]: x against the fp32 rows of the FP8 head (products exact in fp64); -inf
    where sel is -1."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    M, R = sel.shape
    e = np.full((M, R), -np.inf)
    for m in range(M):
        ok = sel[m] >= 0
        t = sel[m][ok]
        e[m, ok] = fp8_rows_f32(W8[t], scale[t]).astype(np.float64) @ x[m]
    return e



# ----------------------------------------------------------------------------------------------
# NEXT f3: the int4 head (the page's comparison point, used at KCAND = 1)
# radiance_drafthead.py, _quantize_head_now (BITS = 4 branch) and the module docstring: the same
# asymmetric min/max quantiser with codes 0..15; byte j of a packed row holds the codes of k = j
# (bits 0-3) and K/2 + j (bits 4-7); the bit-pattern dequant reads 1 + v/16, so S = bf16(16 sc)
# and ZS = bf16(16 sc + zp sc). The page prints no 4-bit kernel: its coarse logits follow from the
# same fold, c = sum_g S P - xs ZS with P = sum_k x (1 + v/16).
# Reading: K must be a multiple of 2 * G (each half of a row holds whole groups), the page's own
# check for this layout.
# ----------------------------------------------------------------------------------------------
def check_shape4(K: int, G: int = GROUP) -> None:
    if K <= 0 or K % (2 * G):
        raise ValueError(f"K = {K} must be a positive multiple of {2 * G} for the int4 head")


def quantize4(W_bits: np.ndarray, G: int = GROUP):
    """quantize() with codes 0..15: q uint8 [N, K], sc, zp fp32 [N, K/G]."""
    return _quantize_rows(lambda a, b: bf16_to_f32(W_bits[a:b]), W_bits.shape, G, levels=15)


def premultiplied_scales4(sc: np.ndarray, zp: np.ndarray):
    """S = bf16(16 sc), ZS = bf16(16 sc + zp sc) (fp32 products and sum, then bf16)."""
    sixteen = np.float32(16.0)
    s16 = (sixteen * sc).astype(np.float32)
    zs = (s16 + (zp * sc).astype(np.float32)).astype(np.float32)
    return f32_to_bf16(s16), f32_to_bf16(zs)


def pack_half_split(q: np.ndarray) -> np.ndarray:
    """uint8 [N, K/2]: byte j = q[j] | q[K/2 + j] << 4."""
    N, K = q.shape
    H = K // 2
    q = q.astype(np.uint8)
    return (q[:, :H] | (q[:, H:] << 4)).astype(np.uint8)


def unpack_half_split(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_half_split: v uint8 [N, K]."""
    return np.concatenate([packed & np.uint8(15), packed >> np.uint8(4)], axis=1).astype(np.uint8)


def pack4(W_bits: np.ndarray, G: int = GROUP):
    """The stored int4 head: (packed uint8 [N, K/2], S bits [N, K/G], ZS bits [N, K/G])."""
    check_shape4(W_bits.shape[1], G)
    q, sc, zp = quantize4(W_bits, G)
    S, ZS = premultiplied_scales4(sc, zp)
    return pack_half_split(q), S, ZS


def dequantize4(packed: np.ndarray, S_bits: np.ndarray, ZS_bits: np.ndarray, G: int = GROUP) -> np.ndarray:
    """fp64 [N, K]: S (1 + v/16) - ZS per group (exact)."""
    v = unpack_half_split(packed).astype(np.float64)
    s = np.repeat(bf16_to_f32(S_bits).astype(np.float64), G, axis=1)
    zs = np.repeat(bf16_to_f32(ZS_bits).astype(np.float64), G, axis=1)
    return s * (1.0 + v / 16.0) - zs


def coarse_logits4(x_bits: np.ndarray, packed: np.ndarray, S_bits: np.ndarray, ZS_bits: np.ndarray,
                   G: int = GROUP) -> np.ndarray:
    """c fp64 [M, N] = x @ dequantize4(...)^T."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    N = packed.shape[0]
    c = np.empty((x.shape[0], N), dtype=np.float64)

    def run(a: int, b: int) -> None:
        c[:, a:b] = x @ dequantize4(packed[a:b], S_bits[a:b], ZS_bits[a:b], G).T

    _map_chunks(run, N)
    return c


def head4(x_bits: np.ndarray, W_bits: np.ndarray, packed: np.ndarray, S_bits: np.ndarray,
          ZS_bits: np.ndarray, kcand: int = 1, R: int = 32, k: int = 1, G: int = GROUP,
          block_n: int = BLOCK_N) -> dict:
    """One call of the int4 head: coarse over the int4 copy, then the same emit, selection, exact
    rerank and finalize as head()."""
    c = coarse_logits4(x_bits, packed, S_bits, ZS_bits, G)
    cs, ci = block_emit(c, kcand, block_n)
    sel = select_top_r(cs, ci, R)
    e = rerank_exact(x_bits, W_bits, sel)
    oi, ov = finalize(e, sel, k)
    return dict(coarse=c, cand_score=cs, cand_idx=ci, sel=sel, exact=e, idx=oi, val=ov)


# ----------------------------------------------------------------------------------------------
# f2: the variants the design is measured against
# radiance_drafthead.py, module docstring (group 128 against 64; quarter-split against a
# contiguous-4 byte layout; the scale applied to the accumulator against a dequantised weight
# tile) and _emit (candidates from block maxima against a top-k over the whole coarse row).
# Group 64 is quantize / pack / coarse_logits with G = 64; the rest follows.
# ----------------------------------------------------------------------------------------------
def pack_contiguous4(q: np.ndarray) -> np.ndarray:
    """uint8 [N, K/4]: byte j = q[4j] | q[4j+1] << 2 | q[4j+2] << 4 | q[4j+3] << 6."""
    q = q.astype(np.uint8)
    return (q[:, 0::4] | (q[:, 1::4] << 2) | (q[:, 2::4] << 4) | (q[:, 3::4] << 6)).astype(np.uint8)


def unpack_contiguous4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_contiguous4: v uint8 [N, K] with v[n, 4j + t] = (byte j >> 2t) & 3."""
    N, Q = packed.shape
    v = np.empty((N, 4 * Q), dtype=np.uint8)
    for t in range(4):
        v[:, t::4] = (packed >> np.uint8(2 * t)) & np.uint8(3)
    return v


def pack_variant(W_bits: np.ndarray, G: int = GROUP, layout: str = "quarter"):
    """(packed, S, ZS) of the same quantiser at group G in the quarter-split or contiguous-4 layout."""
    check_shape(W_bits.shape[1], G)
    q, sc, zp = quantize(W_bits, G)
    S, ZS = premultiplied_scales(sc, zp)
    packed = pack_quarter_split(q) if layout == "quarter" else pack_contiguous4(q)
    return packed, S, ZS


def coarse_logits_contiguous4(x_bits: np.ndarray, packed: np.ndarray, S_bits: np.ndarray,
                              ZS_bits: np.ndarray, G: int = GROUP) -> np.ndarray:
    """c fp64 [M, N] = x @ (S (1 + v/4) - ZS)^T with v read from the contiguous-4 layout."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    N = packed.shape[0]
    c = np.empty((x.shape[0], N), dtype=np.float64)

    def run(a: int, b: int) -> None:
        v = unpack_contiguous4(packed[a:b]).astype(np.float64)
        s = np.repeat(bf16_to_f32(S_bits[a:b]).astype(np.float64), G, axis=1)
        zs = np.repeat(bf16_to_f32(ZS_bits[a:b]).astype(np.float64), G, axis=1)
        c[:, a:b] = x @ (s * (1.0 + v / 4.0) - zs).T

    _map_chunks(run, N)
    return c


def dequantize_tile(packed: np.ndarray, S_bits: np.ndarray, ZS_bits: np.ndarray,
                    G: int = GROUP) -> np.ndarray:
    """bf16 bits [N, K] of the dequantised weight tile: fl32(fl32(S (1 + v/4)) - ZS), then bf16.

    The product is exact in fp32 (8-bit S times a 3-bit 1 + v/4); the difference rounds once in
    fp32 and the tile is rounded to bf16 for the bf16 dot, so the scale reaches the weight and
    not the accumulator."""
    v = unpack_quarter_split(packed)
    d = (np.float32(1.0) + v.astype(np.float32) / np.float32(4.0)).astype(np.float32)
    s = np.repeat(bf16_to_f32(S_bits), G, axis=1).astype(np.float32)
    zs = np.repeat(bf16_to_f32(ZS_bits), G, axis=1).astype(np.float32)
    w = (s * d).astype(np.float32)
    w = (w - zs).astype(np.float32)
    return f32_to_bf16(w)


def coarse_logits_tile(x_bits: np.ndarray, packed: np.ndarray, S_bits: np.ndarray,
                       ZS_bits: np.ndarray, G: int = GROUP) -> np.ndarray:
    """c fp64 [M, N] = x @ dequantize_tile(...)^T (no group sums of x)."""
    x = bf16_to_f32(x_bits).astype(np.float64)
    N = packed.shape[0]
    c = np.empty((x.shape[0], N), dtype=np.float64)

    def run(a: int, b: int) -> None:
        w = bf16_to_f32(dequantize_tile(packed[a:b], S_bits[a:b], ZS_bits[a:b], G)).astype(np.float64)
        c[:, a:b] = x @ w.T

    _map_chunks(run, N)
    return c


def select_tokens(y_bits: np.ndarray, R: int) -> np.ndarray:
    """sel int32 [M, R]: the R largest entries of each bf16 coarse row, best first (value
    descending, index ascending on ties, -0.0 equal to +0.0); -1 past the row's end."""
    y = bf16_to_f32(y_bits).astype(np.float64) + 0.0  # + 0.0 turns -0.0 into +0.0
    M, N = y.shape
    sel = np.full((M, R), -1, dtype=np.int32)
    cols = np.arange(N)
    for m in range(M):
        o = np.lexsort((cols, -y[m]))[:R]
        sel[m, :len(o)] = o
    return sel
