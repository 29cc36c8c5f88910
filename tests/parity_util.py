"""Comparison rules between the HIP path and the oracle.

* Integer/byte outputs whose inputs are identical on both sides (packed codes, S, ZS; the
  selection, finalize and emit steps when fed the same scores): bit-exact.
* Coarse logits: the bf16 row Y within COARSE_TOL * max_n |c[m, n]| of the oracle (plus its
  own rounding to bf16), the tolerance the head is specified with.
* The fp32 scores the kernels carry (the block candidates) must be far closer. Their error
  comes from fp32 rounding in the per-group terms the kernel forms from sums of x: with the
  dequant read as 1 + v/(4f), a group contributes (f S) P' - xs ((f - 1) S + ZS), and the
  rounding of P' and xs (sums of up to 128 exact products) is multiplied by f S and by
  (f - 1) S + ZS. So the budget of a candidate (m, n) is FOLD_C half-ulps (U32, 2^-24 relative)
  of its fold magnitude B = sum_g (f S + |(f - 1) S + ZS|) * sum_{k in g} |x| (fold_magnitude).
  A worst-case summation order could reach ~127 half-ulps per sum; the kernels' orders (MFMA
  blocks of 32 products, wave reductions) stay below 0.6 on every parity case (recorded with
  I2H_PARITY_LOG), and FOLD_C = 2 leaves room for that while a regression by ten times fails.
  Kernels with no such model (the measured alternatives) are held to COARSE_FP32_TOL * max|c|.
* Index outputs derived from coarse scores (block candidates, the selected set): equal, except
  where the oracle's own coarse scores of the two tokens in question lie within twice the row's
  largest candidate budget of each other (each score may be off by its budget): such a
  difference is "tie-excused", and a difference with a wider gap fails. How many of them would
  also pass the specification's wider window (COARSE_TOL) is reported beside.
* Exact rerank scores: within EXACT_TOL absolute of the fp64 dot; index outputs derived from
  them: equal except oracle exact-score ties within EXACT_TOL (EXACT_TIGHT_TOL counted beside).

With I2H_PARITY_LOG set to a file name, every check_path appends one JSON line of its
statistics there (record()).
"""
import json
import os

import numpy as np

import oracle

COARSE_TOL = 2e-3
COARSE_FP32_TOL = 1e-4   # fallback for kernels without a fold model
FOLD_C = 2.0             # half-ulps of the fold magnitude allowed per candidate score
EXACT_TOL = 1e-3
EXACT_TIGHT_TOL = 1e-5


def record(**stats):
    """Append one JSON line of parity statistics to $I2H_PARITY_LOG (if set)."""
    path = os.environ.get("I2H_PARITY_LOG")
    if not path:
        return
    stats = dict(test=os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], **stats)
    with open(path, "a") as f:
        f.write(json.dumps(stats) + "\n")


def row_scale(c):
    return np.max(np.abs(c), axis=1)


def _ratio(a, b):
    return np.divide(a, b, out=np.zeros_like(a, dtype=np.float64), where=b > 0)


def bf16_half_ulp(v):
    """Half a bf16 ulp at |v| (bf16 keeps 8 significant bits); 0 at v = 0."""
    a = np.abs(v)
    e = np.frexp(np.where(a > 0, a, 1.0))[1]
    return np.where(a > 0, np.ldexp(1.0, e - 9), 0.0)


def check_coarse_values(y_bits, c, tol=COARSE_TOL):
    """Y (bf16) against the oracle's coarse logits: the fp32 coarse logits may differ from c by
    tol * max|c| of the row, and Y adds its own round-to-nearest to bf16. Returns the largest
    excess over the bf16 rounding, relative to the row scale."""
    y = oracle.bf16_to_f32(y_bits).astype(np.float64)
    scale = row_scale(c)
    over = np.maximum(np.abs(y - c) - bf16_half_ulp(c), 0.0).max(axis=1)
    err = _ratio(over, scale)
    assert np.all(over <= tol * scale), f"coarse error {err.max():.3g} > {tol}"
    return float(err.max())


def coarse_fp32_error(cs, ci, c):
    """Largest |candidate score - oracle coarse logit| over valid candidates, / row scale."""
    ok = ci >= 0
    got = np.where(ok, cs.astype(np.float64), 0.0)
    want = np.where(ok, np.take_along_axis(c, np.where(ok, ci, 0).astype(np.int64), axis=1), 0.0)
    return float(_ratio(np.abs(got - want).max(axis=1), row_scale(c)).max())


U32 = 2.0 ** -24  # half an fp32 ulp, relative


def fold_magnitude(ci, x_bits, S_bits, ZS_bits, fold):
    """Per valid candidate (m, n): sum over groups g of (f S[n,g] + |(f - 1) S[n,g] + ZS[n,g]|) *
    sum_{k in g} |x[m,k]|, with f = fold[t] for the quarter t that holds g (len(fold) quarters of
    K / len(fold) each). This is the size of the two per-group terms an fp32 evaluation of the
    coarse logit forms from sums of x: f S P' with P' = sum x (1 + v/(4f)) and xs ((f - 1) S +
    ZS), the page's S P - xs ZS rewritten for a dequant whose bias is 1 + v/(4f) (f = 1 is the
    page's own 1 + v/4). Rounding in those sums costs at most a few half-ulps of this size.
    Returns fp64 [M, ncand] (0 for invalid candidates)."""
    M, K = x_bits.shape
    KG = K // 128
    A = np.abs(oracle.bf16_to_f32(x_bits).astype(np.float64)).reshape(M, KG, 128).sum(axis=2)
    f = np.repeat(np.asarray(fold, np.float64), KG // len(fold))
    s = oracle.bf16_to_f32(S_bits).astype(np.float64)
    z = oracle.bf16_to_f32(ZS_bits).astype(np.float64)
    w = f[None, :] * s + np.abs((f[None, :] - 1.0) * s + z)   # [N, KG]
    out = np.zeros(ci.shape, np.float64)
    for m in range(M):
        ok = ci[m] >= 0
        out[m, ok] = w[ci[m][ok]] @ A[m]
    return out


def fold_error_ratio(cs, ci, c, mag):
    """Largest |candidate score - oracle coarse logit| / (U32 * fold magnitude) over valid
    candidates."""
    ok = (ci >= 0) & (mag > 0)
    want = np.take_along_axis(c, np.where(ci >= 0, ci, 0).astype(np.int64), axis=1)
    err = np.abs(cs.astype(np.float64) - want)
    return float(np.max(np.where(ok, err / np.where(ok, U32 * mag, 1.0), 0.0))) if ok.any() else 0.0


def candidate_budget(ci, x_bits, S_bits, ZS_bits, fold):
    """Allowed |score - oracle| per candidate: FOLD_C * U32 * fold magnitude."""
    return FOLD_C * U32 * fold_magnitude(ci, x_bits, S_bits, ZS_bits, fold)


def tie_window(c, budget):
    """Per row: the gap between two tokens' oracle scores within which the GPU may order them
    either way (twice the row's largest budget; without a budget, 2 COARSE_FP32_TOL * max|c|)."""
    if budget is None:
        return 2 * COARSE_FP32_TOL * row_scale(c)
    return 2 * budget.max(axis=1)


def check_candidates(cs, ci, c, kc, block_n=64, budget=None):
    """Block candidates of the GPU against the oracle's coarse logits c (fp64 [M, N]).

    budget (fp64 [M, nblk*kc] or None): allowed error of each candidate's fp32 score (else
    COARSE_FP32_TOL * max|c|). Returns (differences, differences within the coarse tolerance
    COARSE_TOL); every difference must lie within tie_window. Fails on a wider difference, a
    score off by more than its budget, or an invalid list."""
    M, N = c.shape
    nblk = (N + block_n - 1) // block_n
    o_s, o_i = oracle.block_emit(c, kc, block_n)
    scale = row_scale(c)[:, None]
    g_i = ci.reshape(M, nblk, kc).astype(np.int64)
    o_i3 = o_i.reshape(M, nblk, kc).astype(np.int64)
    # structure: valid indices lie in their block, are distinct; -1 only where the oracle has -1
    blk = np.arange(nblk)[None, :, None]
    valid = g_i >= 0
    assert np.array_equal(valid, o_i3 >= 0), "padding entries differ"
    assert np.all(np.where(valid, (g_i // block_n) == blk, True)), "candidate outside its block"
    srt = np.sort(np.where(valid, g_i, -np.arange(1, kc + 1)[None, None, :]), axis=2)
    assert np.all(np.diff(srt, axis=2) != 0), "duplicate candidate"
    # GPU scores are the GPU's own coarse values of those tokens
    gs = cs.reshape(M, nblk, kc).astype(np.float64)
    cg = np.take_along_axis(c, np.where(valid, g_i, 0).reshape(M, -1), axis=1).reshape(M, nblk, kc)
    err = np.where(valid, np.abs(gs - cg), 0.0)
    if budget is None:
        bud = np.broadcast_to(COARSE_FP32_TOL * scale[:, :, None], err.shape)
    else:
        bud = budget.reshape(M, nblk, kc)
    bad = err > bud
    assert not bad.any(), f"{int(bad.sum())} candidate scores off the oracle's coarse logit by more than their budget"
    assert np.array_equal(np.isneginf(gs), ~valid), "padding entries must score -inf, others finite"
    # each GPU list is ordered by the GPU's own scores
    gsv = np.where(valid, gs, -np.inf)
    assert np.all(gsv[:, :, 1:] <= gsv[:, :, :-1]), "candidates not best first"
    diff = valid & (g_i != o_i3)
    co = np.take_along_axis(c, np.where(o_i3 >= 0, o_i3, 0).reshape(M, -1), axis=1).reshape(M, nblk, kc)
    gap = np.abs(cg - co)
    tight = diff & (gap <= tie_window(c, budget)[:, None, None])
    assert np.array_equal(diff, tight), f"{int((diff & ~tight).sum())} candidate differences beyond the tie window"
    loose = diff & (gap <= COARSE_TOL * scale[:, :, None])
    return int(diff.sum()), int(loose.sum())


def check_selection(sel_g, sel_o, c, budget=None):
    """Selected sets: a token in one set but not the other must have an oracle coarse score
    within the row's tie window (tie_window) of the oracle's R-th best score. Returns the rows
    whose sets differ."""
    M, R = sel_o.shape
    scale = row_scale(c)
    win = tie_window(c, budget)
    ex_rows = 0
    for m in range(M):
        go = set(int(t) for t in sel_g[m] if t >= 0)
        oo = set(int(t) for t in sel_o[m] if t >= 0)
        assert len(go) == int((sel_g[m] >= 0).sum()), "duplicate selection"
        assert len(go) == len(oo), "selection sizes differ"
        if go == oo:
            continue
        thr = c[m, sel_o[m][len(oo) - 1]]
        gap = max(abs(c[m, t] - thr) for t in go ^ oo)
        assert gap <= win[m], f"row {m}: selection differs beyond the tie window ({gap / scale[m]:.3g} * max|c|)"
        ex_rows += 1
    return ex_rows


def check_rerank(ex_g, x_bits, W_bits, sel_g):
    """GPU exact scores against the fp64 dot over the GPU's own selection."""
    e = oracle.rerank_exact(x_bits, W_bits, sel_g)
    ok = sel_g >= 0
    assert np.all(np.isneginf(ex_g[~ok]))
    err = np.abs(ex_g[ok].astype(np.float64) - e[ok])
    assert err.size == 0 or err.max() <= EXACT_TOL, f"rerank error {err.max():.3g}"
    return e, float(err.max()) if err.size else 0.0


def check_final(idx_g, val_g, e_on_gpu_sel, sel_g, k):
    """Final indices against the oracle's finalize over the GPU's selection (exact-score ties
    within EXACT_TOL excused); values within EXACT_TOL. Returns (excused, excused within
    EXACT_TIGHT_TOL)."""
    oi, ov = oracle.finalize(e_on_gpu_sel, sel_g, k)
    M = idx_g.shape[0]
    excused = tight = 0
    for m in range(M):
        emap = {int(t): float(v) for t, v in zip(sel_g[m], e_on_gpu_sel[m]) if t >= 0}
        for j in range(k):
            a, b = int(idx_g[m, j]), int(oi[m, j])
            if a == b:
                continue
            assert a in emap and b in emap, f"row {m} place {j}: {a} vs {b}"
            assert abs(emap[a] - emap[b]) <= EXACT_TOL, f"row {m} place {j}: {a} vs {b}"
            excused += 1
            tight += int(abs(emap[a] - emap[b]) <= EXACT_TIGHT_TOL)
        ok = oi[m] >= 0
        assert np.all(np.abs(val_g[m][ok].astype(np.float64) - ov[m][ok]) <= EXACT_TOL)
    return excused, tight


def final_vs_oracle(idx_g, res_o, sel_g, e_on_gpu_sel):
    """Final answer against the oracle's own end-to-end answer. Where the GPU selected the same
    set as the oracle, the answers must agree up to exact-score ties (EXACT_TOL); where the
    sets differ (excused by check_selection), the GPU answer must be the correct finalize of its
    own set, which check_final verifies. Returns (matching places, places excused by a
    selection difference, places excused by an exact tie)."""
    M, k = idx_g.shape
    match = sel_excused = tie_excused = 0
    for m in range(M):
        same = set(int(t) for t in sel_g[m] if t >= 0) == set(int(t) for t in res_o["sel"][m] if t >= 0)
        emap = {int(t): float(v) for t, v in zip(sel_g[m], e_on_gpu_sel[m]) if t >= 0}
        for j in range(k):
            a, b = int(idx_g[m, j]), int(res_o["idx"][m, j])
            if a == b:
                match += 1
            elif not same:
                sel_excused += 1
            else:
                assert abs(emap[a] - emap[b]) <= EXACT_TOL, f"row {m} place {j}: {a} vs oracle {b}"
                tie_excused += 1
    return match, sel_excused, tie_excused
