"""Comparison rules between the HIP path and the oracle.

* Integer/byte outputs whose inputs are identical on both sides (packed codes, S, ZS; the
  selection, finalize and emit steps when fed the same scores): bit-exact.
* Coarse logits (fp32 accumulation in the kernel vs fp64 in the oracle): within
  COARSE_TOL * max_n |c[m, n]| per row.
* Index outputs derived from coarse scores (block candidates, the selected set): equal, except
  where the oracle's own coarse scores of the two tokens in question lie within the coarse
  tolerance of each other ("tie-excused"). A tighter window (TIGHT_TOL) is counted beside it.
* Exact rerank scores: within EXACT_TOL absolute of the fp64 dot; index outputs derived from
  them: equal except oracle exact-score ties within EXACT_TOL.
"""
import numpy as np

import oracle

COARSE_TOL = 2e-3
TIGHT_TOL = 1e-5
EXACT_TOL = 1e-3


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


def check_candidates(cs, ci, c, kc, block_n=64):
    """Block candidates of the GPU against the oracle's coarse logits c (fp64 [M, N]).

    Returns (excused, tight_excused). Fails on any unexcused difference or invalid list."""
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
    assert np.all(np.where(valid, np.abs(gs - cg) <= COARSE_TOL * scale[:, :, None], True)), \
        "candidate score differs from the oracle's coarse logit"
    assert np.array_equal(np.isneginf(gs), ~valid), "padding entries must score -inf, others finite"
    # each GPU list is ordered by the GPU's own scores
    gsv = np.where(valid, gs, -np.inf)
    assert np.all(gsv[:, :, 1:] <= gsv[:, :, :-1]), "candidates not best first"
    diff = valid & (g_i != o_i3)
    co = np.take_along_axis(c, np.where(o_i3 >= 0, o_i3, 0).reshape(M, -1), axis=1).reshape(M, nblk, kc)
    gap = np.abs(cg - co)
    excused = diff & (gap <= COARSE_TOL * scale[:, :, None])
    assert np.array_equal(diff, excused), f"{int((diff & ~excused).sum())} unexcused candidate differences"
    tight = diff & (gap <= TIGHT_TOL * scale[:, :, None])
    return int(diff.sum()), int(tight.sum())


def check_selection(sel_g, sel_o, c):
    """Selected sets: a token in one set but not the other must have an oracle coarse score
    within tolerance of the oracle's R-th best score. Returns (excused rows, tight rows)."""
    M, R = sel_o.shape
    scale = row_scale(c)
    ex_rows = tight_rows = 0
    for m in range(M):
        go = set(int(t) for t in sel_g[m] if t >= 0)
        oo = set(int(t) for t in sel_o[m] if t >= 0)
        assert len(go) == int((sel_g[m] >= 0).sum()), "duplicate selection"
        assert len(go) == len(oo), "selection sizes differ"
        if go == oo:
            continue
        thr = c[m, sel_o[m][len(oo) - 1]]
        gap = max(abs(c[m, t] - thr) for t in go ^ oo)
        assert gap <= COARSE_TOL * scale[m], f"row {m}: selection differs beyond tolerance ({gap / scale[m]:.3g})"
        ex_rows += 1
        tight_rows += int(gap <= TIGHT_TOL * scale[m])
    return ex_rows, tight_rows


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
    within EXACT_TOL excused); values within EXACT_TOL. Returns the excused count."""
    oi, ov = oracle.finalize(e_on_gpu_sel, sel_g, k)
    M = idx_g.shape[0]
    excused = 0
    for m in range(M):
        emap = {int(t): float(v) for t, v in zip(sel_g[m], e_on_gpu_sel[m]) if t >= 0}
        for j in range(k):
            a, b = int(idx_g[m, j]), int(oi[m, j])
            if a == b:
                continue
            assert a in emap and b in emap, f"row {m} place {j}: {a} vs {b}"
            assert abs(emap[a] - emap[b]) <= EXACT_TOL, f"row {m} place {j}: {a} vs {b}"
            excused += 1
        ok = oi[m] >= 0
        assert np.all(np.abs(val_g[m][ok].astype(np.float64) - ov[m][ok]) <= EXACT_TOL)
    return excused


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
