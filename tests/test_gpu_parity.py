"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Inputs come from synth_inputs; expected values come only from oracle/. Rules in parity_util.
"""
import numpy as np
import pytest
import torch

import oracle
import parity_util as pu
import synth_inputs as si

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def i2h():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import bit_quantized_lm_int2_amd as lib
    lib.lib()  # the HIP library must load; there is no fallback
    return lib


DEV = "cuda:0"


def dev_bf16(b):
    return torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(DEV)


def host(t):
    if t.dtype == torch.bfloat16:
        return si.bits(t)
    return t.cpu().numpy()


def say(*a):
    print(*a, flush=True)


# ---------------------------------------------------------------------------------------------
# pack: bit-exact
# ---------------------------------------------------------------------------------------------
def degenerate_rows(K):
    rows = [np.full(K, 0x3F00, np.uint16),              # constant 0.5
            np.full(K, 0xBF00, np.uint16),              # constant -0.5
            np.zeros(K, np.uint16),                     # all zero
            (np.arange(K) % 7 + 0x3C00).astype(np.uint16),   # all positive (lo > 0)
            (np.arange(K) % 5 + 0xBC00).astype(np.uint16),   # all negative (hi < 0)
            np.where(np.arange(K) % 2 == 0, 0x7E00, 0xFE00).astype(np.uint16),  # huge +-2^125
            np.where(np.arange(K) % 3 == 0, 0x0001, 0x8001).astype(np.uint16)]  # subnormal
    return np.stack(rows)


@pytest.mark.parametrize("N,K", [(4096, 512), (1000, 1024), (37, 5120), (5, 2048)])
def test_pack_bit_exact(i2h, N, K):
    say(f"pack N={N} K={K}")
    W = si.bits(si.gen_weight(N, K, seed=100 + N))
    W = np.concatenate([W, degenerate_rows(K)])
    p, S, ZS = i2h.pack(dev_bf16(W))
    po, So, ZSo = oracle.pack(W)
    assert np.array_equal(host(p), po)
    assert np.array_equal(host(S), So)
    assert np.array_equal(host(ZS), ZSo)


def test_pack_strided_rows(i2h):
    K = 1024
    wide = si.gen_weight(300, K + 64, seed=7).to(DEV)
    W = wide[:, 32:32 + K]   # row stride K + 64, 64-byte offset
    p, S, ZS = i2h.pack(W)
    po, So, ZSo = oracle.pack(si.bits(W))
    assert np.array_equal(host(p), po) and np.array_equal(host(S), So) and np.array_equal(host(ZS), ZSo)


def test_pack_exact_grid_head(i2h):
    from test_oracle_pins import grid_head
    Wb, q, zp, sc = grid_head(500, 1024, 21)
    p, S, ZS = i2h.pack(dev_bf16(Wb))
    assert np.array_equal(host(p), oracle.pack_quarter_split(q.astype(np.uint8)))
    assert np.array_equal(oracle.bf16_to_f32(host(S)).astype(np.float64), 4 * sc)
    assert np.array_equal(oracle.bf16_to_f32(host(ZS)).astype(np.float64), (4 + zp) * sc)


# ---------------------------------------------------------------------------------------------
# xsum
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,K", [(1, 512), (72, 5120), (3, 16384), (5, 640), (2, 256)])
def test_xsum(i2h, M, K):
    xb = si.bits(si.gen_x(M, K, outliers=8, seed=3))
    xs = host(i2h.xsum(dev_bf16(xb)))
    want = oracle.group_sums(xb)
    absx = np.abs(oracle.bf16_to_f32(xb).astype(np.float64)).reshape(M, K // 128, 128).sum(2)
    assert np.all(np.abs(xs - want) <= 128 * 2.0 ** -24 * absx + 1e-30)


# ---------------------------------------------------------------------------------------------
# selection and finalize on identical inputs: bit-exact, ties included
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,kc,R,grid", [(1, 124160, 8, 32, 0), (5, 4096, 8, 32, 4), (3, 248320, 8, 32, 0),
                                           (4, 643, 8, 100, 2), (2, 5000, 1, 1, 1), (2, 9000, 64, 128, 8),
                                           (3, 4096, 8, 1024, 0), (1, 1000, 8, 32, 0.25),
                                           (2, 524288, 2, 64, 0), (3, 20000, 16, 64, 2), (2, 20000, 16, 65, 0),
                                           (2, 70000, 8, 64, 0)])
def test_select_bit_exact(i2h, M, N, kc, R, grid):
    say(f"select M={M} N={N} kc={kc} R={R}")
    sc = si.gen_scores(M, N, seed=N + R).numpy()
    if grid:
        sc = (np.round(sc * grid) / grid).astype(np.float32)  # many exact ties
    cs, ci = oracle.block_emit(sc.astype(np.float64), kc)
    want = oracle.select_top_r(cs, ci, R)
    got = i2h.select(torch.from_numpy(cs.astype(np.float32)).to(DEV), torch.from_numpy(ci).to(DEV), kc, R)
    assert np.array_equal(host(got), want)


def test_select_periodic_scores(i2h):
    """Block scores repeat every 16 blocks, so every wave's list reaches deep into the ties and
    far more than 64 list entries clear the first-pass bound."""
    N = 124160
    c = -(((np.arange(N) // 64) % 16).astype(np.float64))[None, :].repeat(2, 0)
    c[1] *= 0.5
    cs, ci = oracle.block_emit(c, 8)
    want = oracle.select_top_r(cs, ci, 32)
    got = i2h.select(torch.from_numpy(cs.astype(np.float32)).to(DEV), torch.from_numpy(ci).to(DEV), 8, 32)
    assert np.array_equal(host(got), want)


def test_select_all_equal_scores(i2h):
    cs, ci = oracle.block_emit(np.zeros((2, 124160)), 8)
    want = oracle.select_top_r(cs, ci, 32)
    got = i2h.select(torch.from_numpy(cs.astype(np.float32)).to(DEV), torch.from_numpy(ci).to(DEV), 8, 32)
    assert np.array_equal(host(got), want)


@pytest.mark.parametrize("M,N,K,kc,R,k,grid", [
    (1, 124160, 5120, 8, 32, 1, 0),    # the draft-slot shape: two blocks per thread
    (3, 248320, 5120, 8, 32, 16, 0),   # the full vocabulary: four blocks per thread, top-16
    (2, 4096, 512, 8, 32, 16, 4),      # many exact score ties
    (2, 643, 1024, 3, 64, 64, 2),      # kcand 3; R above the number of candidates; every place
    (4, 9000, 2048, 1, 1, 1, 0),       # one candidate per block, one token
    (2, 70000, 16384, 8, 64, 16, 1),   # R = 64, the largest K
])
def test_select_rerank_fused(i2h, M, N, K, kc, R, k, grid):
    """The fused selection + rerank + top-k against the three separate calls (bit for bit) and the
    oracle's selection; exact scores against the fp64 dot where the weight fits on the host."""
    say(f"select_rerank M={M} N={N} K={K} kc={kc} R={R} k={k}")
    sc = si.gen_scores(M, N, seed=N + R + 7).numpy()
    if grid:
        sc = (np.round(sc * grid) / grid).astype(np.float32)
    cs, ci = oracle.block_emit(sc.astype(np.float64), kc)
    want_sel = oracle.select_top_r(cs, ci, R)
    cs_d, ci_d = torch.from_numpy(cs.astype(np.float32)).to(DEV), torch.from_numpy(ci).to(DEV)
    g = torch.Generator(device=DEV).manual_seed(N + K)
    W = (0.02 * torch.randn(N, K, generator=g, device=DEV)).to(torch.bfloat16)
    x = torch.randn(M, K, generator=g, device=DEV).to(torch.bfloat16)
    sel = i2h.select(cs_d, ci_d, kc, R)
    ex = i2h.rerank(x, W, sel)
    oi, ov = i2h.finalize(ex, sel, k)
    fi, fv, fsel, fex = i2h.select_rerank_topk(cs_d, ci_d, kc, R, x, W, k, want_sel=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(fsel), want_sel)
    assert torch.equal(fsel, sel) and torch.equal(fex, ex), "fused selection / exact scores differ"
    assert torch.equal(fi, oi) and torch.equal(fv, ov), "fused top-k differs"
    if N * K <= 100_000_000:
        pu.check_rerank(host(fex), si.bits(x), si.bits(W), host(fsel))


def _bound_counts(cs_row, ci_row, kc, R):
    """What the fused tail's ranking bound lets through on a row: the blocks at or above the
    smallest of its 16 waves' ceil(R / 16)-th best block keys (thread t holds blocks t, t + 1024,
    ...; wave t // 64; a block key is (best score descending, block ascending)), and the valid
    entries of those blocks at or above (that bound's score, the last token of its block)."""
    nblk = cs_row.shape[0] // kc
    best = cs_row[::kc].astype(np.float64)
    order = np.lexsort((np.arange(nblk), -best))
    rank = np.empty(nblk, np.int64)
    rank[order] = np.arange(nblk)
    t, worst = (R + 15) // 16, -1
    for w in range(16):
        r = np.sort(rank[(np.arange(nblk) % 1024) // 64 == w])
        assert r.size >= t
        worst = max(worst, int(r[t - 1]))
    bT = int(order[worst])
    sT = best[bT]
    own = (best > sT) | ((best == sT) & (np.arange(nblk) <= bT))
    sc, tk = cs_row.reshape(nblk, kc).astype(np.float64), ci_row.reshape(nblk, kc)
    above = (sc > sT) | ((sc == sT) & (tk <= 64 * bT + 63))
    return int(own.sum()), int((above & own[:, None] & (tk >= 0)).sum())


def test_select_rerank_gather_paths(i2h):
    """Rows built so that the ranking bound lets through 32 entries (every wave has two far-ahead
    blocks: one ranking, 8 threads per key), about 200 (one wave's second best sits low: one
    ranking, 4 threads per key) and nearly every block (one wave holds no high block: more than
    256 entries, so the general path, whose block ranking takes the radix passes). Each row's
    counts are checked on the host first; the fused tail must still equal the separate calls and
    the oracle's selection."""
    N, K, kc, R, k = 124160, 1024, 8, 32, 4
    sc = si.gen_scores(3, N, seed=5).numpy().astype(np.float64)
    nb = N // 64
    wave_of = (np.arange(nb) % 1024) // 64
    for w in range(16):
        b0, b1 = np.flatnonzero(wave_of == w)[:2]
        sc[0, 64 * b0] = 10.0 + w / 64
        sc[0, 64 * b1 + 5] = 9.0 + w / 64
    for b in np.flatnonzero(wave_of == 15):
        sc[1, 64 * b:64 * b + 64] = -5.0
        sc[2, 64 * b:64 * b + 64] = -100.0
    b0, b1 = np.flatnonzero(wave_of == 15)[:2]
    sc[1, 64 * b0] = 3.0
    sc[1, 64 * b1] = 2.95
    cs, ci = oracle.block_emit(sc, kc)
    counts = [_bound_counts(cs[m], ci[m], kc, R) for m in range(3)]
    (_, e0), (_, e1), (b2, e2) = counts
    assert e0 == 32 and 128 < e1 <= 256 and e2 > 256 and b2 > 256, counts
    want_sel = oracle.select_top_r(cs, ci, R)
    cs_d, ci_d = torch.from_numpy(cs.astype(np.float32)).to(DEV), torch.from_numpy(ci).to(DEV)
    g = torch.Generator(device=DEV).manual_seed(91)
    W = (0.02 * torch.randn(N, K, generator=g, device=DEV)).to(torch.bfloat16)
    x = torch.randn(3, K, generator=g, device=DEV).to(torch.bfloat16)
    sel = i2h.select(cs_d, ci_d, kc, R)
    ex = i2h.rerank(x, W, sel)
    oi, ov = i2h.finalize(ex, sel, k)
    fi, fv, fsel, fex = i2h.select_rerank_topk(cs_d, ci_d, kc, R, x, W, k, want_sel=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(fsel), want_sel)
    assert torch.equal(fsel, sel) and torch.equal(fex, ex), "fused selection / exact scores differ"
    assert torch.equal(fi, oi) and torch.equal(fv, ov), "fused top-k differs"


@pytest.mark.parametrize("M,R,k,grid", [(3, 32, 1, 0), (3, 32, 16, 2), (2, 100, 100, 1), (4, 1024, 16, 4),
                                        (1, 1, 1, 0)])
def test_finalize_bit_exact(i2h, M, R, k, grid):
    e = si.gen_scores(M, R, seed=R + k).numpy()
    if grid:
        e = (np.round(e * grid) / grid).astype(np.float32)
    sel = si.gen_rows(M, R, 300000, seed=R).numpy()
    sel[0, R // 2] = -1
    oi, ov = oracle.finalize(e.astype(np.float64), sel, k)
    gi, gv = i2h.finalize(torch.from_numpy(e).to(DEV), torch.from_numpy(sel).to(DEV), k)
    assert np.array_equal(host(gi), oi)
    assert np.array_equal(host(gv).astype(np.float64), ov)


# ---------------------------------------------------------------------------------------------
# rerank
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,K,R", [(1, 4096, 512, 32), (16, 20000, 5120, 32), (3, 300, 16384, 7)])
def test_rerank(i2h, M, N, K, R):
    xb = si.bits(si.gen_x(M, K, outliers=8, seed=5))
    Wb = si.bits(si.gen_weight(N, K, seed=6))
    sel = si.gen_rows(M, R, N, seed=8).numpy()
    sel[0, 0] = -1
    sel[-1, -1] = N + 5   # out of range: -inf
    ex = host(i2h.rerank(dev_bf16(xb), dev_bf16(Wb), torch.from_numpy(sel).to(DEV)))
    assert np.isneginf(ex[0, 0]) and np.isneginf(ex[-1, -1])
    s2 = sel.copy()
    s2[-1, -1] = -1
    pu.check_rerank(ex, xb, Wb, s2)


# ---------------------------------------------------------------------------------------------
# coarse pass on a head whose every sum is exact in fp32: the whole path is bit-exact,
# so the tie rules of the emit, selection and finalize are checked exactly
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,kc,R,k", [(3, 4096, 8, 32, 16), (17, 643, 8, 40, 5), (1, 2000, 64, 128, 1),
                                        (40, 1000, 3, 32, 16)])
def test_exact_arithmetic_head_bit_exact(i2h, M, N, kc, R, k):
    from test_oracle_pins import grid_head
    K = 512
    Wb, q, zp, sc = grid_head(N, K, 31)
    # same sc = 2^-4 everywhere keeps every partial sum exact in fp32
    qg = q.reshape(N, K // 128, 128)
    w = (2.0 ** -4 * (qg - zp[:, :, None])).reshape(N, K)
    Wb = oracle.f32_to_bf16(w.astype(np.float32))
    rng = np.random.default_rng(M)
    xf = rng.integers(-2, 3, size=(M, K)).astype(np.float32)
    xf[0] = 0.0                                   # a row of pure ties
    xb = oracle.f32_to_bf16(xf)
    x, W = dev_bf16(xb), dev_bf16(Wb)
    p, S, ZS = i2h.pack(W)
    xs = i2h.xsum(x)
    cs, ci, y = i2h.coarse_topk(x, xs, p, S, ZS, kcand=kc, want_y=True)
    sel = i2h.select(cs, ci, kc, R)
    ex = i2h.rerank(x, W, sel)
    oi, ov = i2h.finalize(ex, sel, k)
    po, So, ZSo = oracle.pack(Wb)
    res = oracle.head(xb, Wb, po, So, ZSo, kcand=kc, R=R, k=k)
    assert np.array_equal(host(y), oracle.f32_to_bf16(res["coarse"].astype(np.float32)))
    assert np.array_equal(host(ci), res["cand_idx"])
    assert np.array_equal(host(cs).astype(np.float64), res["cand_score"])
    assert np.array_equal(host(sel), res["sel"])
    assert np.array_equal(host(ex).astype(np.float64), res["exact"])
    assert np.array_equal(host(oi), res["idx"])
    assert np.array_equal(host(ov).astype(np.float64), res["val"])


# ---------------------------------------------------------------------------------------------
# end to end on Gaussian heads, tolerance rules
# ---------------------------------------------------------------------------------------------
def gpu_paths(i2h, x, W, p, S, ZS, kc, R, k):
    """The head through its separate entry points, two ways: (a) the kernels i2h_head runs
    (group sums in the coarse kernel when it can, fused rerank+finalize), checked bit for bit
    against i2h_head itself; (b) xsum, coarse_topk, select, rerank, finalize one by one."""
    M, K = x.shape
    own = i2h.coarse_sums_x(M, K)
    xs = None if own else i2h.xsum(x)
    cs, ci, y = i2h.coarse_topk(x, xs, p, S, ZS, kcand=kc, want_y=True)
    sel = i2h.select(cs, ci, kc, R)
    ex = torch.empty(M, R, dtype=torch.float32, device=x.device)
    oi, ov = i2h.rerank_topk(x, W, sel, k, exact=ex)
    hi, hv = i2h.head(x, p, S, ZS, W, kcand=kc, R=R, k=k)
    torch.cuda.synchronize()
    assert torch.equal(hi, oi) and torch.equal(hv, ov), "i2h_head differs from its own kernels"
    a = dict(cs=cs, ci=ci, y=y, sel=sel, ex=ex, oi=oi, ov=ov)
    xs_b = i2h.xsum(x)
    cs_b, ci_b, y_b = i2h.coarse_topk(x, xs_b, p, S, ZS, kcand=kc, want_y=True)
    sel_b = i2h.select(cs_b, ci_b, kc, R)
    ex_b = i2h.rerank(x, W, sel_b)
    oi_b, ov_b = i2h.finalize(ex_b, sel_b, k)
    torch.cuda.synchronize()
    b = dict(cs=cs_b, ci=ci_b, y=y_b, sel=sel_b, ex=ex_b, oi=oi_b, ov=ov_b)
    return a, b


FOLD2 = (32.0, 8.0, 2.0, 1.0)  # the int2 kernels' bias fold per quarter (mask dequant 1 + v/(4f))


def check_path(g, res, rows, xr, Wb, kc, k, label, scales, fold=FOLD2):
    c = res["coarse"]
    yh, csh, cih = host(g["y"])[rows], host(g["cs"])[rows], host(g["ci"])[rows]
    ok = cih >= 0
    # Y is the bf16 rounding of the same fp32 logits the candidates carry
    assert np.array_equal(np.take_along_axis(yh, np.where(ok, cih, 0).astype(np.int64), axis=1)[ok],
                          oracle.f32_to_bf16(csh[ok]))
    err = pu.check_coarse_values(yh, c)
    err32 = pu.coarse_fp32_error(csh, cih, c)
    mag = pu.fold_magnitude(cih, xr, scales[0], scales[1], fold)
    fold_ratio = pu.fold_error_ratio(csh, cih, c, mag)
    budget = pu.FOLD_C * pu.U32 * mag
    cand_diff, cand_loose = pu.check_candidates(csh, cih, c, kc, budget=budget)
    g_sel = host(g["sel"])[rows]
    sel_rows = pu.check_selection(g_sel, res["sel"], c, budget=budget)
    e_g, rerr = pu.check_rerank(host(g["ex"])[rows], xr, Wb, g_sel)
    fin_ex, fin_tight = pu.check_final(host(g["oi"])[rows], host(g["ov"])[rows], e_g, g_sel, k)
    match, sel_excused, tie_excused = pu.final_vs_oracle(host(g["oi"])[rows], res, g_sel, e_g)
    say(f"  [{label}] rows={len(rows)} coarse_err(bf16 Y)={err:.2e} coarse_err(fp32)={err32:.2e} "
        f"cand_diff={cand_diff} sel_diff_rows={sel_rows} rerank_err={rerr:.2e} final match={match} "
        f"sel_excused={sel_excused} tie_excused={tie_excused} (finalize ties {fin_ex}, tight {fin_tight})")
    pu.record(path=label, rows=int(len(rows)), k=int(k), K=int(xr.shape[1]), N=int(c.shape[1]), coarse_err_y=err,
              coarse_err_fp32=err32, fold_error_ratio=fold_ratio, tie_window=float(pu.tie_window(c, budget).max()
                                                                                  / max(pu.row_scale(c).max(), 1e-300)),
              cand_diff=cand_diff, cand_diff_within_coarse_tol=cand_loose, sel_diff_rows=sel_rows,
              rerank_err=rerr, final_places=int(len(rows) * k), final_match=match, final_sel_excused=sel_excused,
              final_tie_excused=tie_excused, finalize_ties=fin_ex, finalize_ties_tight=fin_tight)
    return match


def run_and_check(i2h, xb, Wb, kc=8, R=32, k=1, packed_o=None, coarse_o=None, rows=None):
    """Both GPU paths against the oracle; rows: subset of rows the oracle checks."""
    x, W = dev_bf16(xb), dev_bf16(Wb)
    p, S, ZS = i2h.pack(W)
    a, b = gpu_paths(i2h, x, W, p, S, ZS, kc, R, k)
    rows = np.arange(xb.shape[0]) if rows is None else np.asarray(rows)
    if packed_o is None:
        packed_o = oracle.pack(Wb)
        assert np.array_equal(host(p), packed_o[0])
        assert np.array_equal(host(S), packed_o[1]) and np.array_equal(host(ZS), packed_o[2])
    po, So, ZSo = packed_o
    xr = xb[rows]
    res = oracle.head(xr, Wb, po, So, ZSo, kcand=kc, R=R, k=k, coarse=None if coarse_o is None else coarse_o[rows])
    match = check_path(a, res, rows, xr, Wb, kc, k, "head kernels", scales=(So, ZSo))
    check_path(b, res, rows, xr, Wb, kc, k, "separate calls", scales=(So, ZSo))
    return dict(match=match, places=len(rows) * k, res=res, gpu_idx=host(a["oi"])[rows])


@pytest.mark.parametrize("M,N,K,kc,R,k", [
    (1, 4096, 512, 8, 32, 1),      # the tiny head
    (3, 4133, 512, 8, 32, 16),     # ragged tail block of 37 columns
    (17, 643, 1024, 8, 100, 16),   # tail block with 3 < kcand columns; R above the valid count
    (33, 3000, 5120, 8, 32, 1),    # three m-tiles of 16 rows, one partly filled
    (64, 2048, 2048, 16, 64, 16),
    (72, 1500, 512, 8, 32, 16),    # the 72-row band
    (130, 700, 512, 4, 16, 4),     # more rows than one launch holds
    (5, 4096, 16384, 8, 32, 1),    # largest K
    (2, 2000, 512, 1, 1, 1),       # one candidate per block, one reranked token
    (9, 4133, 512, 8, 32, 16),     # many-row kernel, 16-row tile, ragged tail block
    (16, 130, 5120, 8, 16, 1),     # three blocks: one workgroup with an idle wave
    (24, 3001, 5120, 12, 64, 16),  # 32-row tile; kcand above 8 (counted emit)
    (40, 1000, 512, 3, 16, 4),     # 64-row tile, three candidates per block
    (4, 1037, 5120, 8, 32, 16),    # 3-4 rows through the 16-row tile, ragged tail
    (2, 1037, 5120, 8, 32, 16),    # two rows through the one-row kernel's 2-row form, ragged tail
    (2, 1500, 4096, 8, 32, 1),     # the 2-row form unrolled for other K of the family
    (2, 999, 2048, 3, 16, 4),
    (2, 3001, 3072, 8, 64, 16),
    (2, 640, 1024, 8, 32, 1),
    (65, 1000, 5120, 8, 32, 1),    # a 64-row launch and a 1-row chunk on the M = 1 kernel with xs
    (33, 643, 5120, 8, 32, 16),    # 64-row tile with one row of its last m-tile, tail block
    (1, 1, 512, 8, 32, 1),         # a one-token vocabulary: one valid candidate
    (5, 63, 512, 8, 8, 4),         # one partial block
    (40, 65, 5120, 8, 16, 16),     # nine valid candidates for R = 16: empty places in the top-16
    (16, 3001, 4096, 8, 32, 1),    # tiles built for other K of the family: 16, 32 and 64 rows
    (24, 2000, 3072, 8, 32, 16),
    (50, 1500, 2048, 8, 32, 4),
    (3, 1100, 1024, 8, 32, 1),
    (2, 700, 1536, 8, 32, 1),      # a K with no tile: the small kernel for up to 4 rows
    (1, 2001, 4096, 8, 32, 1),     # the M = 1 kernel unrolled for other K of the family
    (1, 1999, 3072, 8, 32, 16),
    (1, 777, 2048, 8, 32, 1),
    (1, 640, 1024, 8, 32, 1),
])
def test_head_parity(i2h, M, N, K, kc, R, k):
    say(f"head M={M} N={N} K={K} kc={kc} R={R} k={k}")
    xb = si.bits(si.gen_x(M, K, outliers=8 if K >= 1024 else 0, seed=M + K))
    Wb = si.bits(si.gen_weight(N, K, seed=N + K))
    run_and_check(i2h, xb, Wb, kc=kc, R=R, k=k)


@pytest.mark.parametrize("M,N,K,k", [(1, 4133, 5120, 1), (16, 4133, 5120, 16), (40, 2000, 512, 4)])
def test_head_graph_replay(i2h, M, N, K, k):
    """i2h_head captured in a HIP graph (the library allocates, clears and synchronises nothing):
    three replays, with eager work and a synchronisation between them, each give the eager result
    bit for bit."""
    say(f"graph replay M={M} N={N} K={K} k={k}")
    xb = si.bits(si.gen_x(M, K, outliers=8 if K >= 1024 else 0, seed=M + 7))
    Wb = si.bits(si.gen_weight(N, K, seed=N + 3))
    x, W = dev_bf16(xb), dev_bf16(Wb)
    p, S, ZS = i2h.pack(W)
    ws = torch.empty(i2h.workspace_bytes(M, N, K, 8, 32), dtype=torch.uint8, device=DEV)
    oi = torch.empty(M, k, dtype=torch.int32, device=DEV)
    ov = torch.empty(M, k, dtype=torch.float32, device=DEV)
    ei, ev = i2h.head(x, p, S, ZS, W, k=k)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        i2h.head(x, p, S, ZS, W, k=k, workspace=ws, out=(oi, ov))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        i2h.head(x, p, S, ZS, W, k=k, workspace=ws, out=(oi, ov))
    for r in range(3):
        oi.fill_(-7)
        ov.fill_(0.0)
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(oi, ei) and torch.equal(ov, ev), f"replay {r} differs from the eager call"


@pytest.mark.parametrize("M,N,K,kc,R,k", [
    (1, 124160, 5120, 8, 32, 1),  # the draft slot: 32 workgroups of one token each
    (3, 20011, 5120, 8, 32, 16),  # ragged tail block
    (16, 9000, 2048, 8, 32, 4),   # the largest row count that splits (4 per row)
    (2, 5000, 512, 8, 5, 5),      # R below the split: one token per workgroup
    (1, 7000, 5120, 8, 64, 64),   # the largest R: 2 tokens per workgroup, every one returned
    (4, 3000, 1024, 1, 16, 16),   # one candidate per block
    (4, 200003, 5120, 8, 32, 16), # four blocks per thread, 16 workgroups per row, ragged tail
    (16, 248320, 5120, 8, 32, 16),  # the full vocabulary at 16 rows: four per row
])
def test_head_split_tail(i2h, M, N, K, kc, R, k):
    """Up to 16 rows the head splits each row's exact rerank over several workgroups, with an
    arrival count per row in the workspace that the head's first kernel zeroes. Its outputs equal
    those of the one-workgroup tail (i2h_select_rerank_topk on the same candidates) bit for bit,
    on a workspace filled with garbage and again on a second call that reuses it."""
    say(f"split tail M={M} N={N} K={K} kc={kc} R={R} k={k}")
    xb = si.bits(si.gen_x(M, K, outliers=8, seed=M + 31))
    Wb = si.bits(si.gen_weight(N, K, seed=N + 5))
    x, W = dev_bf16(xb), dev_bf16(Wb)
    p, S, ZS = i2h.pack(W)
    xs = None if i2h.coarse_sums_x(M, K) else i2h.xsum(x)
    cs, ci, _ = i2h.coarse_topk(x, xs, p, S, ZS, kcand=kc)
    ei, ev = i2h.select_rerank_topk(cs, ci, kc, R, x, W, k)
    ws = torch.full((i2h.workspace_bytes(M, N, K, kc, R),), 0xFF, dtype=torch.uint8, device=DEV)
    for call in range(2):
        oi, ov = i2h.head(x, p, S, ZS, W, kcand=kc, R=R, k=k, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(oi, ei) and torch.equal(ov, ev), f"call {call} differs from the one-workgroup tail"


def test_head_zero_rows(i2h):
    """x rows of zeros: every score ties, the tie rules decide (lowest indices win)."""
    K, N = 512, 4096
    xb = si.bits(si.gen_x(4, K, seed=9))
    xb[1] = 0
    xb[3] = 0x8000  # negative zeros
    Wb = si.bits(si.gen_weight(N, K, seed=10))
    out = run_and_check(i2h, xb, Wb, k=16)
    want = [b * 64 + j for b in range(4) for j in range(8)][:16]
    assert list(out["gpu_idx"][1]) == want and list(out["gpu_idx"][3]) == want


# ---------------------------------------------------------------------------------------------
# full sizes: one rank's 124160-row vocab slice at M = 1 to 64, and the full 248320-row vocab
# ---------------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def slice_head():
    cfg = si.WORKLOADS["draft_band_m64_k5120_n124160"]
    say("generating the 124160 x 5120 head")
    Wb = si.bits(si.gen_weight(cfg["N"], cfg["K"]))
    xb = si.bits(si.gen_x(64, cfg["K"], outliers=cfg["outliers"]))
    packed_o = oracle.pack(Wb)
    say("oracle coarse, 64 rows")
    coarse_o = oracle.coarse_logits(xb, *packed_o)
    return xb, Wb, packed_o, coarse_o


@pytest.mark.parametrize("M", [1, 5, 16, 32, 40, 64])   # small kernel; 16-, 32- and 64-row tiles
def test_vocab_slice_full_size(i2h, slice_head, M):
    xb, Wb, packed_o, coarse_o = slice_head
    say(f"vocab slice M={M}")
    p, S, ZS = i2h.pack(dev_bf16(Wb))
    assert np.array_equal(host(p), packed_o[0])
    assert np.array_equal(host(S), packed_o[1]) and np.array_equal(host(ZS), packed_o[2])
    out = run_and_check(i2h, xb[:M], Wb, packed_o=packed_o, coarse_o=coarse_o[:M])
    say(f"  argmax match vs oracle: {out['match']}/{out['places']}")


@pytest.fixture(scope="module")
def full_vocab_head():
    cfg = si.WORKLOADS["full_vocab_top16_k5120_n248320"]
    N, K = cfg["N"], cfg["K"]
    say("generating the 248320 x 5120 head")
    Wb = si.bits(si.gen_weight(N, K))
    xb = si.bits(si.gen_x(72, K, outliers=cfg["outliers"]))
    say("oracle pack of the full vocabulary")
    packed_o = oracle.pack(Wb)
    say("oracle coarse, 72 rows of the full vocabulary")
    coarse_o = oracle.coarse_logits(xb, *packed_o)
    return xb, Wb, packed_o, coarse_o


def test_full_vocab_pack_sampled(i2h, full_vocab_head):
    """The pack of the 248320-row head, bit-exact on sampled vocab rows."""
    xb, Wb, packed_o, _ = full_vocab_head
    p, S, ZS = i2h.pack(dev_bf16(Wb))
    pick = np.sort(np.random.default_rng(0).choice(Wb.shape[0], 4096, replace=False))
    assert np.array_equal(host(p)[pick], packed_o[0][pick])
    assert np.array_equal(host(S)[pick], packed_o[1][pick]) and np.array_equal(host(ZS)[pick], packed_o[2][pick])


# every row count of the full-vocabulary band (each takes a different kernel, chunking or split
# of the tail: the M = 1 kernel, the 16-, 32- and 64-row tiles, 64 + 8 rows; four blocks per
# thread in the tail, split over 16 workgroups per row at 4 rows and 4 at 16); every row is
# checked against the oracle
@pytest.mark.parametrize("M", [1, 2, 4, 8, 16, 32, 64, 72])
def test_full_vocab_top16(i2h, full_vocab_head, M):
    xb, Wb, packed_o, coarse_o = full_vocab_head
    say(f"full vocabulary M={M}")
    out = run_and_check(i2h, xb[:M], Wb, k=16, packed_o=packed_o, coarse_o=coarse_o[:M])
    say(f"  top-16 match vs oracle: {out['match']}/{out['places']}")


# ---------------------------------------------------------------------------------------------
# drop-in logits row: bit-exact
# ---------------------------------------------------------------------------------------------
_TDT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _logits_inputs(M, N, R, seed):
    g = np.random.default_rng(seed)
    y_bits = oracle.f32_to_bf16(g.normal(0, 4, (M, N)).astype(np.float32))
    sel = np.stack([g.choice(N, R, replace=False) for _ in range(M)]).astype(np.int32)
    sel[0, -3:] = -1                      # fewer than R reranked tokens in row 0
    ex = g.normal(0, 8, (M, R)).astype(np.float32)
    bias = g.normal(0, 2, N).astype(np.float32)
    return y_bits, sel, ex, bias


def _bias_args(bias, bias_dtype):
    if bias_dtype is None:
        return None, None
    t = torch.from_numpy(bias).to(_TDT[bias_dtype])
    ref = si.bits(t) if bias_dtype == "bf16" else t.numpy()
    return t.to(DEV), ref


@pytest.mark.parametrize("topk_only", [False, True])
@pytest.mark.parametrize("bias_dtype", [None, "bf16", "fp16", "fp32"])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp16", "fp32"])
def test_logits_row_bit_exact(i2h, topk_only, bias_dtype, out_dtype):
    M, N, R = 3, 4133, 32                 # N not a multiple of 8: rows start unaligned in the flat pass
    y_bits, sel, ex, bias = _logits_inputs(M, N, R, seed=11)
    bt, bref = _bias_args(bias, bias_dtype)
    say(f"logits topk={topk_only} bias={bias_dtype} out={out_dtype}")
    out = i2h.logits(None if topk_only else dev_bf16(y_bits), torch.from_numpy(sel).to(DEV),
                     torch.from_numpy(ex).to(DEV), topk_only=topk_only, bias=bt, out_dtype=_TDT[out_dtype],
                     out=torch.empty(M, N, dtype=_TDT[out_dtype], device=DEV))
    want = oracle.logits_row(y_bits, sel, ex, topk_only, bref, bias_dtype, out_dtype)
    got = host(out) if out_dtype != "fp16" else out.cpu().view(torch.int16).numpy().view(np.uint16)
    assert got.dtype == want.dtype and np.array_equal(got, want)


@pytest.mark.parametrize("topk_only", [False, True])
def test_logits_row_full_vocab_in_place(i2h, topk_only):
    """The draft-slot row (M = 1, N = 124160) and a full-vocab block (M = 4, N = 248320), written
    over the coarse row itself, with a bf16 bias."""
    for M, N in ((1, 124160), (4, 248320)):
        y_bits, sel, ex, bias = _logits_inputs(M, N, 32, seed=12 + M)
        bt, bref = _bias_args(bias, "bf16")
        y = dev_bf16(y_bits)
        out = i2h.logits(y, torch.from_numpy(sel).to(DEV), torch.from_numpy(ex).to(DEV), topk_only=topk_only,
                         bias=bt, out=y)
        assert out.data_ptr() == y.data_ptr()
        assert np.array_equal(host(out), oracle.logits_row(y_bits, sel, ex, topk_only, bref, "bf16", "bf16"))


# ---------------------------------------------------------------------------------------------
# FP8 e4m3 per-row-scale weight source: pack bit-exact; rerank within the fp32 accumulation bound
# ---------------------------------------------------------------------------------------------
def _fp8_degenerate_rows(K):
    return np.stack([np.zeros(K, np.uint8),                                  # all zero
                     np.full(K, 0x38, np.uint8),                             # constant 1.0
                     (np.arange(K) % 8 + 0x38).astype(np.uint8),             # all positive
                     (np.arange(K) % 5 + 0xB8).astype(np.uint8),             # all negative
                     np.where(np.arange(K) % 2 == 0, 0x7E, 0xFE).astype(np.uint8),  # +-448
                     np.where(np.arange(K) % 3 == 0, 0x01, 0x81).astype(np.uint8)])  # subnormal codes


@pytest.mark.parametrize("N,K", [(1000, 1024), (37, 5120)])
def test_pack_fp8_bit_exact(i2h, N, K):
    say(f"pack_fp8 N={N} K={K}")
    W8, scale = si.gen_weight_fp8(N, K, seed=200 + N)
    W8 = np.concatenate([W8.numpy(), _fp8_degenerate_rows(K)])
    scale = np.concatenate([scale.numpy(), np.array([1.0, 0.5, 2.0 ** -10, 3.0, 1e-3, 7.0], np.float32)])
    p, S, ZS = i2h.pack_fp8(torch.from_numpy(W8).to(DEV), torch.from_numpy(scale).to(DEV))
    po, So, ZSo = oracle.pack_fp8(W8, scale)
    assert np.array_equal(host(p), po)
    assert np.array_equal(host(S), So) and np.array_equal(host(ZS), ZSo)


def test_pack_fp8_strided_rows(i2h):
    K = 1024
    W8, scale = si.gen_weight_fp8(300, K + 64, seed=9)
    Wd = W8.to(DEV)[:, 24:24 + K]   # row stride K + 64 bytes, 24-byte offset (8-byte aligned)
    p, S, ZS = i2h.pack_fp8(Wd, scale.to(DEV))
    po, So, ZSo = oracle.pack_fp8(W8.numpy()[:, 24:24 + K], scale.numpy())
    assert np.array_equal(host(p), po) and np.array_equal(host(S), So) and np.array_equal(host(ZS), ZSo)


def _fp8_rerank_check(ex_g, x_bits, W8, scale, sel):
    """GPU fp32 dots against the fp64 dots of the same fp32 rows: within the fp32 accumulation
    bound K * 2^-23 * sum |x w|."""
    e = oracle.rerank_exact_fp8(x_bits, W8, scale, sel)
    ok = sel >= 0
    assert np.all(np.isneginf(ex_g[~ok]))
    xf = np.abs(oracle.bf16_to_f32(x_bits).astype(np.float64))
    for m, j in zip(*np.nonzero(ok)):
        row = np.abs(oracle.fp8_rows_f32(W8[sel[m, j]][None], scale[sel[m, j]][None])[0].astype(np.float64))
        bound = x_bits.shape[1] * 2.0 ** -23 * float(xf[m] @ row)
        assert abs(float(ex_g[m, j]) - e[m, j]) <= bound, (m, j)


def test_rerank_fp8(i2h):
    M, N, K, R = 3, 2000, 5120, 32
    x = si.gen_x(M, K, outliers=8, seed=31)
    W8, scale = si.gen_weight_fp8(N, K, seed=32)
    sel = si.gen_rows(M, R, N, seed=33).numpy()
    sel[0, 5] = -1
    sel[2, 7] = N + 3
    ex = i2h.rerank_fp8(x.to(DEV), W8.to(DEV), scale.to(DEV), torch.from_numpy(sel).to(DEV))
    sel_o = np.where(sel < N, sel, -1)
    _fp8_rerank_check(host(ex), si.bits(x), W8.numpy(), scale.numpy(), sel_o)


@pytest.mark.parametrize("M,N,kc,R,k", [(2, 124160, 8, 32, 1), (3, 5000, 8, 32, 16)])
def test_select_rerank_fused_fp8(i2h, M, N, kc, R, k):
    """The fused FP8 tail against select + rerank_fp8 + finalize (bit for bit) and the oracle."""
    K = 5120
    say(f"select_rerank_fp8 M={M} N={N}")
    sc = si.gen_scores(M, N, seed=N + 5).numpy()
    cs, ci = oracle.block_emit(sc.astype(np.float64), kc)
    want_sel = oracle.select_top_r(cs, ci, R)
    cs_d, ci_d = torch.from_numpy(cs.astype(np.float32)).to(DEV), torch.from_numpy(ci).to(DEV)
    x = si.gen_x(M, K, outliers=8, seed=34)
    W8, scale = si.gen_weight_fp8(N, K, seed=35)
    xd, W8d, sd = x.to(DEV), W8.to(DEV), scale.to(DEV)
    sel = i2h.select(cs_d, ci_d, kc, R)
    ex = i2h.rerank_fp8(xd, W8d, sd, sel)
    oi, ov = i2h.finalize(ex, sel, k)
    fi, fv, fsel, fex = i2h.select_rerank_topk_fp8(cs_d, ci_d, kc, R, xd, W8d, sd, k, want_sel=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(fsel), want_sel)
    assert torch.equal(fsel, sel) and torch.equal(fex, ex), "fused FP8 selection / exact scores differ"
    assert torch.equal(fi, oi) and torch.equal(fv, ov), "fused FP8 top-k differs"
    _fp8_rerank_check(host(fex), si.bits(x), W8.numpy(), scale.numpy(), host(fsel))


# ---------------------------------------------------------------------------------------------
# int4 head (KCAND = 1, the page's comparison point): pack bit-exact; coarse and head as the
# int2 head's parity rules
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("N,K", [(1000, 1024), (37, 5120), (5, 256)])
def test_pack4_bit_exact(i2h, N, K):
    say(f"pack4 N={N} K={K}")
    W = si.bits(si.gen_weight(N, K, seed=300 + N))
    W = np.concatenate([W, degenerate_rows(K)])
    p, S, ZS = i2h.pack4(dev_bf16(W))
    po, So, ZSo = oracle.pack4(W)
    assert np.array_equal(host(p), po)
    assert np.array_equal(host(S), So) and np.array_equal(host(ZS), ZSo)


def run_and_check4(i2h, xb, Wb, kc=1, R=32, k=1):
    x, W = dev_bf16(xb), dev_bf16(Wb)
    p, S, ZS = i2h.pack4(W)
    po, So, ZSo = oracle.pack4(Wb)
    assert np.array_equal(host(p), po) and np.array_equal(host(S), So) and np.array_equal(host(ZS), ZSo)
    xs = i2h.xsum(x)
    cs, ci, y = i2h.coarse4_topk(x, xs, p, S, ZS, kcand=kc, want_y=True)
    oi, ov, sel, ex = i2h.select_rerank_topk(cs, ci, kc, R, x, W, k, want_sel=True)
    torch.cuda.synchronize()
    g = dict(cs=cs, ci=ci, y=y, sel=sel, ex=ex, oi=oi, ov=ov)
    res = oracle.head4(xb, Wb, po, So, ZSo, kcand=kc, R=R, k=k)
    rows = np.arange(xb.shape[0])
    return check_path(g, res, rows, xb, Wb, kc, k, "int4 head", scales=(So, ZSo), fold=(1.0,))


@pytest.mark.parametrize("M,N,K,kc,R,k", [(1, 4096, 512, 1, 32, 1), (3, 4133, 5120, 1, 32, 1),
                                          (20, 2000, 1024, 8, 32, 16), (40, 1000, 512, 4, 16, 4),
                                          (1, 124160, 5120, 1, 32, 1)])
def test_int4_head_parity(i2h, M, N, K, kc, R, k):
    say(f"int4 head M={M} N={N} K={K} kc={kc} R={R} k={k}")
    xb = si.bits(si.gen_x(M, K, outliers=8 if K >= 1024 else 0, seed=M + K + 1))
    Wb = si.bits(si.gen_weight(N, K, seed=N + K + 1))
    run_and_check4(i2h, xb, Wb, kc=kc, R=R, k=k)


# ---------------------------------------------------------------------------------------------
# token-level selection over the coarse row: bit-exact indices
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("M,N,R,levels", [(3, 1000, 32, 0), (2, 37, 64, 0), (4, 4099, 32, 2), (2, 8191, 100, 1),
                                          (1, 124160, 32, 0), (2, 248320, 1024, 0), (2, 124160, 16, 3),
                                          (3, 9000, 1024, 1), (2, 16385, 32, 0), (3, 50001, 64, 2),
                                          (1, 124160, 1024, 1), (2, 248320, 512, 0)])
@pytest.mark.parametrize("chunked", [True, False])
def test_select_tokens_exact(i2h, M, N, R, levels, chunked):
    say(f"select_tokens M={M} N={N} R={R} levels={levels} chunked={chunked}")
    y = si.gen_coarse_row(M, N, seed=300 + N, levels=levels)
    sel = i2h.select_tokens(y.to(DEV), R, chunked=chunked)
    torch.cuda.synchronize()
    assert np.array_equal(host(sel), oracle.select_tokens(si.bits(y), R))


def test_select_tokens_all_ties_and_signed_zeros(i2h):
    say("select_tokens ties")
    y = np.zeros((3, 20000), np.uint16)
    y[1, ::2] = 0x8000                       # -0.0 and +0.0 interleaved: all equal
    y[2] = 0x3F80
    y[2, 19990:] = 0x4000                    # ten larger entries at the end, then ties
    want = oracle.select_tokens(y, 40)
    for chunked in (True, False):
        sel = i2h.select_tokens(dev_bf16(y), 40, chunked=chunked)
        torch.cuda.synchronize()
        assert np.array_equal(host(sel), want)


# ---------------------------------------------------------------------------------------------
# design alternatives (group 64, contiguous-4 bytes, dequantised weight tile): pack bit-exact,
# coarse candidates within the coarse tolerance of the oracle's variant
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("group,layout", [(128, "quarter"), (64, "quarter"), (128, "contiguous"), (64, "contiguous")])
@pytest.mark.parametrize("N,K", [(1000, 1024), (37, 5120), (300, 512)])
def test_pack_variant_bit_exact(i2h, group, layout, N, K):
    say(f"pack_variant G={group} {layout} N={N} K={K}")
    W = si.bits(si.gen_weight(N, K, seed=500 + N + group))
    W = np.concatenate([W, degenerate_rows(K)])
    p, S, ZS = i2h.pack_variant(dev_bf16(W), group, layout)
    torch.cuda.synchronize()
    po, So, ZSo = oracle.pack_variant(W, G=group, layout=layout)
    assert np.array_equal(host(p), po)
    assert np.array_equal(host(S), So) and np.array_equal(host(ZS), ZSo)


def variant_oracle(xb, p, S, ZS, group, layout, scaling):
    if scaling == "tile":
        assert layout == "quarter"
        return oracle.coarse_logits_tile(xb, p, S, ZS, group)
    if layout == "contiguous":
        return oracle.coarse_logits_contiguous4(xb, p, S, ZS, group)
    return oracle.coarse_logits(xb, p, S, ZS, group)


# the design and the three alternatives, each one property away from it
VARIANTS = [(128, "quarter", "accumulator"), (64, "quarter", "accumulator"), (128, "contiguous", "accumulator"),
            (128, "quarter", "tile")]


@pytest.mark.parametrize("group,layout,scaling", VARIANTS)
@pytest.mark.parametrize("M,N,K,kc,sums", [(1, 4096, 512, 8, "kernel"), (1, 3001, 5120, 8, "given"),
                                           (5, 1000, 512, 8, "kernel"), (3, 777, 5120, 16, "given"),
                                           (16, 2011, 5120, 4, "kernel")])
def test_coarse_variant(i2h, group, layout, scaling, M, N, K, kc, sums):
    """One row through the one-row kernel, more through the 16-row tile; the group sums of x taken
    in the kernel or given (the weight tile takes none)."""
    say(f"coarse_variant G={group} {layout} {scaling} M={M} N={N} K={K} kc={kc} sums={sums}")
    xb = si.bits(si.gen_x(M, K, outliers=8 if K >= 1024 else 0, seed=600 + M + K))
    Wb = si.bits(si.gen_weight(N, K, seed=700 + N + K))
    p, S, ZS = oracle.pack_variant(Wb, G=group, layout=layout)
    x = dev_bf16(xb)
    xs = i2h.xsum_group(x, group) if scaling == "accumulator" and sums == "given" else None
    cs, ci = i2h.coarse_variant_topk(x, xs, torch.from_numpy(p).to(DEV), dev_bf16(S), dev_bf16(ZS), group, layout,
                                     scaling, kc)
    torch.cuda.synchronize()
    c = variant_oracle(xb, p, S, ZS, group, layout, scaling)
    pu.check_candidates(host(cs), host(ci), c, kc)


def test_coarse_variant_rejects_two_changes(i2h):
    """Group 64 with the contiguous layout changes two properties at once: not a measured form."""
    x = torch.zeros(1, 512, dtype=torch.bfloat16, device=DEV)
    p = torch.zeros(64, 128, dtype=torch.uint8, device=DEV)
    S = torch.zeros(64, 8, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError):
        i2h.coarse_variant_topk(x, None, p, S, S, 64, "contiguous", "accumulator", 8)


@pytest.mark.parametrize("group,layout,scaling", VARIANTS[1:])
@pytest.mark.parametrize("M", [1, 16])
def test_coarse_variant_full_vocab_slice(i2h, group, layout, scaling, M):
    """The workload's head (N = 124160, K = 5120) in each alternative, packed on the GPU (bit-exact
    against the oracle's pack), at one row and at 16."""
    N, K, kc = 124160, 5120, 8
    say(f"coarse_variant full size G={group} {layout} {scaling} M={M}")
    xb = si.bits(si.gen_x(M, K, outliers=8, seed=800 + M))
    Wb = si.bits(si.gen_weight(N, K, seed=801))
    W = dev_bf16(Wb)
    pg, Sg, ZSg = i2h.pack_variant(W, group, layout)
    x = dev_bf16(xb)
    cs, ci = i2h.coarse_variant_topk(x, None, pg, Sg, ZSg, group, layout, scaling, kc)
    torch.cuda.synchronize()
    p, S, ZS = oracle.pack_variant(Wb, G=group, layout=layout)
    assert np.array_equal(host(pg), p) and np.array_equal(host(Sg), S) and np.array_equal(host(ZSg), ZS)
    pu.check_candidates(host(cs), host(ci), variant_oracle(xb, p, S, ZS, group, layout, scaling), kc)
