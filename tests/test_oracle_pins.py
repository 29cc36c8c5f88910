"""Pins of the oracle against what the page and mathematics fix (CPU only).

Each test names the property it pins. None of them re-types an oracle formula: they use values
worked by hand (tests/golden), exact constructions whose result is known in closed form, brute
force on small inputs with exact (fractions / fsum) arithmetic, library routines for special
cases, and invariants any correct implementation must satisfy.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from conftest import read_golden


def hexs(s):
    return [int(t, 16) for t in s.split()]


def f32(b):
    return float(np.uint32(b).view(np.float32))


def bf(b):
    return float(np.uint32(int(b) << 16).view(np.float32))


# ---------------------------------------------------------------------------------------------
# bf16 rounding: hand-worked values and the library cast
# ---------------------------------------------------------------------------------------------
def test_bf16_rounding_hand_values():
    _, rows = read_golden("bf16_rounding.txt")
    src = np.array([int(r[0], 16) for r in rows], dtype=np.uint32).view(np.float32)
    want = [int(r[1], 16) for r in rows]
    assert list(oracle.f32_to_bf16(src)) == want


def test_bf16_rounding_matches_torch_cast():
    g = torch.Generator().manual_seed(5)
    a = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 8)
    # force exact halves and near halves
    u = a.view(torch.int32)
    u[:1000] = (u[:1000] & ~0xFFFF) | 0x8000
    u[1000:2000] = (u[1000:2000] & ~0xFFFF) | 0x7FFF
    want = a.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.f32_to_bf16(a.numpy())
    assert np.array_equal(got, want)
    back = oracle.bf16_to_f32(want)
    assert np.array_equal(back, a.to(torch.bfloat16).float().numpy())


# ---------------------------------------------------------------------------------------------
# P-2: pack worked example, round trip, dequant bit pattern
# ---------------------------------------------------------------------------------------------
def test_pack_worked_example():
    kv, _ = read_golden("pack_worked_example.txt")
    q = np.array([[int(t) for t in kv["q"].split()]], dtype=np.uint8)
    packed = oracle.pack_quarter_split(q)
    assert list(packed[0]) == hexs(kv["packed"])
    assert np.array_equal(oracle.unpack_quarter_split(packed), q)


def test_pack_round_trip_random():
    rng = np.random.default_rng(0)
    q = rng.integers(0, 4, size=(37, 2048), dtype=np.uint8)
    p = oracle.pack_quarter_split(q)
    assert p.shape == (37, 512)
    assert np.array_equal(oracle.unpack_quarter_split(p), q)


def test_dequant_bit_pattern_identity_exhaustive():
    """P-1. The page's bit-pattern dequant: for every byte b and quarter t, the 16-bit pattern
    0x3F80 | ((b << (5 - 2t)) & 0x60) (t < 3), ((b >> 1) & 0x60) | 0x3F80 (t = 3) is the bf16
    value 1 + ((b >> 2t) & 3) / 4. The HIP coarse kernel relies on it; the worked byte is in
    the golden file."""
    kv, _ = read_golden("pack_worked_example.txt")
    for b in range(256):
        for t in range(4):
            pat = (0x3F80 | ((b << (5 - 2 * t)) & 0x60)) if t < 3 else (((b >> 1) & 0x60) | 0x3F80)
            assert bf(pat) == 1.0 + ((b >> (2 * t)) & 3) / 4.0
    pats = [(0x3F80 | ((0x9C << (5 - 2 * t)) & 0x60)) if t < 3 else (((0x9C >> 1) & 0x60) | 0x3F80)
            for t in range(4)]
    assert pats == hexs(kv["dequant_9C"])


# ---------------------------------------------------------------------------------------------
# Quantiser: hand-worked group, degenerate group, invariants
# ---------------------------------------------------------------------------------------------
def test_quantize_hand_group():
    kv, _ = read_golden("quantize_group_example.txt")
    head = hexs(kv["w_head"])
    w = np.array(head + [0] * int(kv["w_tail_zeros"]), dtype=np.uint16)[None, :]
    w = np.concatenate([w, np.zeros((1, 384), np.uint16)], axis=1)  # K = 512
    q, sc, zp = oracle.quantize(w)
    assert float(sc[0, 0]) == float(kv["sc"]) and float(zp[0, 0]) == float(kv["zp"])
    assert list(q[0, :5]) == [int(t) for t in kv["q_head"].split()]
    assert np.all(q[0, 5:128] == int(kv["q_tail"]))
    S, ZS = oracle.premultiplied_scales(sc, zp)
    assert S[0, 0] == int(kv["S"], 16) and ZS[0, 0] == int(kv["ZS"], 16)


def test_quantize_constant_group():
    kv, _ = read_golden("quantize_group_example.txt")
    w = np.full((1, 512), int(kv["const_w"], 16), dtype=np.uint16)
    q, sc, zp = oracle.quantize(w)
    assert sc[0, 0].view(np.uint32) == int(kv["const_sc_bits"], 16)
    assert float(zp[0, 0]) == float(kv["const_zp"]) and np.all(q[0, :128] == int(kv["const_q"]))
    S, ZS = oracle.premultiplied_scales(sc, zp)
    assert S[0, 0] == int(kv["const_S"], 16) and ZS[0, 0] == int(kv["const_ZS"], 16)


def test_quantize_invariants_random():
    """P-4. Codes and zero points in {0..3}; each code is the nearest grid point (and the zero
    point the nearest integer) away from exact ties; sc is the correctly rounded (hi - lo)/3;
    reconstruction error within sc (1/2 + 2^-20) when the group straddles zero."""
    W = si.bits(si.gen_weight(96, 1024, seed=77))
    q, sc, zp = oracle.quantize(W)
    assert q.max() <= 3 and zp.min() >= 0 and zp.max() <= 3
    w = oracle.bf16_to_f32(W).astype(np.float64).reshape(96, 8, 128)
    lo, hi = w.min(2), w.max(2)
    # correctly rounded division: within half an ulp of the exact quotient
    for n in range(0, 96, 7):
        for g in range(8):
            exact = (Fraction(float(hi[n, g])) - Fraction(float(lo[n, g]))) / 3
            ulp = Fraction(2) ** (math.frexp(float(sc[n, g]))[1] - 24)
            assert abs(Fraction(float(sc[n, g])) - exact) <= ulp / 2
    s = sc.astype(np.float64)[:, :, None]
    z = zp.astype(np.float64)[:, :, None]
    t = w / s + z
    qq = q.reshape(96, 8, 128).astype(np.float64)
    grid = np.arange(4.0)
    dist = np.abs(t[..., None] - grid)
    best = dist.argmin(-1)
    second = np.sort(dist, -1)[..., 1]
    clear = (second - dist.min(-1)) > 1e-5
    assert np.array_equal(qq[clear], best[clear])
    zt = -lo / sc.astype(np.float64)
    zd = np.abs(zt[..., None] - grid)
    zclear = (np.sort(zd, -1)[..., 1] - zd.min(-1)) > 1e-5
    assert np.array_equal(zp[zclear], zd.argmin(-1)[zclear])
    straddle = ((lo <= 0) & (hi >= 0))[:, :, None]
    err = np.abs(w - s * (qq - z))
    assert np.all(np.where(straddle, err <= s * (0.5 + 2.0 ** -20), True))


def test_premultiplied_scales_properties():
    """S is the bf16 nearest to 4 sc; ZS is within one bf16 ulp (plus an fp32 rounding) of
    (4 + zp) sc."""
    W = si.bits(si.gen_weight(64, 512, seed=78))
    q, sc, zp = oracle.quantize(W)
    S, ZS = oracle.premultiplied_scales(sc, zp)
    s4 = 4.0 * sc.astype(np.float64)  # exact: a power-of-two multiple
    for s_bits, v in zip(S.ravel(), s4.ravel()):
        d = abs(bf(s_bits) - v)
        dn, up = abs(bf(int(s_bits) - 1) - v), abs(bf(int(s_bits) + 1) - v)
        assert d <= dn and d <= up
        if d == dn or d == up:
            assert int(s_bits) % 2 == 0  # exact half: the even neighbour
    zs = (4.0 + zp.astype(np.float64)) * sc.astype(np.float64)
    ZSf = oracle.bf16_to_f32(ZS).astype(np.float64)
    half_ulp = np.ldexp(1.0, np.frexp(ZSf)[1] - 9)  # bf16 keeps 8 significant bits
    assert np.all(np.abs(ZSf - zs) <= half_ulp + zs * 2.0 ** -22)


def test_quantize_matches_eager_fp32_ops():
    """Cross-check (not a pin): the page quantises with eager torch fp32 ops; running that
    sequence of library ops on the CPU must give the same bits."""
    W = si.gen_weight(300, 1024, seed=79)
    w = W.float().reshape(300, 8, 128)
    lo, hi = w.amin(2), w.amax(2)
    sc = ((hi - lo) / 3).clamp(min=1e-8)
    zp = torch.round(-lo / sc).clamp(0, 3)
    qt = torch.round(w / sc[:, :, None] + zp[:, :, None]).clamp(0, 3).to(torch.uint8).reshape(300, 1024)
    S = (4.0 * sc).to(torch.bfloat16)
    ZS = (4.0 * sc + zp * sc).to(torch.bfloat16)
    q, sco, zpo = oracle.quantize(si.bits(W))
    So, ZSo = oracle.premultiplied_scales(sco, zpo)
    assert np.array_equal(q, qt.numpy())
    assert np.array_equal(So, si.bits(S)) and np.array_equal(ZSo, si.bits(ZS))


# ---------------------------------------------------------------------------------------------
# P-3: a head on the exact int2 grid: the coarse logits are the exact bf16 logits
# ---------------------------------------------------------------------------------------------
def grid_head(N, K, seed):
    """W whose every group is sc * (q - zp) with sc a power of two and both q = 0 and q = 3
    present, so the quantiser must recover q, zp and sc exactly and S (1 + v/4) - ZS = W."""
    rng = np.random.default_rng(seed)
    G = 128
    ng = K // G
    q = rng.integers(0, 4, size=(N, K)).astype(np.int64)
    qg = q.reshape(N, ng, G)
    qg[:, :, 0] = 0
    qg[:, :, 1] = 3
    zp = rng.integers(0, 4, size=(N, ng))
    e = rng.integers(-12, -3, size=(N, ng))
    sc = np.ldexp(1.0, e)
    w = (sc[:, :, None] * (qg - zp[:, :, None])).reshape(N, K)
    Wb = oracle.f32_to_bf16(w.astype(np.float32))
    assert np.array_equal(oracle.bf16_to_f32(Wb).astype(np.float64), w)  # exact in bf16
    return Wb, q.reshape(N, K), zp, sc


def test_exact_grid_head_recovers_codes_and_logits():
    N, K = 200, 1024
    Wb, q, zp, sc = grid_head(N, K, 3)
    qo, sco, zpo = oracle.quantize(Wb)
    assert np.array_equal(qo, q) and np.array_equal(zpo, zp) and np.array_equal(sco, sc)
    packed, S, ZS = oracle.pack(Wb)
    # S and ZS are the exact values 4 sc and (4 + zp) sc
    assert np.array_equal(oracle.bf16_to_f32(S).astype(np.float64), 4 * sc)
    assert np.array_equal(oracle.bf16_to_f32(ZS).astype(np.float64), (4 + zp) * sc)
    x = si.bits(si.gen_x(3, K, seed=9))
    c = oracle.coarse_logits(x, packed, S, ZS)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(Wb).astype(np.float64)
    for m in range(3):
        for n in range(0, N, 13):
            want = math.fsum(xf[m] * wf[n])  # exact products, correctly rounded sum
            bound = K * 2.0 ** -52 * np.sum(np.abs(xf[m] * wf[n]))
            assert abs(c[m, n] - want) <= bound


def test_bias_fold_grouped_form_equals_per_weight_form():
    """The page's identity: each group contributes S * sum x (1 + v/4) - ZS * sum x. Evaluated
    exactly (fractions) on a small head, it equals the oracle's per-weight form."""
    N, K = 5, 512
    W = si.bits(si.gen_weight(N, K, seed=80))
    packed, S, ZS = oracle.pack(W)
    x = si.bits(si.gen_x(2, K, seed=10))
    c = oracle.coarse_logits(x, packed, S, ZS)
    xf = [[Fraction(float(v)) for v in row] for row in oracle.bf16_to_f32(x)]
    Q = K // 4
    for m in range(2):
        for n in range(N):
            tot = Fraction(0)
            for g in range(K // 128):
                s = Fraction(bf(S[n, g]))
                zs = Fraction(bf(ZS[n, g]))
                p = Fraction(0)
                sx = Fraction(0)
                for k in range(g * 128, g * 128 + 128):
                    t, j = divmod(k, Q)
                    v = (int(packed[n, j]) >> (2 * t)) & 3
                    p += xf[m][k] * (1 + Fraction(v, 4))
                    sx += xf[m][k]
                tot += s * p - zs * sx
            assert abs(float(tot) - c[m, n]) <= 1e-12 * max(1.0, abs(float(tot)))


# ---------------------------------------------------------------------------------------------
# a3: group sums
# ---------------------------------------------------------------------------------------------
def test_group_sums_against_fsum():
    x = si.bits(si.gen_x(4, 1024, outliers=8, seed=11))
    xs = oracle.group_sums(x)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    for m in range(4):
        for g in range(8):
            assert xs[m, g] == pytest.approx(math.fsum(xf[m, g * 128:(g + 1) * 128]), abs=1e-12)


# ---------------------------------------------------------------------------------------------
# P-7 / P-8: emit and select are sorts; brute force with Python sorted() on small inputs
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("N,kc", [(256, 8), (200, 8), (131, 3), (70, 16), (64, 64), (65, 1)])
def test_block_emit_brute_force(N, kc):
    rng = np.random.default_rng(N + kc)
    c = rng.integers(-4, 5, size=(3, N)).astype(np.float64) * 0.5  # many exact ties
    s, i = oracle.block_emit(c, kc)
    nblk = (N + 63) // 64
    assert s.shape == (3, nblk * kc)
    for m in range(3):
        for b in range(nblk):
            cols = list(range(64 * b, min(N, 64 * b + 64)))
            best = sorted(cols, key=lambda n: (-c[m, n], n))[:kc]
            want = best + [-1] * (kc - len(best))
            assert list(i[m, b * kc:(b + 1) * kc]) == want
            for r, n in enumerate(want):
                assert s[m, b * kc + r] == (c[m, n] if n >= 0 else -np.inf)


@pytest.mark.parametrize("R", [1, 5, 32, 100])
def test_select_brute_force(R):
    rng = np.random.default_rng(R)
    c = rng.integers(-6, 7, size=(4, 700)).astype(np.float64)
    s, i = oracle.block_emit(c, 4)
    sel = oracle.select_top_r(s, i, R)
    for m in range(4):
        pool = [(s[m, t], i[m, t]) for t in range(s.shape[1]) if i[m, t] >= 0]
        want = [n for _, n in sorted(pool, key=lambda p: (-p[0], p[1]))[:R]]
        assert list(sel[m, :len(want)]) == want
        assert all(v == -1 for v in sel[m, len(want):])


def test_select_is_top_r_of_all_candidates_with_ties():
    """All-equal scores (x = 0 gives this): the R smallest candidate token indices win."""
    c = np.zeros((1, 1000))
    s, i = oracle.block_emit(c, 8)
    sel = oracle.select_top_r(s, i, 32)
    want = sorted(int(t) for t in i[0] if t >= 0)[:32]
    assert list(sel[0]) == want


# ---------------------------------------------------------------------------------------------
# P-9: rerank is the exact dot; finalize is a sort
# ---------------------------------------------------------------------------------------------
def test_rerank_against_fsum():
    K, N = 1024, 300
    x = si.bits(si.gen_x(2, K, outliers=8, seed=13))
    W = si.bits(si.gen_weight(N, K, seed=81))
    sel = si.gen_rows(2, 17, N, seed=14).numpy()
    sel[1, 3] = -1
    e = oracle.rerank_exact(x, W, sel)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(W).astype(np.float64)
    for m in range(2):
        for j in range(17):
            if sel[m, j] < 0:
                assert e[m, j] == -np.inf
                continue
            prods = xf[m] * wf[sel[m, j]]
            assert abs(e[m, j] - math.fsum(prods)) <= K * 2.0 ** -52 * np.abs(prods).sum()


def test_finalize_brute_force():
    rng = np.random.default_rng(2)
    e = rng.integers(-3, 4, size=(5, 32)).astype(np.float64)
    sel = np.stack([rng.permutation(1000)[:32] for _ in range(5)]).astype(np.int32)
    sel[0, 5] = -1
    e[0, 5] = -np.inf
    for k in (1, 16, 32):
        oi, ov = oracle.finalize(e, sel, k)
        for m in range(5):
            pool = [(e[m, j], sel[m, j]) for j in range(32) if sel[m, j] >= 0]
            want = sorted(pool, key=lambda p: (-p[0], p[1]))[:k]
            assert list(oi[m, :len(want)]) == [n for _, n in want]
            assert list(ov[m, :len(want)]) == [v for v, _ in want]


# ---------------------------------------------------------------------------------------------
# P-5 / P-6: settings where the method must reduce to the exact bf16 head
# ---------------------------------------------------------------------------------------------
def brute_topk(ex, k):
    return [sorted(range(ex.shape[1]), key=lambda n: (-ex[m, n], n))[:k] for m in range(ex.shape[0])]


def test_all_tokens_reranked_equals_brute_force():
    """P-5. With KCAND = BLOCK_N and R = N every token is reranked exactly, so argmax and
    top-16 are those of the dense bf16 head."""
    N, K = 256, 512
    W = si.bits(si.gen_weight(N, K, seed=82))
    x = si.bits(si.gen_x(3, K, seed=15))
    packed, S, ZS = oracle.pack(W)
    ex = oracle.exact_logits(x, W)
    for k in (1, 16):
        r = oracle.head(x, W, packed, S, ZS, kcand=64, R=N, k=k)
        want = brute_topk(ex, k)
        for m in range(3):
            assert list(r["idx"][m]) == want[m]
            assert np.allclose(r["val"][m], ex[m, want[m]], rtol=0, atol=1e-12)


def test_planted_winner_is_found():
    """P-6. A token whose exact logit beats every other by far more than the coarse error
    must be the argmax, and must head the top-16."""
    N, K = 4096, 512
    W = si.gen_weight(N, K, seed=83)
    x = si.gen_x(2, K, seed=16)
    for m, t in enumerate((1234, 4095)):
        W[t] = (x[m].float() * 0.05).to(torch.bfloat16)
    Wb, xb = si.bits(W), si.bits(x)
    packed, S, ZS = oracle.pack(Wb)
    r = oracle.head(xb, Wb, packed, S, ZS, k=16)
    assert list(r["idx"][:, 0]) == [1234, 4095]


def test_in_set_invariant_and_recall():
    """P-6. Whenever the dense argmax is among the reranked tokens, the method returns it."""
    N, K = 4096, 512
    W = si.bits(si.gen_weight(N, K, seed=84))
    x = si.bits(si.gen_x(64, K, seed=17))
    packed, S, ZS = oracle.pack(W)
    r = oracle.head(x, W, packed, S, ZS)
    ex = oracle.exact_logits(x, W)
    win = ex.argmax(1)
    hits = 0
    for m in range(64):
        if win[m] in set(r["sel"][m]):
            hits += 1
            assert r["idx"][m, 0] == win[m]
    assert hits == int((r["idx"][:, 0] == win).sum())
    assert hits >= 48  # recall is high but not exact on Gaussian data (reported, not pinned)


def test_zero_input_row_tie_rules():
    """x = 0: every coarse and exact score is 0, so every choice falls to the tie rules: the
    four lowest blocks' first eight columns are selected and token 0 wins."""
    N, K = 4096, 512
    W = si.bits(si.gen_weight(N, K, seed=85))
    packed, S, ZS = oracle.pack(W)
    x = np.zeros((1, K), dtype=np.uint16)
    r = oracle.head(x, W, packed, S, ZS, k=16)
    want_sel = [b * 64 + j for b in range(4) for j in range(8)]
    assert list(r["sel"][0]) == want_sel
    assert list(r["idx"][0]) == want_sel[:16]


# ---------------------------------------------------------------------------------------------
# P-10: sizes the page prints; shape rule
# ---------------------------------------------------------------------------------------------
def test_storage_bytes_match_page():
    kv, _ = read_golden("storage_bytes.txt")
    b = oracle.storage_bytes(int(kv["N"]), int(kv["K"]))
    assert b["int2_total"] == 178_790_400
    assert round(b["int2_total"] / 2 ** 30, 3) == float(kv["int2_head_gib"])
    assert round(b["bf16_weight"] / 2 ** 30, 2) == float(kv["bf16_head_gib"])
    assert round(b["packed"] / 2 ** 20) == int(kv["int2_packed_mib"])


def test_shape_rule():
    oracle.check_shape(512)
    oracle.check_shape(5120)
    for K in (0, 256, 640, 5000):
        with pytest.raises(ValueError):
            oracle.check_shape(K)


# ---------------------------------------------------------------------------------------------
# Drop-in logits row (radiance_drafthead.py, _apply_head_int2: write-back of the exact scores,
# embedding bias, head dtype).
# ---------------------------------------------------------------------------------------------
def _bf(vals):
    return oracle.f32_to_bf16(np.asarray(vals, dtype=np.float32)).reshape(1, -1)


def test_logits_row_hand_example():
    """Worked by hand: y = [1, 2, -3, 0.5], tokens 2 and 0 reranked to 7.25 and 0.1."""
    y = _bf([1.0, 2.0, -3.0, 0.5])
    sel = np.array([[2, 0]], np.int32)
    ex = np.array([[7.25, 0.1]], np.float32)
    b01 = 0.10009765625                        # bf16(0.1) = 0x3DCD
    out = oracle.bf16_to_f32(oracle.logits_row(y, sel, ex, topk_only=False))
    assert out.tolist() == [[b01, 2.0, 7.25, 0.5]]
    out = oracle.bf16_to_f32(oracle.logits_row(y, sel, ex, topk_only=True))
    assert out.tolist() == [[b01, -math.inf, 7.25, -math.inf]]
    # bf16 bias: each sum is rounded back to bf16 (0.6000977 -> 0.6015625; 2 + 2^-8 -> 2)
    bias = _bf([0.5, 2.0 ** -8, 1.0, -0.5])[0]
    out = oracle.bf16_to_f32(oracle.logits_row(y, sel, ex, False, bias, "bf16"))
    assert out.tolist() == [[0.6015625, 2.0, 8.25, 0.0]]
    # fp32 bias: the row becomes fp32 and keeps the exact sums
    out = oracle.logits_row(y, sel, ex, False, np.array([0.5, 2.0 ** -8, 1.0, -0.5], np.float32), "fp32", "fp32")
    assert out.tolist() == [[b01 + 0.5, 2.0 + 2.0 ** -8, 8.25, 0.0]]


def test_logits_row_rejects_tokens_outside_the_row():
    """The write-back is a scatter over the row: -1 marks an empty slot, anything else outside
    [0, N) is an error, not a skipped entry."""
    y = _bf([1.0, 2.0, -3.0, 0.5])
    ex = np.array([[7.25, 0.1]], np.float32)
    assert oracle.logits_row(y, np.array([[-1, 3]], np.int32), ex, False).shape == (1, 4)
    for bad in ([[4, 0]], [[0, -2]], [[2, 11]]):
        with pytest.raises(ValueError):
            oracle.logits_row(y, np.array(bad, np.int32), ex, False)
        with pytest.raises(ValueError):
            oracle.logits_row(y, np.array(bad, np.int32), ex, True)


def test_logits_row_rounding_ties():
    """Half-way sums round to the even neighbour: bf16 at 1 + 2^-8 and 1 + 3*2^-8 (spacing 2^-7),
    fp16 at 1 + 3*2^-11 (spacing 2^-10)."""
    sel = np.full((1, 1), -1, np.int32)
    ex = np.zeros((1, 1), np.float32)
    y = _bf([1.0, 1.0078125])
    out = oracle.bf16_to_f32(oracle.logits_row(y, sel, ex, False, _bf([2.0 ** -8, 2.0 ** -8])[0], "bf16"))
    assert out.tolist() == [[1.0, 1.015625]]
    y = _bf([1.0, 1.0])
    out = oracle.logits_row(y, sel, ex, False, np.array([3 * 2.0 ** -11, 2.0 ** -11], np.float16), "fp16", "fp16")
    assert out.view(np.float16).astype(np.float64).tolist() == [[1.0 + 2.0 ** -9, 1.0]]


@pytest.mark.parametrize("topk_only", [False, True])
@pytest.mark.parametrize("bias_dtype", [None, "bf16", "fp16", "fp32"])
@pytest.mark.parametrize("out_dtype", ["bf16", "fp16", "fp32"])
def test_logits_row_matches_eager_torch_steps(topk_only, bias_dtype, out_dtype):
    """The page's steps as eager torch CPU ops (fill, scatter of ex.to(bf16), + bias with torch's
    type promotion, .to(head dtype)) on random rows."""
    g = np.random.default_rng(5)
    M, N, R = 3, 257, 7
    y_bits = oracle.f32_to_bf16(g.normal(0, 4, (M, N)).astype(np.float32))
    sel = np.stack([g.choice(N, R, replace=False) for _ in range(M)]).astype(np.int32)
    sel[1, -2:] = -1
    ex = g.normal(0, 8, (M, R)).astype(np.float32)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
    bias_np, bias_t = None, None
    if bias_dtype is not None:
        b = g.normal(0, 2, N).astype(np.float32)
        bias_t = torch.from_numpy(b).to(tdt[bias_dtype])
        bias_np = oracle.f32_to_bf16(b) if bias_dtype == "bf16" else b.astype(np.float16 if bias_dtype == "fp16" else np.float32)
    got = oracle.logits_row(y_bits, sel, ex, topk_only, bias_np, bias_dtype, out_dtype)
    y = torch.from_numpy(y_bits.astype(np.int16)).view(torch.bfloat16).clone()
    if topk_only:
        y.fill_(float("-inf"))
    for m in range(M):
        ok = sel[m] >= 0
        y[m].scatter_(0, torch.from_numpy(sel[m][ok]).long(), torch.from_numpy(ex[m][ok]).to(torch.bfloat16))
    if bias_t is not None:
        y = y + bias_t
    y = y.to(tdt[out_dtype])
    want = y.view(torch.int16).numpy().view(np.uint16) if out_dtype != "fp32" else y.numpy()
    assert got.dtype == want.dtype and np.array_equal(got, want)


# ---------------------------------------------------------------------------------------------
# FP8 e4m3 weight source (radiance_drafthead.py, _rerank_exact FP8 branch; _quantize_head_now)
# ---------------------------------------------------------------------------------------------
def test_fp8_decode_hand_values():
    """1.0 = 0x38, the smallest subnormal 2^-9 = 0x01, the smallest normal 2^-6 = 0x08, the
    largest finite 448 = 0x7E, -1.0 = 0xB8; the page's formula reads 0x7F (a NaN code of e4m3fn)
    as 480."""
    got = oracle.fp8_e4m3_decode(np.array([0x38, 0x01, 0x08, 0x7E, 0xB8, 0x00, 0x7F], np.uint8))
    assert got.tolist() == [1.0, 2.0 ** -9, 2.0 ** -6, 448.0, -1.0, 0.0, 480.0]


def test_fp8_decode_matches_torch_e4m3fn():
    """Every byte except the two NaN codes against torch's float8_e4m3fn -> float32 conversion."""
    b = np.arange(256, dtype=np.uint8)
    ok = (b & 0x7F) != 0x7F
    t = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(oracle.fp8_e4m3_decode(b)[ok], t[ok])


def test_fp8_rerank_against_fsum():
    K, N = 1024, 200
    x = si.bits(si.gen_x(2, K, outliers=8, seed=15))
    W8, sc = si.gen_weight_fp8(N, K, seed=83)
    sel = si.gen_rows(2, 11, N, seed=16).numpy()
    sel[0, 2] = -1
    e = oracle.rerank_exact_fp8(x, W8.numpy(), sc.numpy(), sel)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    rows = (W8.view(torch.float8_e4m3fn).float() * sc[:, None]).numpy().astype(np.float64)  # torch fp32 ops
    for m in range(2):
        for j in range(11):
            if sel[m, j] < 0:
                assert e[m, j] == -np.inf
                continue
            prods = xf[m] * rows[sel[m, j]]
            assert abs(e[m, j] - math.fsum(prods)) <= K * 2.0 ** -52 * np.abs(prods).sum()


def test_fp8_quantize_matches_eager_fp32_ops():
    """Cross-check: the page's quantiser as eager torch fp32 ops on the FP8 head's fp32 rows
    (torch's e4m3fn decode times the row scale)."""
    W8, scale = si.gen_weight_fp8(300, 1024, seed=84)
    w = (W8.view(torch.float8_e4m3fn).float() * scale[:, None]).reshape(300, 8, 128)
    lo, hi = w.amin(2), w.amax(2)
    sc = ((hi - lo) / 3).clamp(min=1e-8)
    zp = torch.round(-lo / sc).clamp(0, 3)
    qt = torch.round(w / sc[:, :, None] + zp[:, :, None]).clamp(0, 3).to(torch.uint8).reshape(300, 1024)
    S = (4.0 * sc).to(torch.bfloat16)
    ZS = (4.0 * sc + zp * sc).to(torch.bfloat16)
    q, sco, zpo = oracle.quantize_fp8(W8.numpy(), scale.numpy())
    So, ZSo = oracle.premultiplied_scales(sco, zpo)
    assert np.array_equal(q, qt.numpy())
    assert np.array_equal(So, si.bits(S)) and np.array_equal(ZSo, si.bits(ZS))


def test_pack_fp8_hand_example():
    """The hand-worked FP8 row (tests/golden/fp8_pack_example.txt): subnormal codes, a zero point
    clamped from -1 to 0, a code clamped from 4 to 3, both half-way codes rounded to even."""
    kv, _ = read_golden("fp8_pack_example.txt")
    row = np.concatenate([np.tile(np.array(hexs(kv[f"pattern{t}"]), np.uint8), 32) for t in range(4)])
    packed, S, ZS = oracle.pack_fp8(row[None, :], np.array([float(kv["scale"])], np.float32))
    assert packed.shape == (1, 128)
    assert packed[0].tolist() == hexs(kv["packed_pattern"]) * 32
    assert S[0].tolist() == hexs(kv["S"]) and ZS[0].tolist() == hexs(kv["ZS"])


def test_pack_fp8_matches_eager_torch_chain():
    """The whole FP8 pack as eager torch ops: the e4m3fn decode times the row scale (fp32), the
    quantiser, the bias-4 premultiply and the quarter-split bytes assembled by shifts."""
    N, K = 260, 1024
    W8, scale = si.gen_weight_fp8(N, K, seed=88)
    w = (W8.view(torch.float8_e4m3fn).float() * scale[:, None]).reshape(N, K // 128, 128)
    lo, hi = w.amin(2), w.amax(2)
    sc = ((hi - lo) / 3).clamp(min=1e-8)
    zp = torch.round(-lo / sc).clamp(0, 3)
    q = torch.round(w / sc[:, :, None] + zp[:, :, None]).clamp(0, 3).to(torch.uint8).reshape(N, K)
    Q = K // 4
    packed = q[:, :Q] | (q[:, Q:2 * Q] << 2) | (q[:, 2 * Q:3 * Q] << 4) | (q[:, 3 * Q:] << 6)
    S = (4.0 * sc).to(torch.bfloat16)
    ZS = (4.0 * sc + zp * sc).to(torch.bfloat16)
    po, So, ZSo = oracle.pack_fp8(W8.numpy(), scale.numpy())
    assert np.array_equal(po, packed.numpy())
    assert np.array_equal(So, si.bits(S)) and np.array_equal(ZSo, si.bits(ZS))


# ---------------------------------------------------------------------------------------------
# int4 head (radiance_drafthead.py, _quantize_head_now BITS = 4: codes 0..15, half-split bytes,
# bias 16)
# ---------------------------------------------------------------------------------------------
def test_pack_half_split_worked_example():
    """By hand: K = 8, q = [1 2 15 0 | 3 4 5 6]: byte j = q[j] | q[4 + j] << 4."""
    q = np.array([[1, 2, 15, 0, 3, 4, 5, 6]], np.uint8)
    assert oracle.pack_half_split(q).tolist() == [[0x31, 0x42, 0x5F, 0x60]]
    assert np.array_equal(oracle.unpack_half_split(oracle.pack_half_split(q)), q)


def test_pack_half_split_round_trip_random():
    q = np.random.default_rng(3).integers(0, 16, (7, 512)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_half_split(oracle.pack_half_split(q)), q)


def grid_head4(N, K, seed):
    """W whose every group is sc * (q - zp) with sc a power of two, q in 0..15 with 0 and 15
    present, zp in 0..15: exact in bf16, so the 4-bit quantiser must recover q, zp and sc."""
    rng = np.random.default_rng(seed)
    G = 128
    ng = K // G
    q = rng.integers(0, 16, size=(N, K)).astype(np.int64)
    qg = q.reshape(N, ng, G)
    qg[:, :, 0] = 0
    qg[:, :, 1] = 15
    zp = rng.integers(0, 16, size=(N, ng))
    e = rng.integers(-14, -6, size=(N, ng))
    sc = np.ldexp(1.0, e)
    w = (sc[:, :, None] * (qg - zp[:, :, None])).reshape(N, K)
    Wb = oracle.f32_to_bf16(w.astype(np.float32))
    assert np.array_equal(oracle.bf16_to_f32(Wb).astype(np.float64), w)
    return Wb, q.reshape(N, K), zp, sc


def test_int4_exact_grid_head_recovers_codes_and_logits():
    N, K = 150, 1024
    Wb, q, zp, sc = grid_head4(N, K, 5)
    q4, sc4, zp4 = oracle.quantize4(Wb)
    assert np.array_equal(q4, q) and np.array_equal(zp4, zp) and np.array_equal(sc4.astype(np.float64), sc)
    p, S, ZS = oracle.pack4(Wb)
    assert np.array_equal(oracle.bf16_to_f32(S).astype(np.float64), 16 * sc)
    assert np.array_equal(oracle.bf16_to_f32(ZS).astype(np.float64), (16 + zp) * sc)
    # the bias-16 fold reproduces the weight exactly, so the coarse logits are the exact ones
    assert np.array_equal(oracle.dequantize4(p, S, ZS), oracle.bf16_to_f32(Wb).astype(np.float64))
    x = si.bits(si.gen_x(3, K, outliers=4, seed=41))
    assert np.allclose(oracle.coarse_logits4(x, p, S, ZS), oracle.exact_logits(x, Wb), rtol=0, atol=1e-9)


def block_top(vals, kc, block_n=64):
    """Per row, the kc best (value, token) pairs of each 64-column block by repeated pick (largest
    value, lower column on ties), in pure Python."""
    out = []
    for row in vals:
        r = []
        for b0 in range(0, len(row), block_n):
            cols = list(range(b0, min(b0 + block_n, len(row))))
            for _ in range(kc):
                best = cols[0]
                for c in cols[1:]:
                    if row[c] > row[best]:
                        best = c
                r.append((float(row[best]), best))
                cols.remove(best)
        out.append(r)
    return out


def test_head4_all_tokens_reranked_equals_brute_force():
    """P-5 for the int4 head: with KCAND = BLOCK_N and R = N every token is reranked exactly, so
    argmax and top-16 are those of the dense bf16 head."""
    N, K = 256, 512
    W = si.bits(si.gen_weight(N, K, seed=89))
    x = si.bits(si.gen_x(3, K, outliers=4, seed=42))
    p4, S4, ZS4 = oracle.pack4(W)
    ex = oracle.exact_logits(x, W)
    for k in (1, 16):
        r = oracle.head4(x, W, p4, S4, ZS4, kcand=64, R=N, k=k)
        want = brute_topk(ex, k)
        for m in range(3):
            assert list(r["idx"][m]) == want[m]
            assert np.allclose(r["val"][m], ex[m, want[m]], rtol=0, atol=1e-12)


@pytest.mark.parametrize("kcand", [1, 3])
def test_head4_exact_grid_head_end_to_end(kcand):
    """On an exact int4 grid the coarse logits are the exact bf16 logits, so every step is fixed
    by brute force: the block candidates are each block's kcand best exact logits, the selection
    the R best of those, and the result the best of the selection by exact score."""
    N, K, R = 1000, 512, 12                # 16 blocks, the last one 40 columns wide
    Wb, _, _, _ = grid_head4(N, K, 6)
    x = si.bits(si.gen_x(2, K, outliers=4, seed=43))
    p4, S4, ZS4 = oracle.pack4(Wb)
    r = oracle.head4(x, Wb, p4, S4, ZS4, kcand=kcand, R=R, k=4)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(Wb).astype(np.float64)
    exact = [[math.fsum(xf[m] * wf[n]) for n in range(N)] for m in range(2)]
    assert np.allclose(r["coarse"], np.array(exact), rtol=0, atol=1e-9)
    cands = block_top(exact, kcand)
    for m in range(2):
        assert r["cand_idx"][m].tolist() == [t for _, t in cands[m]]
        assert np.allclose(r["cand_score"][m], [v for v, _ in cands[m]], rtol=0, atol=1e-9)
        top = sorted(cands[m], key=lambda p: (-p[0], p[1]))[:R]
        assert len(top) == R and r["sel"][m].tolist() == [t for _, t in top]
        assert r["idx"][m].tolist() == [t for _, t in top[:4]]


def test_int4_quantize_matches_eager_fp32_ops():
    """Cross-check: the page's 4-bit quantiser and bias-16 premultiply as eager torch fp32 ops."""
    W = si.gen_weight(200, 1024, seed=87)
    w = W.float().reshape(200, 8, 128)
    lo, hi = w.amin(2), w.amax(2)
    sc = ((hi - lo) / 15).clamp(min=1e-8)
    zp = torch.round(-lo / sc).clamp(0, 15)
    qt = torch.round(w / sc[:, :, None] + zp[:, :, None]).clamp(0, 15).to(torch.uint8).reshape(200, 1024)
    S = (16.0 * sc).to(torch.bfloat16)
    ZS = (16.0 * sc + zp * sc).to(torch.bfloat16)
    q, sco, zpo = oracle.quantize4(si.bits(W))
    So, ZSo = oracle.premultiplied_scales4(sco, zpo)
    assert np.array_equal(q, qt.numpy())
    assert np.array_equal(So, si.bits(S)) and np.array_equal(ZSo, si.bits(ZS))
    packed = (qt[:, :512] | (qt[:, 512:] << 4)).numpy()
    assert np.array_equal(oracle.pack_half_split(q), packed)


def test_int4_shape_rule():
    oracle.check_shape4(256)
    oracle.check_shape4(5120)
    for bad in (0, 128, 384, 5000):
        with pytest.raises(ValueError):
            oracle.check_shape4(bad)


# ---------------------------------------------------------------------------------------------
# The measured alternatives (radiance_drafthead.py, module docstring and _emit): token-level
# selection, the contiguous-4 layout, the dequantised weight tile, group 64
# ---------------------------------------------------------------------------------------------
def brute_top_r(vals, R):
    """Repeated pick of the best remaining entry in pure Python: the largest value, and of equal
    values the lowest index (a strict > keeps the earlier one; -0.0 > 0.0 is false)."""
    left = list(range(len(vals)))
    out = []
    while left and len(out) < R:
        best = left[0]
        for i in left[1:]:
            if vals[i] > vals[best]:
                best = i
        out.append(best)
        left.remove(best)
    return out + [-1] * (R - len(out))


def test_select_tokens_brute_force_with_ties():
    rng = np.random.default_rng(17)
    pool = np.array([0x0000, 0x8000, 0x3F80, 0xBF80, 0x4000, 0x7F80, 0xFF80, 0x3F81, 0x0001, 0x8001],
                    np.uint16)  # +-0, +-1, 2, +-inf, a neighbour of 1, +-the smallest subnormal
    for N, R in [(1, 1), (5, 8), (37, 5), (200, 32), (64, 64)]:
        y = pool[rng.integers(0, len(pool), size=(3, N))]
        sel = oracle.select_tokens(y, R)
        for m in range(3):
            assert sel[m].tolist() == brute_top_r([bf(b) for b in y[m]], R)


def test_select_tokens_all_equal_and_short_rows():
    y = np.full((2, 100), 0x3F80, np.uint16)
    assert oracle.select_tokens(y, 10).tolist() == [list(range(10))] * 2
    y = np.array([[0x3F80, 0x4000, 0x3F80]], np.uint16)
    assert oracle.select_tokens(y, 5).tolist() == [[1, 0, 2, -1, -1]]


def test_select_tokens_equals_block_path_with_whole_blocks():
    """With KCAND = BLOCK_N every column is a block candidate, so the block path's selection over
    the same row must give the same tokens in the same order."""
    z = np.random.default_rng(5).normal(size=(3, 1000)).astype(np.float32)
    z[:, 100:140] = z[:, 60:100]  # repeated values across blocks
    y = oracle.f32_to_bf16(z)
    c = oracle.bf16_to_f32(y).astype(np.float64)
    cs, ci = oracle.block_emit(c, 64)
    for R in (1, 32, 300):
        assert np.array_equal(oracle.select_top_r(cs, ci, R), oracle.select_tokens(y, R))


def test_pack_contiguous4_worked_example():
    """By hand: K = 8, q = [1 2 3 0 0 3 2 1]: byte j = q[4j] | q[4j+1] << 2 | q[4j+2] << 4 | q[4j+3] << 6."""
    q = np.array([[1, 2, 3, 0, 0, 3, 2, 1]], np.uint8)
    assert oracle.pack_contiguous4(q).tolist() == [[0x39, 0x6C]]
    assert np.array_equal(oracle.unpack_contiguous4(oracle.pack_contiguous4(q)), q)


def test_contiguous4_layout_changes_no_value():
    q = np.random.default_rng(8).integers(0, 4, (9, 1024)).astype(np.uint8)
    assert np.array_equal(oracle.unpack_contiguous4(oracle.pack_contiguous4(q)), q)
    W = si.gen_weight(40, 1024, seed=21)
    pq, S, ZS = oracle.pack_variant(si.bits(W), layout="quarter")
    pc, S2, ZS2 = oracle.pack_variant(si.bits(W), layout="contiguous")
    assert np.array_equal(S, S2) and np.array_equal(ZS, ZS2)
    assert np.array_equal(oracle.unpack_contiguous4(pc), oracle.unpack_quarter_split(pq))
    x = si.bits(si.gen_x(2, 1024, seed=4))
    assert np.array_equal(oracle.coarse_logits_contiguous4(x, pc, S, ZS), oracle.coarse_logits(x, pq, S, ZS))


def test_dequantize_tile_hand_rounding():
    """By hand, S = bf16 1.0078125 (0x3F81), ZS = 0.5 (0x3F00), one group of K = 4 with codes
    (3, 1, 0, 2) in a quarter-split byte (3 | 1 << 2 | 0 << 4 | 2 << 6 = 0x87):
      v = 3: 1.0078125 * 1.75 - 0.5 = 1.263671875 -> 33.75/128 above 1 -> 34 -> 0x3FA2
      v = 1: 1.0078125 * 1.25 - 0.5 = 0.759765625 = 0.5 (1 + 66.5/128) -> tie, even 66 -> 0x3F42
      v = 0: 0.5078125 = 0.5 (1 + 2/128) exact -> 0x3F02
      v = 2: 1.51171875 - 0.5 = 1.01171875 = 1 + 1.5/128 -> tie, even 2 -> 0x3F82"""
    t = oracle.dequantize_tile(np.array([[0x87]], np.uint8), np.array([[0x3F81]], np.uint16),
                               np.array([[0x3F00]], np.uint16), G=4)
    assert [hex(v) for v in t[0]] == ["0x3fa2", "0x3f42", "0x3f02", "0x3f82"]


def grid_head_g(N, K, G, seed):
    """grid_head at any group size G."""
    rng = np.random.default_rng(seed)
    ng = K // G
    q = rng.integers(0, 4, size=(N, K)).astype(np.int64)
    qg = q.reshape(N, ng, G)
    qg[:, :, 0] = 0
    qg[:, :, 1] = 3
    zp = rng.integers(0, 4, size=(N, ng))
    sc = np.ldexp(1.0, rng.integers(-12, -3, size=(N, ng)))
    w = (sc[:, :, None] * (qg - zp[:, :, None])).reshape(N, K)
    Wb = oracle.f32_to_bf16(w.astype(np.float32))
    assert np.array_equal(oracle.bf16_to_f32(Wb).astype(np.float64), w)
    return Wb, q.reshape(N, K), zp, sc


def test_dequantize_tile_on_exact_grid_is_the_weight():
    """On the exact int2 grid S (1 + v/4) - ZS = sc (v - zp) is a bf16 value, so the rounded tile is
    the weight itself and the tile-scaled logits equal the accumulator-scaled ones."""
    Wb, q, zp, sc = grid_head_g(60, 1024, 128, 12)
    packed, S, ZS = oracle.pack(Wb)
    assert np.array_equal(oracle.dequantize_tile(packed, S, ZS), Wb)
    x = si.bits(si.gen_x(2, 1024, seed=6))
    assert np.array_equal(oracle.coarse_logits_tile(x, packed, S, ZS), oracle.coarse_logits(x, packed, S, ZS))


def test_group64_exact_grid_head():
    N, K, G = 80, 1024, 64
    Wb, q, zp, sc = grid_head_g(N, K, G, 14)
    qo, sco, zpo = oracle.quantize(Wb, G)
    assert np.array_equal(qo, q) and np.array_equal(zpo, zp) and np.array_equal(sco, sc)
    packed, S, ZS = oracle.pack_variant(Wb, G=G)
    assert S.shape == (N, K // G)
    assert np.array_equal(oracle.bf16_to_f32(ZS).astype(np.float64), (4 + zp) * sc)
    x = si.bits(si.gen_x(2, K, seed=10))
    c = oracle.coarse_logits(x, packed, S, ZS, G)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wf = oracle.bf16_to_f32(Wb).astype(np.float64)
    for m in range(2):
        for n in range(0, N, 7):
            want = math.fsum(xf[m] * wf[n])
            assert abs(c[m, n] - want) <= K * 2.0 ** -52 * np.sum(np.abs(xf[m] * wf[n]))
    with pytest.raises(ValueError):
        oracle.pack_variant(Wb[:, :128], G=G)  # K = 128 is not four quarters of whole groups
