"""The GPU parity rules themselves (CPU only): a coarse error of the size the kernels show passes,
one ten times larger fails, and a swap of two candidates is excused only inside the tie window.
The perturbations are planted on the oracle's own outputs, on the CPU."""
import numpy as np
import pytest

import oracle
import parity_util as pu
import synth_inputs as si

FOLD2 = (32.0, 8.0, 2.0, 1.0)


@pytest.fixture(scope="module")
def head():
    N, K, M, kc = 4096, 512, 2, 8
    Wb = si.bits(si.gen_weight(N, K, seed=61))
    xb = si.bits(si.gen_x(M, K, seed=62))
    p, S, ZS = oracle.pack(Wb)
    c = oracle.coarse_logits(xb, p, S, ZS)
    cs, ci = oracle.block_emit(c, kc)
    mag = pu.fold_magnitude(ci, xb, S, ZS, FOLD2)
    return c, cs, ci, mag, kc


def _signs(shape, seed):
    return np.where(np.random.default_rng(seed).random(shape) < 0.5, -1.0, 1.0)


def _perturbed(cs, ci, delta, kc):
    """Scores moved by delta, each block's list then reordered best first by its own scores (as
    a kernel orders what it computed)."""
    M, n = cs.shape
    s = (cs + delta).reshape(M, n // kc, kc)
    i = ci.reshape(M, n // kc, kc)
    o = np.lexsort((i, -s), axis=2)
    return np.take_along_axis(s, o, 2).reshape(M, n), np.take_along_axis(i, o, 2).reshape(M, n)


def test_measured_error_size_passes(head):
    """0.6 half-ulps of the fold magnitude, the largest ratio measured on the kernels, passes."""
    c, cs, ci, mag, kc = head
    got, gi = _perturbed(cs, ci, 0.6 * pu.U32 * mag * _signs(cs.shape, 1), kc)
    gmag = pu.fold_magnitude(gi, si.bits(si.gen_x(2, 512, seed=62)), *oracle.pack(si.bits(si.gen_weight(4096, 512, seed=61)))[1:], FOLD2)
    assert pu.fold_error_ratio(got, gi, c, gmag) == pytest.approx(0.6, rel=1e-6)
    pu.check_candidates(got, gi, c, kc, budget=pu.FOLD_C * pu.U32 * gmag)


def test_ten_times_the_measured_error_fails(head):
    c, cs, ci, mag, kc = head
    got, gi = _perturbed(cs, ci, 6.0 * pu.U32 * mag * _signs(cs.shape, 2), kc)
    with pytest.raises(AssertionError, match="budget|tie window"):
        pu.check_candidates(got, gi, c, kc, budget=pu.FOLD_C * pu.U32 * mag)


def test_fold_budget_is_far_inside_the_specified_tolerance(head):
    """The candidate budget is a small fraction of the coarse tolerance the head is specified
    with (2e-3 of the row's largest logit)."""
    c, cs, ci, mag, kc = head
    budget = pu.FOLD_C * pu.U32 * mag
    assert (budget.max(axis=1) / pu.row_scale(c)).max() < 0.1 * pu.COARSE_TOL


def _planted_swap(c, kc, gap):
    """Oracle logits with the best two columns of row 0, block 0 planted `gap` apart, the oracle's
    candidates of those logits, and a kernel's list that has the two the other way round (both
    scored half-way between)."""
    c2 = c.copy()
    cs, ci = oracle.block_emit(c2, kc)
    a, b = ci[0, 0], ci[0, 1]
    c2[0, b] = c2[0, a] - gap
    cs, ci = oracle.block_emit(c2, kc)
    assert (ci[0, 0], ci[0, 1]) == (a, b)
    gs, gi = cs.copy(), ci.copy()
    gi[0, 0], gi[0, 1] = b, a
    gs[0, 0] = gs[0, 1] = c2[0, a] - gap / 2
    return c2, gs, gi


def test_swap_inside_the_tie_window_is_excused(head):
    c, cs, ci, mag, kc = head
    budget = pu.FOLD_C * pu.U32 * mag
    bmax = np.full_like(budget, budget.max())
    win = pu.tie_window(c, bmax)
    c2, gs, gi = _planted_swap(c, kc, 0.5 * win[0])
    diff, _ = pu.check_candidates(gs, gi, c2, kc, budget=bmax)
    assert diff == 2


def test_swap_outside_the_tie_window_fails(head):
    c, cs, ci, mag, kc = head
    budget = pu.FOLD_C * pu.U32 * mag
    win = pu.tie_window(c, budget)
    c2, gs, gi = _planted_swap(c, kc, 3 * win[0])
    # the swapped scores are 1.5 windows from the oracle's: a kernel cannot order the two so
    # without missing one of them by more than its budget
    with pytest.raises(AssertionError, match="budget|tie window"):
        pu.check_candidates(gs, gi, c2, kc, budget=budget)
