"""Pins of the rank-allocation oracle against facts fixed outside it:
hand-computed entropies and a worked allocation, exhaustive search on tiny
inputs, budget conservation, and the behaviour the pages state (slowly
decaying spectra receive more rank)."""
import itertools
import math

import numpy as np
import pytest

from oracle import rank_alloc as ra_


def spectra(rhos, d=128, heads=1, scale=1.0):
    return np.array([[scale * rho ** np.arange(d) for _ in range(heads)] for rho in rhos])


def test_entropy_closed_forms():
    H, p = ra_.block_distribution(np.ones((1, 8)))
    assert abs(H - math.log(8)) < 1e-12 and np.allclose(p, 1 / 8)
    H, p = ra_.block_distribution(np.array([[5.0, 0, 0, 0]]))
    assert H == 0.0 and p[0] == 1.0
    H, p = ra_.block_distribution(np.array([[3.0, 4.0]]))          # energies 9, 16
    np.testing.assert_allclose(p, [0.36, 0.64])
    assert abs(H - (-(0.36 * math.log(0.36) + 0.64 * math.log(0.64)))) < 1e-12


def test_head_averaging_and_empty_heads():
    # heads with distributions (1/2, 1/2, 0) and (1, 0, 0): mean (3/4, 1/4, 0)
    H, p = ra_.block_distribution(np.array([[1.0, 1.0, 0.0], [7.0, 0.0, 0.0]]))
    np.testing.assert_allclose(p, [0.75, 0.25, 0.0])
    assert abs(H - (-(0.75 * math.log(0.75) + 0.25 * math.log(0.25)))) < 1e-12
    # a head without energy contributes nothing: the other head's (1/2, 1/2)
    H, p = ra_.block_distribution(np.array([[2.0, 2.0], [0.0, 0.0]]))
    np.testing.assert_allclose(p, [0.5, 0.5])
    assert abs(H - math.log(2)) < 1e-12
    H, p = ra_.block_distribution(np.zeros((2, 4)))
    assert H == 0.0 and np.all(p == 0)


def test_worked_allocation():
    """Two one-head blocks, d = 3: A = (2, 1, 0) has p = (0.8, 0.2, 0) and
    H_A = 0.50040242; B = (1, 1, 1) has p = 1/3 each and H_B = ln 3.  Unit
    gains: A 0.40032, 0.10008, 0; B 0.36620 three times.  The greedy order
    is A, B, B, B, A, A."""
    sig = np.array([[[2.0, 1.0, 0.0]], [[1.0, 1.0, 1.0]]])
    want = [[0, 0], [1, 0], [1, 1], [1, 2], [1, 3], [2, 3], [3, 3]]
    for budget, w in enumerate(want):
        assert list(ra_.allocate(sig, budget, 0)) == w, budget
    H_A, _ = ra_.block_distribution(sig[0])
    assert abs(H_A - 0.50040242353) < 1e-10


def test_worked_allocation_where_entropy_decides():
    """A = (3, 1, 0, 0): p = (0.9, 0.1, 0, 0), H_A = 0.32508297; B = (1, 1, 1,
    1): p = 1/4 each, H_B = ln 4.  A's first unit adds more energy (0.9 >
    0.25) but gains less (0.29257 < 0.34657): B fills first, then A."""
    sig = np.array([[[3.0, 1.0, 0.0, 0.0]], [[1.0, 1.0, 1.0, 1.0]]])
    want = [[0, 0], [0, 1], [0, 2], [0, 3], [0, 4], [1, 4], [2, 4], [3, 4], [4, 4]]
    for budget, w in enumerate(want):
        assert list(ra_.allocate(sig, budget, 0)) == w, budget
    H_A, _ = ra_.block_distribution(sig[0])
    assert abs(H_A - 0.3250829734) < 1e-9


@pytest.mark.parametrize("r_min,unit", [(0, 1), (1, 1), (0, 2), (1, 2)])
def test_greedy_equals_exhaustive_optimum(r_min, unit):
    rng = np.random.default_rng(7 + r_min + 3 * unit)
    d, nb = 5, 3
    sig = np.sort(rng.gamma(1.0, 1.0, size=(nb, 2, d)), axis=-1)[..., ::-1] * rng.uniform(0.2, 5, (nb, 1, 1))
    per = (d - r_min) // unit
    for k in range(0, nb * per + 1):
        budget = nb * r_min + k * unit
        best = max(ra_.objective(sig, [r_min + unit * c for c in cs], r_min, unit)
                   for cs in itertools.product(range(per + 1), repeat=nb) if sum(cs) == k)
        got = ra_.allocate(sig, budget, r_min, unit)
        assert got.sum() == budget
        assert abs(ra_.objective(sig, got, r_min, unit) - best) <= 1e-12 * max(1.0, best)


def test_budget_conservation_and_bounds():
    rng = np.random.default_rng(3)
    sig = np.sort(rng.gamma(0.7, 1.0, size=(9, 4, 64)), axis=-1)[..., ::-1]
    for budget in (9 * 4, 100, 300, 9 * 64):
        r = ra_.allocate(sig, budget, 4)
        assert r.sum() == budget and r.min() >= 4 and r.max() <= 64
    r = ra_.allocate(sig, 9 * 8 + 16 * 10, 8, unit=16)
    assert r.sum() == 9 * 8 + 160 and np.all((r - 8) % 16 == 0)


def test_slowly_decaying_spectrum_gets_more_rank():
    """The pages' stated preference, at a 25% budget."""
    r = ra_.allocate(spectra([0.6, 0.95], heads=2), 64, 8)
    assert r[1] > r[0]


def test_scale_invariance_and_tie_break():
    base = spectra([0.8, 0.9, 0.7], heads=2)
    scaled = base.copy()
    scaled[0] *= 1000.0
    assert np.array_equal(ra_.allocate(base, 120, 4), ra_.allocate(scaled, 120, 4))
    same = spectra([0.85, 0.85, 0.85])
    r = ra_.allocate(same, 3 * 10 + 2, 10)
    assert list(r) == [11, 11, 10]            # equal gains: lowest block index first


def test_zero_energy_block_keeps_minimum_until_others_are_full():
    sig = np.concatenate([spectra([0.9], d=8), np.zeros((1, 1, 8))])
    assert list(ra_.allocate(sig, 2 + 6, 1)) == [7, 1]
    assert list(ra_.allocate(sig, 8 + 3, 1)) == [8, 3]    # A is full: the rest goes to B


def test_invalid_budgets():
    sig = spectra([0.9, 0.8], d=16)
    for b, rmin, u in [(1, 1, 1), (33, 0, 1), (5, 1, 2)]:
        with pytest.raises(ValueError):
            ra_.allocate(sig, b, rmin, u)
