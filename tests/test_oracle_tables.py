"""Pins for the oracle's static entropy table (O1).

D-Quant derives the probability model from N(0,1) (sections 1, 3.2) and
sharpens it as p' ~ p^alpha with alpha = 1.4 (sections 4.4, 5.1). The cell
masses are checked against scipy.stats.norm; the integer table against the
invariants any rANS table at precision 2^p must satisfy.
"""
import math

import numpy as np
import pytest
import scipy.stats

import oracle

CONFIGS = [(8, 37), (6, 37), (8, 32), (6, 32)]


def scipy_cell_masses(t):
    edges = np.concatenate([[-np.inf], t.bounds, [np.inf]])
    return np.diff(scipy.stats.norm.cdf(edges))


@pytest.mark.parametrize("M,C", CONFIGS)
def test_table_invariants(M, C):
    t = oracle.make_table(M, C)
    assert t.feasible
    assert int(t.freq.sum()) == 1 << t.prob_bits
    assert np.array_equal(t.freq, t.freq[::-1])                 # symmetric
    assert np.all(t.freq >= t.f_min) and t.f_min == 1 << (t.prob_bits - 8)
    assert t.cum[0] == 0 and t.cum[-1] == 1 << t.prob_bits
    assert np.array_equal(np.diff(t.cum), t.freq)
    for m in range(M):                                            # slot table inverts cum
        assert np.all(t.sym[t.cum[m]:t.cum[m + 1]] == m)
    assert np.array_equal(t.recon, -t.recon[::-1])                # symmetric grid
    assert np.allclose(np.diff(t.recon), t.step, rtol=1e-15)
    assert np.allclose(t.bounds, (t.recon[:-1] + t.recon[1:]) / 2)
    # costs never decrease outward from the centre
    half = M // 2
    assert np.all(np.diff(t.cost[half:]) >= 0)
    assert t.budget_fx == (8 * C - 24) << 16


@pytest.mark.parametrize("M,C", CONFIGS)
def test_masses_match_scipy_normal(M, C):
    t = oracle.make_table(M, C)
    assert np.allclose(t.mass, scipy_cell_masses(t), rtol=1e-12, atol=1e-15)
    assert abs(t.mass.sum() - 1.0) < 1e-14


@pytest.mark.parametrize("M", [4, 5, 6, 7, 8])
def test_unsharpened_high_precision_frequencies_track_normal(M):
    # alpha = 1, p = 16, a step where no level is clamped: f / 2^p -> N(0,1) cell masses
    t = oracle.make_table(M, 400, step=0.5, alpha=1.0, prob_bits=16)
    ref = scipy_cell_masses(t)
    assert np.all(ref * 2 ** 16 > t.f_min)
    assert np.max(np.abs(t.freq / 2.0 ** 16 - ref)) <= M / 2.0 ** 16


def test_sharpening_ratio():
    t1 = oracle.make_table(8, 37, alpha=1.0)
    t2 = oracle.make_table(8, 37, alpha=1.4)
    # q'_m / q'_j = (p_m / p_j)^alpha
    r1 = t1.sharpened / t1.sharpened[3]
    r2 = t2.sharpened / t2.sharpened[3]
    assert np.allclose(r2, r1 ** 1.4, rtol=1e-12)
    assert abs(t2.sharpened.sum() - 1) < 1e-15
    # sharpening moves mass to the centre
    assert t2.sharpened[3] > t1.sharpened[3] and t2.sharpened[0] < t1.sharpened[0]


def test_cost_fixed_point_exact_for_powers_of_two():
    t = oracle.make_table(8, 32, step=1.1)
    for f, c in zip(t.freq, t.cost):
        if f & (f - 1) == 0:
            assert c == (t.prob_bits - int(math.log2(f))) << 16
        assert abs(c / 65536.0 + math.log2(f / 1024.0)) <= 0.5 / 65536.0


def test_infeasible_containers_are_flagged():
    # all-central stream: 128 * ~1.49 bits > 8*20 - 24 bits
    assert not oracle.make_table(8, 20, step=0.9).feasible
    assert oracle.make_table(8, 37, step=0.9).feasible


@pytest.mark.parametrize("M", [3, 5, 7])
def test_odd_level_count(M):
    t = oracle.make_table(M, 37, step=0.9)
    assert t.recon[M // 2] == 0.0 and t.inner[M // 2] == -1
    assert int(t.freq.sum()) == 1024 and np.array_equal(t.freq, t.freq[::-1])


@pytest.mark.parametrize("M,C", CONFIGS)
def test_nearest_level_brute_force_and_ties(M, C):
    t = oracle.make_table(M, C)
    z = np.random.default_rng(50).standard_normal(20000) * 2
    m = oracle.nearest_level(z, t)
    # away from midpoints the nearest level is the argmin of |z - level|
    assert np.array_equal(m, np.argmin(np.abs(z[:, None] - t.recon[None, :]), axis=1))
    # an exact midpoint goes to the level nearer zero
    for j, b in enumerate(t.bounds):            # b lies between levels j and j+1
        got = int(oracle.nearest_level(np.array([b]), t)[0])
        if b > 0:
            assert got == j
        elif b < 0:
            assert got == j + 1
        else:
            assert got == M // 2 - 1
        assert abs(t.recon[got]) <= abs(t.recon[j + (1 if got == j else 0)])


def test_feasibility_follows_drift_reachability():
    """Drift only moves a symbol inward to a strictly cheaper level (section 4.3),
    so feasibility is judged on the levels drift can end at. A grid so narrow
    that the outer cells are the likeliest (cheapest) cannot be drifted into
    budget, and is rejected; every table judged feasible encodes adversarial
    streams (all values in the outermost cells, alternating signs) without error."""
    assert not oracle.make_table(6, 32, step=0.3).feasible
    x = np.tile(np.array([9.0, -9.0] * 64), (4, 1))
    x[1] = np.linspace(-3, 3, 128)
    x[2, ::3] = 0.0
    x[3] = np.random.default_rng(0).standard_normal(128)
    checked = 0
    for M in (4, 6, 8):
        for C in (24, 28, 32, 37):
            for step in (0.3, 0.6, 0.9, 1.2, 1.6):
                t = oracle.make_table(M, C, step=step)
                if t.feasible:
                    r = oracle.encode_streams(x, t)
                    assert (r.lengths <= C).all()
                    checked += 1
    assert checked > 10
