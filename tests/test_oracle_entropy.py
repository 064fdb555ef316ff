"""Pins for entropy tracking and the rate measures (D-Quant section 3.1, 3.2).

The rANS code length of nearest-level symbols of N(0,1) rows must track the
empirical cross-entropy under the table's model, and with no sharpening the
closed-form entropy of quantised N(0,1). The paper's Coding Gain and Normal
Gap definitions are checked on distributions with known values.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import measures


def code_length_bits(m, t):
    cont, ln = oracle.rans_encode(m, t)
    xf = cont[:, 0].astype(np.int64) | (cont[:, 1].astype(np.int64) << 8) | (cont[:, 2].astype(np.int64) << 16)
    return 8.0 * (ln - 3) + np.log2(xf / oracle.STATE_LOW)


@pytest.mark.parametrize("M,C", [(8, 37), (6, 37), (8, 32)])
def test_code_length_tracks_cross_entropy(M, C):
    t = oracle.make_table(M, C)
    z = oracle.normalize(oracle.fwht(np.random.default_rng(30).standard_normal((20000, 128))))[2]
    m = oracle.nearest_level(z, t)
    per_sym = code_length_bits(m, t).sum() / m.size
    ce = measures.cross_entropy(measures.histogram(m, M), t.freq / 1024.0)
    assert abs(per_sym - ce) < 0.01


def test_unsharpened_code_length_tracks_normal_entropy():
    t = oracle.make_table(8, 37, step=0.9, alpha=1.0)
    z = oracle.normalize(oracle.fwht(np.random.default_rng(31).standard_normal((20000, 128))))[2]
    m = oracle.nearest_level(z, t)
    per_sym = code_length_bits(m, t).sum() / m.size
    H = measures.entropy(t.mass)   # closed form from the N(0,1) cell masses
    assert abs(per_sym - H) < 0.02


def test_measure_definitions():
    u = np.full(8, 1 / 8)
    assert measures.coding_gain(u) == pytest.approx(0.0, abs=1e-15)
    assert measures.entropy(u) == pytest.approx(3.0)
    p = np.array([0.5, 0.25, 0.125, 0.125])
    assert measures.entropy(p) == pytest.approx(1.75)
    assert measures.coding_gain(p) == pytest.approx(0.25)
    q = np.array([0.25, 0.25, 0.25, 0.25])
    # normal gap = CE - H = KL(p || q)
    kl = sum(pi * math.log2(pi / qi) for pi, qi in zip(p, q))
    assert measures.normal_gap(p, q) == pytest.approx(kl)
    assert measures.normal_gap(p, p) == pytest.approx(0.0, abs=1e-15)
    assert measures.nmse(np.ones(4), np.zeros(4)) == 1.0
