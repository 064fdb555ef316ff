"""Pins for the oracle's fixed-size container and drift (O5-O8).

D-Quant section 4.2: every stream satisfies sum_i r(m_i) <= B = 8C - sigma
and fits its container; section 4.3: drift solves
min sum (x - x_hat)^2 s.t. the rate constraint, moving expensive symbols to
nearby cheaper ones; the paper's appendix observes every drifted symbol
landing on a neighbouring level (paragraph "Drift makes only sparse, local
corrections"). Checked here: container length bounds (including
adversarial rows), the rANS information identity, the one-level inward
property, minimality of the move set, and Everett's generalised-Lagrange
optimality by brute force on short streams.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle.codec import stream_cost, _apply_prefix

CONFIGS = [(8, 37), (6, 37), (8, 32), (6, 32)]


def adversarial_rows(rng):
    rows = []
    e = np.zeros(128); e[5] = 3.0; rows.append(e)                         # one-hot -> |z| = 1 everywhere
    rows.append(np.ones(128))                                             # constant
    rows.append(np.full(128, -7.5))
    o = np.zeros(128); o[[3, 17, 90, 101]] = [10, -10, 10, 10]; rows.append(o)   # outlier channels only
    rows.append(np.where(np.arange(128) % 2 == 0, 1.0, -1.0))             # alternating
    rows.append(oracle.fwht(np.eye(128)[7]))                              # a Hadamard row -> one huge z
    rows.append(rng.standard_t(2, 128))                                   # heavy tails
    rows.append(rng.standard_normal(128) * 1e-30)                         # tiny scale
    rows.append(rng.standard_normal(128) * 1e30)                          # huge scale (fp16 norm overflows)
    rows.append(np.zeros(128))
    s = np.zeros(128); s[::16] = rng.standard_normal(8) * 5; rows.append(s)  # sparse
    return np.array(rows)


@pytest.mark.parametrize("M,C", CONFIGS)
def test_every_container_fits_and_decodes(M, C):
    t = oracle.make_table(M, C)
    rng = np.random.default_rng(20)
    x = np.concatenate([rng.standard_normal((2000, 128)), adversarial_rows(rng),
                        rng.standard_normal((200, 128)) * np.where(rng.random((200, 128)) < 0.03, 10, 1)])
    r = oracle.encode_streams(x, t)
    assert np.all(r.lengths <= C)
    sym, ok = oracle.decode_streams(r.containers, t)
    assert ok.all() and np.array_equal(sym, r.symbols)
    assert stream_cost(r.symbols, t).max() <= t.budget_fx + 8 * oracle.COST_ONE


@pytest.mark.parametrize("M,C", CONFIGS)
def test_information_identity(M, C):
    """8 * emitted + log2(x_final / L) lies within the per-step rounding bounds
    around sum_i log2(2^p / f_{m_i}) (exact rANS arithmetic)."""
    t = oracle.make_table(M, C)
    p = t.prob_bits
    m = oracle.nearest_level(oracle.normalize(oracle.fwht(np.random.default_rng(21).standard_normal((3000, 128))))[2], t)
    cont, ln = oracle.rans_encode(m, t)
    xf = cont[:, 0].astype(np.int64) | (cont[:, 1].astype(np.int64) << 8) | (cont[:, 2].astype(np.int64) << 16)
    emitted = ln - 3
    info = 8.0 * emitted + np.log2(xf / oracle.STATE_LOW)
    r_true = np.log2((1 << p) / t.freq[m]).sum(axis=1)
    a = -math.log2(1 - 2.0 ** (p - 16))
    c = math.log2(1 + 2.0 ** (p - 16))
    b = math.log2(1 + 2.0 ** -8)
    n = m.shape[1]
    assert np.all(info <= r_true + n * c + 1e-9)
    assert np.all(info >= r_true - n * a - emitted * b - 1e-9)


@pytest.mark.parametrize("M,C", CONFIGS)
def test_drift_moves_to_the_nearest_cheaper_inner_level(M, C):
    t = oracle.make_table(M, C)
    x = np.random.default_rng(22).standard_normal((3000, 128))
    r = oracle.encode_streams(x, t)
    assert not r.fallback.any()
    d = r.symbols - r.nearest
    ch = d != 0
    # one drift move per changed symbol, to its drift target
    assert np.array_equal(r.symbols[ch], t.inner[r.nearest[ch]])
    # no symbol moves by more than one level (the paper's drift analysis in the appendix)
    assert np.abs(d).max() <= 1
    # moves go toward zero and to a strictly cheaper level
    assert np.all(np.abs(t.recon[r.symbols[ch]]) < np.abs(t.recon[r.nearest[ch]]))
    assert np.all(t.cost[r.symbols[ch]] < t.cost[r.nearest[ch]])
    # streams that were within budget and fit as nearest-level are untouched
    R0 = stream_cost(r.nearest, t)
    _, ln0 = oracle.rans_encode(r.nearest, t)
    untouched = (R0 <= t.budget_fx) & (ln0 <= C)
    assert np.all(r.changed[untouched] == 0)
    assert np.all(r.rounds[untouched] == 0)


DEFAULT_TABLES = [(8, 37), (6, 37), (8, 32), (6, 32), (8, 41), (6, 27)]


@pytest.mark.parametrize("M,C", DEFAULT_TABLES)
def test_every_drift_target_is_the_adjacent_inner_level(M, C):
    """Table property behind the one-level invariant: the quantised
    frequencies keep the strict outward order of the N(0,1) cell masses, so
    each non-central level's adjacent inner neighbour is strictly cheaper and
    is its drift target; the central level(s) never drift."""
    t = oracle.make_table(M, C)
    half = M // 2
    assert np.all(np.diff(t.mass[:half]) > 0)
    assert np.all(np.diff(t.freq[:half + (M % 2)]) > 0)
    for m in range(M):
        if t.recon[m] < 0 and m + 1 < M and t.recon[m + 1] < 0 or (M % 2 and m == half - 1):
            assert t.inner[m] == m + 1 and t.cost[m + 1] < t.cost[m]
        elif t.recon[m] > 0 and t.recon[m - 1] > 0 or (M % 2 and m == half + 1):
            assert t.inner[m] == m - 1 and t.cost[m - 1] < t.cost[m]
        else:
            assert t.inner[m] == -1


def test_tied_tail_frequencies_are_separated():
    """At 32 bytes and 8 levels the two outermost key cells both round below
    the floor 2^(p-8) = 4; the second one, strictly more probable, gets one
    unit more, so its cost is strictly lower (a tie would send level 0 two
    levels inward)."""
    t = oracle.make_table(8, 32)
    assert t.mass[1] > t.mass[0] and t.sharpened[1] * 1024 < 4 and t.sharpened[0] * 1024 < 4
    assert t.freq[0] == 4 and t.freq[1] == 5 and t.cost[1] < t.cost[0]
    assert t.inner.tolist() == [1, 2, 3, -1, -1, 4, 5, 6]


@pytest.mark.parametrize("M,C", DEFAULT_TABLES)
def test_gaussian_drift_never_moves_more_than_one_level(M, C):
    """Seeded N(0,1) streams on every default table, outermost levels
    included: every changed symbol moves exactly one level inward."""
    t = oracle.make_table(M, C)
    x = np.random.default_rng(1000 + 7 * M + C).standard_normal((20000, 128))
    r = oracle.encode_streams(x, t)
    assert not r.fallback.any()
    d = r.symbols - r.nearest
    assert np.abs(d).max() <= 1
    assert np.all(np.abs(t.recon[r.symbols[d != 0]]) < np.abs(t.recon[r.nearest[d != 0]]))
    if (M, C) == (8, 32):   # the sample reaches the outermost levels, so the pin covers them
        assert np.count_nonzero((d != 0) & ((r.nearest == 0) | (r.nearest == M - 1))) > 0


@pytest.mark.parametrize("M,C", CONFIGS)
def test_drift_is_minimal(M, C):
    """Undoing the last move of a drifted stream breaks the rate condition
    or the container fit."""
    t = oracle.make_table(M, C)
    x = np.random.default_rng(23).standard_normal((1500, 128))
    r = oracle.encode_streams(x, t)
    dr_idx = np.nonzero(r.changed > 0)[0]
    assert len(dr_idx) > 100
    order, n_cand, dr_sorted, _ = oracle.drift_candidates(r.z[dr_idx], r.nearest[dr_idx], t)
    k = r.changed[dr_idx]
    # the stored symbols are exactly the first k candidates moved
    assert np.array_equal(_apply_prefix(r.nearest[dr_idx], order, t.inner, k), r.symbols[dr_idx])
    prev = _apply_prefix(r.nearest[dr_idx], order, t.inner, k - 1)
    over_rate = stream_cost(prev, t) > t.budget_fx
    _, ln = oracle.rans_encode(prev, t)
    assert np.all(over_rate | (ln > C))


def test_everett_optimality_brute_force():
    """Among all subsets of candidate moves whose rate is no higher than the
    selected prefix's, none has lower distortion (Everett 1963), whenever the
    selected prefix is strictly separated in key from the next candidate."""
    t = oracle.make_table(8, 37)
    rng = np.random.default_rng(24)
    checked = 0
    for trial in range(60):
        n = 14
        z = rng.standard_normal((1, n)) * 1.3
        m0 = oracle.nearest_level(z, t)
        order, n_cand, dr_sorted, inner = oracle.drift_candidates(z, m0, t)
        nc = int(n_cand[0])
        if nc < 2:
            continue
        R0 = int(stream_cost(m0, t)[0])
        need = int(dr_sorted[0, :nc].sum() * rng.uniform(0.2, 0.8))
        budget = R0 - need
        csum = np.concatenate([[0], np.cumsum(dr_sorted[0, :nc])])
        k = int(np.argmax(R0 - csum <= budget))
        cand = order[0, :nc]
        keys = []
        for i in cand:
            dd = (z[0, i] - t.recon[inner[0, i]]) ** 2 - (z[0, i] - t.recon[m0[0, i]]) ** 2
            keys.append(dd / (t.cost[m0[0, i]] - t.cost[inner[0, i]]))
        if k < nc and not keys[k - 1] < keys[k]:
            continue

        def rate_dist(subset):
            m = m0[0].copy()
            for i in subset:
                m[i] = inner[0, i]
            return int(t.cost[m].sum()), float(((z[0] - t.recon[m]) ** 2).sum())

        r_sel, d_sel = rate_dist(cand[:k])
        for bits in itertools.product([0, 1], repeat=nc):
            sub = [cand[j] for j in range(nc) if bits[j]]
            r_s, d_s = rate_dist(sub)
            if r_s <= r_sel:
                assert d_s >= d_sel - 1e-12
        checked += 1
    assert checked >= 20


def test_tiny_container_forces_fallback_and_still_fits():
    # C = 30 with 8 levels at the step tuned for 37 bytes: some streams need a second round
    t = oracle.make_table(8, 30, step=0.9)
    assert t.feasible
    x = np.random.default_rng(25).standard_normal((400, 128))
    r = oracle.encode_streams(x, t)
    assert np.all(r.lengths <= 30)
    assert r.fallback.any()
    sym, ok = oracle.decode_streams(r.containers, t)
    assert ok.all() and np.array_equal(sym, r.symbols)
