"""Pins of O13-O17, the per-token stream format (one 1024-value stream per
token over all 8 KV heads, token-wise min-max affine grid, drift, rANS, least-
squares refit with fp16 metadata; sections 4.2, 4.3, 4.5, 5.1 and the
appendix paragraph "Compared configurations"): closed
forms of the expected maximum, brute force for the nearest level, a library
least-squares solve for the refit, exact invariances of the min-max grid, and
the container and drift invariants the paper states."""
import math

import numpy as np
import pytest

from oracle import token as tk
from oracle.codec import fwht

K_CFG, V_CFG = (8, 331), (6, 231)


@pytest.fixture(scope="module")
def tables():
    return {cfg: tk.make_token_table(*cfg) for cfg in (K_CFG, V_CFG)}


def _tokens(seed, S=48, outliers=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((S, 8, 128))
    if outliers:
        x[:, :, :4] *= 10.0
    return x


def test_expected_max_closed_forms():
    """E[max] of 1, 2, 3 standard normals: 0, 1/sqrt(pi), 3/(2 sqrt(pi))."""
    assert abs(tk.expected_max(1)) < 1e-12
    assert abs(tk.expected_max(2) - 1 / math.sqrt(math.pi)) < 1e-12
    assert abs(tk.expected_max(3) - 3 / (2 * math.sqrt(math.pi))) < 1e-12


def test_expected_max_1024_against_sampling():
    """e_1024 against the mean maximum of 4000 seeded samples of 1024 values
    (standard error about 0.007)."""
    rng = np.random.default_rng(11)
    mx = rng.standard_normal((4000, 1024)).max(axis=1)
    e = tk.expected_max(1024)
    assert abs(e - mx.mean()) < 4 * mx.std() / math.sqrt(len(mx))
    assert tk.token_step(8) == pytest.approx(2 * e / 7, rel=1e-15)


def test_grid_index_brute_force():
    """Nearest level in grid units against argmin |u - m|, with exact
    midpoints going to the level nearer the centre."""
    rng = np.random.default_rng(2)
    for M in (2, 3, 6, 8, 9):
        u = np.concatenate([rng.uniform(0, M - 1, 500), np.arange(0, M - 1) + 0.5, np.arange(M, dtype=float)])
        got = tk.grid_index(u, M)
        half = (M - 1) / 2
        for ui, gi in zip(u, got):
            d = np.abs(ui - np.arange(M))
            best = np.nonzero(d == d.min())[0]
            if len(best) == 1:
                assert gi == best[0]
            else:                                   # a midpoint: the level nearer the centre
                dc = np.abs(best - half)
                want = best[np.argmin(dc)] if dc[0] != dc[1] else best[0]
                assert gi == want, (M, ui)


def test_rotation_is_per_head_hadamard():
    """y = [H x_0, .., H x_7] with H the 128-point Hadamard matrix."""
    from scipy.linalg import hadamard
    x = _tokens(3, S=4)
    y = tk.rotate_tokens(x)
    Hm = hadamard(128).astype(np.float64)
    for h in range(8):
        assert np.allclose(y[:, h * 128:(h + 1) * 128], x[:, h] @ Hm.T, rtol=0, atol=1e-12)


def test_fold_sum_matches_exact_sum_on_integers():
    rng = np.random.default_rng(4)
    v = rng.integers(-1000, 1000, (5, 1024)).astype(np.float64)
    assert np.array_equal(tk.fold_sum(v), v.sum(axis=1))


@pytest.mark.parametrize("cfg", [K_CFG, V_CFG])
def test_round_trip_and_container(tables, cfg):
    """decode(container) gives the stored symbols with a clean final state;
    every stream fits its C bytes."""
    t = tables[cfg]
    r = tk.encode_tokens(_tokens(5, outliers=cfg == K_CFG), t)
    sym, ok = tk.decode_tokens(r.containers, t)
    assert ok.all()
    assert np.array_equal(sym, r.symbols)
    assert np.all(r.lengths <= t.container)


@pytest.mark.parametrize("cfg", [K_CFG, V_CFG])
def test_min_max_grid_and_nearest(tables, cfg):
    """Before drift: the minimum sits on level 0, the maximum on level M-1,
    and every symbol is the brute-force nearest level of (y - o)/s."""
    t = tables[cfg]
    M = t.levels
    r = tk.encode_tokens(_tokens(6), t)
    assert np.all(r.nearest[np.arange(len(r.y)), r.y.argmin(1)] == 0)
    assert np.all(r.nearest[np.arange(len(r.y)), r.y.argmax(1)] == M - 1)
    levels = r.o[:, None, None] + r.s[:, None, None] * np.arange(M)[None, None, :]
    d = np.abs(r.y[:, :, None] - levels)
    assert np.all(d[np.arange(len(r.y))[:, None], np.arange(1024)[None, :], r.nearest] <= d.min(-1) * (1 + 1e-9) + 1e-12)


@pytest.mark.parametrize("cfg", [K_CFG, V_CFG])
def test_refit_is_least_squares(tables, cfg):
    """(o*, s*) equals numpy's least-squares solution of y ~ [1, m] for the
    stored symbols, and the fp16 metadata is its single rounding."""
    t = tables[cfg]
    r = tk.encode_tokens(_tokens(7), t)
    o_star, s_star, o16, s16 = tk.refit(r.y, r.symbols)
    for i in range(len(r.y)):
        A = np.stack([np.ones(1024), r.symbols[i].astype(np.float64)], axis=1)
        (o_ls, s_ls), *_ = np.linalg.lstsq(A, r.y[i], rcond=None)
        assert o_star[i] == pytest.approx(o_ls, rel=1e-10, abs=1e-10)
        assert s_star[i] == pytest.approx(s_ls, rel=1e-10)
    assert np.array_equal(r.o16, o_star.astype(np.float16)) and np.array_equal(r.s16, s_star.astype(np.float16))
    # the refit never does worse than the min-max grid it replaces (before fp16 rounding)
    e_fit = ((r.y - (o_star[:, None] + s_star[:, None] * r.symbols)) ** 2).sum(1)
    e_mm = ((r.y - (r.o[:, None] + r.s[:, None] * r.symbols)) ** 2).sum(1)
    assert np.all(e_fit <= e_mm * (1 + 1e-12))


@pytest.mark.parametrize("cfg", [K_CFG, V_CFG])
def test_drift_is_one_level_inward(tables, cfg):
    """In a single drift round every changed symbol moves to its level's drift
    target (one level toward the centre for these tables); the coded cost then
    fits the budget or the stream's rANS length fits the container."""
    t = tables[cfg]
    r = tk.encode_tokens(_tokens(8), t)
    one = r.rounds <= 1
    assert one.any()
    ch = (r.symbols != r.nearest) & one[:, None]
    assert np.all(r.symbols[ch] == t.inner[r.nearest[ch]])
    assert np.all(np.abs(r.symbols - r.nearest)[one] <= 1)
    # no drift when the nearest symbols already fit
    nod = r.rounds == 0
    assert np.array_equal(r.symbols[nod], r.nearest[nod])


@pytest.mark.parametrize("cfg", [K_CFG, V_CFG])
def test_power_of_two_scale_invariance(tables, cfg):
    """x -> 4x leaves u, symbols and containers unchanged and scales the fp16
    metadata by 4 exactly: nothing depends on the absolute scale."""
    t = tables[cfg]
    x = _tokens(9, S=16)
    a = tk.encode_tokens(x, t)
    b = tk.encode_tokens(4.0 * x, t)
    assert np.array_equal(a.symbols, b.symbols) and np.array_equal(a.containers, b.containers)
    assert np.array_equal(b.o16.astype(np.float64), 4.0 * a.o16.astype(np.float64))
    assert np.array_equal(b.s16.astype(np.float64), 4.0 * a.s16.astype(np.float64))


def test_constant_and_zero_tokens_reconstruct_exactly(tables):
    """A stream with max = min (every rotated value equal) puts every symbol on
    the central level and reconstructs exactly; a zero token gives zeros."""
    t = tables[K_CFG]
    y = np.full((1, 1024), 2.5)
    x = (fwht(y.reshape(1, 8, 128)) / 128.0)            # rotates back to the constant 2.5
    r = tk.encode_tokens(np.concatenate([x, np.zeros((1, 8, 128))]), t)
    assert np.all(r.symbols == 3)
    xh = tk.reconstruct_tokens(r.symbols, r.o16, r.s16)
    assert np.array_equal(xh[0], x[0]) and np.array_equal(xh[1], np.zeros((8, 128)))


@pytest.mark.parametrize("cfg", [K_CFG, V_CFG])
def test_reconstruction_is_the_inverse_rotation(tables, cfg):
    """x_hat = H (o16 + s16 m) / 128 per head: rotating x_hat forward gives back
    exactly the grid values (H H = 128 I)."""
    t = tables[cfg]
    r = tk.encode_tokens(_tokens(10, S=8), t)
    xh = tk.reconstruct_tokens(r.symbols, r.o16, r.s16)
    yh = r.o16.astype(np.float64)[:, None] + r.s16.astype(np.float64)[:, None] * r.symbols
    assert np.allclose(tk.rotate_tokens(xh), yh, rtol=0, atol=1e-12)


def test_mean_removal_is_undone(tables):
    """With a rotated mean removed before coding and added back after, a
    token that equals its mean reconstructs to it (all-zero residual)."""
    t = tables[K_CFG]
    rng = np.random.default_rng(12)
    mu = rng.standard_normal((3, 1024))
    x = fwht(mu.reshape(3, 8, 128)) / 128.0            # rotates to mu exactly enough
    y = tk.rotate_tokens(x)
    r = tk.encode_tokens(x, t, mean_rot=y)              # residual exactly zero
    assert np.all(r.symbols == 3) and not np.any(r.o16) and not np.any(r.s16)
    xh = tk.reconstruct_tokens(r.symbols, r.o16, r.s16, mean_rot=y)
    assert np.allclose(xh, x, rtol=0, atol=1e-12)


@pytest.mark.parametrize("cfg", [K_CFG, V_CFG])
def test_drift_moves_the_cheapest_distortion_per_bit(tables, cfg):
    """Single-round streams: every moved symbol has a distortion-per-bit key
    (grid units) no larger than any candidate left in place (the Lagrangian
    threshold structure of section 4.3), and undoing the last-moved symbol
    (largest key, then largest index) breaks the container constraint."""
    from oracle.codec import rans_encode
    t = tables[cfg]
    r = tk.encode_tokens(_tokens(13, S=64), t)
    checked = 0
    for i in np.nonzero(r.rounds == 1)[0]:
        m0, m1, u = r.nearest[i], r.symbols[i], r.u[i]
        inner = t.inner[m0]
        cand = (inner >= 0) & (t.cost[m0] > t.cost[np.where(inner >= 0, inner, m0)])
        dr = (t.cost[m0] - t.cost[np.where(cand, inner, m0)]).astype(np.float64)
        key = np.where(cand, ((u - inner) ** 2 - (u - m0) ** 2) / np.where(cand, dr, 1.0), np.inf)
        moved = m1 != m0
        assert np.all(cand[moved])
        if moved.any() and (cand & ~moved).any():
            assert key[moved].max() <= key[cand & ~moved].min()
        j = np.nonzero(moved)[0]
        last = j[np.lexsort((j, key[j]))[-1]]
        back = m1.copy()
        back[last] = m0[last]
        _, ln = rans_encode(back[None], t, t.container)
        assert t.cost[back].sum() > t.budget_fx or ln[0] > t.container
        checked += 1
    assert checked > 0
