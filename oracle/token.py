"""O13-O17 — the per-token stream format: one stream of 1024 values per token
(all 8 KV heads), a token-wise min-max affine grid, drift, rANS, and a
least-squares refit of (o, s) stored in fp16.

TEST INFRASTRUCTURE ONLY (see the package header).

Paper anchors (D-Quant, arXiv 2609.19880):
* section 4.2: the affine grid x_hat = o + s*m, m in {0, .., M-1}, and the
  container constraint sum_i r(m_i) <= 8C - sigma;
* section 4.3: the drift objective, squared error on that grid;
* section 4.5 "Encoding": one wave per stream, the final affine refit and the
  rANS encode in the same wave;
* section 5.1: 331- and 231-byte key / value containers with 8 / 6 levels,
  each token quantised as one group of 1024 values;
* appendix, paragraph "Compared configurations": the format the paper
  measures groups each token on its own, sets its affine grid from the
  token's minimum and maximum, refits that grid by least squares and keeps
  the grid parameters as two fp16 numbers.

Readings:
* the stream is the 8 heads' rotated values in head-major order, each head
  rotated by its own 128-point Hadamard (y = H x, unnormalised);
* the grid is min-max over the stream: o = min y, s = (max y - min y)/(M-1),
  both fp64; u = (y - o)/s is the value in grid units and the nearest level
  is taken in u, an exact midpoint going to the level nearer the grid centre;
  a stream with max = min has every symbol at level (M-1)//2;
* the entropy table is the N(0,1) table of the symmetric M-level grid whose
  step is the min-max grid of an average stream: 2 e_n / (M - 1), e_n the
  expected maximum of n = 1024 i.i.d. N(0,1) values;
* drift distances are taken in grid units: moving a value from level m to m'
  costs (u - m')^2 - (u - m)^2 (the objective of section 4.3 divided by s^2,
  which leaves every comparison unchanged); candidates, ordering and rounds
  are those of the per-head coder (O6-O8);
* the refit is the least-squares line through (m_i, y_i) over the final
  symbols, its sums taken by a fixed halving tree; (o*, s*) are each rounded
  once to fp16 (nearest even); with all symbols equal, s* = 0 and o* is the
  mean.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from .codec import fwht, rans_decode, rans_encode
from .tables import STATE_LOW, Table, make_table

TOKEN_HEADS = 8
TOKEN_N = TOKEN_HEADS * 128


# ----------------------------------------------------------------------------
# O13 the static table of the min-max grid


def expected_max(n: int, steps: int = 40000, lo: float = -12.0, hi: float = 12.0) -> float:
    """e_n = E[max of n i.i.d. N(0,1)] = integral of x n phi(x) Phi(x)^(n-1) dx,
    by the composite Simpson rule on [lo, hi] (the integrand is below 1e-30
    outside it for the n used here)."""
    if steps % 2:
        steps += 1
    h = (hi - lo) / steps
    total = 0.0
    for i in range(steps + 1):
        x = lo + i * h
        phi = math.exp(-0.5 * x * x) / math.sqrt(2.0 * math.pi)
        cdf = 0.5 * math.erfc(-x / math.sqrt(2.0))
        f = x * n * phi * cdf ** (n - 1)
        w = 1.0 if i in (0, steps) else (4.0 if i % 2 else 2.0)
        total += w * f
    return total * h / 3.0


def token_step(levels: int, n: int = TOKEN_N) -> float:
    """Grid step, in N(0,1) units, of the min-max grid of an average stream."""
    return 2.0 * expected_max(n) / (levels - 1)


def make_token_table(levels: int, container: int, alpha: float = 1.4, prob_bits: int = 10,
                     step: float | None = None) -> Table:
    """O13: the entropy table of the per-token format (1024 symbols per stream)."""
    return make_table(levels, container, token_step(levels) if step is None else step, alpha, prob_bits,
                      n=TOKEN_N)


# ----------------------------------------------------------------------------
# O14 rotation, grid and nearest level


def rotate_tokens(x: np.ndarray) -> np.ndarray:
    """x [S, 8, 128] -> y [S, 1024]: each head's y = H x, heads in order."""
    x = np.asarray(x, dtype=np.float64)
    return fwht(x).reshape(x.shape[0], TOKEN_N)


def fold_sum(v: np.ndarray) -> np.ndarray:
    """Sum over the last axis (a power of two) by halving: v_j <- v_j + v_{j+w}
    for j < w, w = n/2, n/4, .., 1. Returns v_0."""
    s = np.array(v, dtype=np.float64, copy=True)
    w = s.shape[-1] // 2
    while w >= 1:
        s[..., :w] = s[..., :w] + s[..., w:2 * w]
        w //= 2
    return s[..., 0].copy()


def grid_index(u: np.ndarray, levels: int) -> np.ndarray:
    """Nearest level of u on the grid 0..M-1; an exact midpoint j - 1/2 goes
    to the level nearer the centre (M-1)/2 (to the lower level at the centre
    itself)."""
    half = (levels - 1) / 2.0
    m = np.zeros(np.shape(u), dtype=np.int64)
    for j in range(1, levels):
        b = j - 0.5
        m += (u > b) if b >= half else (u >= b)
    return m


def affine_grid(y: np.ndarray, levels: int):
    """Min-max grid of each stream: (o [S], s [S], u [S, n]); u = 0 where s = 0."""
    o = y.min(axis=-1)
    s = (y.max(axis=-1) - o) / (levels - 1)
    u = np.zeros_like(y)
    nz = s > 0
    u[nz] = (y[nz] - o[nz, None]) / s[nz, None]
    return o, s, u


# ----------------------------------------------------------------------------
# O15 drift in grid units


def drift_candidates_u(u: np.ndarray, m: np.ndarray, table: Table):
    """Candidate moves of one drift round: m -> inner[m] where that is strictly
    cheaper; distortion increase (u - m')^2 - (u - m)^2, key = increase / rate
    decrease (fp64), ordered by (key, index). Same returns as O6."""
    inner = table.inner[m]
    has = inner >= 0
    inner_safe = np.where(has, inner, m)
    dr = np.where(has, table.cost[m] - table.cost[inner_safe], 0)
    cand = has & (dr > 0)
    a = u - inner_safe.astype(np.float64)
    b = u - m.astype(np.float64)
    dd = a * a - b * b
    key = np.full(u.shape, np.inf)
    key[cand] = dd[cand] / dr[cand].astype(np.float64)
    order = np.argsort(key, axis=-1, kind="stable")
    n_cand = cand.sum(axis=-1)
    dr_sorted = np.take_along_axis(np.where(cand, dr, 0), order, axis=-1)
    return order, n_cand, dr_sorted


def _apply_prefix(m, order, inner_of_level, k):
    out = m.copy()
    n = m.shape[1]
    r, j = np.nonzero(np.arange(n)[None, :] < k[:, None])
    idx = order[r, j]
    out[r, idx] = inner_of_level[m[r, idx]]
    return out


# ----------------------------------------------------------------------------
# O16 refit


def refit(y: np.ndarray, m: np.ndarray):
    """Least-squares (o*, s*) of y ~ o + s m per stream, sums by fold_sum:
    mbar = sum m / n, ybar = sum y / n, Smm = sum (m - mbar)^2,
    Smy = sum (m - mbar)(y - ybar), s* = Smy / Smm, o* = ybar - s* mbar
    (s* = 0, o* = ybar when Smm = 0). Returns (o*, s*, o16, s16)."""
    n = y.shape[-1]
    mf = m.astype(np.float64)
    mbar = fold_sum(mf) / n
    ybar = fold_sum(y) / n
    dm = mf - mbar[:, None]
    dy = y - ybar[:, None]
    smm = fold_sum(dm * dm)
    smy = fold_sum(dm * dy)
    s_star = np.zeros_like(smm)
    nz = smm > 0
    s_star[nz] = smy[nz] / smm[nz]
    o_star = ybar - s_star * mbar
    with np.errstate(over="ignore"):
        return o_star, s_star, o_star.astype(np.float16), s_star.astype(np.float16)


# ----------------------------------------------------------------------------
# O17 the whole per-token cache write, its decoder and reconstruction


@dataclass
class TokenEncodeResult:
    containers: np.ndarray   # uint8 [S, C]
    o16: np.ndarray          # float16 [S]: refit offset
    s16: np.ndarray          # float16 [S]: refit step
    symbols: np.ndarray      # int64 [S, 1024]
    nearest: np.ndarray      # int64 [S, 1024]
    lengths: np.ndarray      # int64 [S]
    rounds: np.ndarray       # int64 [S]
    y: np.ndarray            # float64 [S, 1024]: rotated values (minus the mean, if any)
    o: np.ndarray            # float64 [S]: min-max grid offset
    s: np.ndarray            # float64 [S]: min-max grid step
    u: np.ndarray            # float64 [S, 1024]: grid units

    @property
    def changed(self) -> np.ndarray:
        return (self.symbols != self.nearest).sum(axis=-1)


def encode_tokens(x: np.ndarray, table: Table, mean_rot: np.ndarray | None = None) -> TokenEncodeResult:
    """Encode tokens x [S, 8, 128] into C-byte containers plus fp16 (o, s).

    Per stream: y (O14), minus ``mean_rot`` [S, 1024] if given; the min-max
    grid and nearest levels; then the drift rounds of the per-head coder
    (smallest prefix k0 of the (key, index)-ordered candidates whose rate
    decreases bring R under B_fx, then k0, k0+1, .. until the rANS stream
    fits; all candidates move and a new round starts if none fits); finally
    the refit of (o, s) to the stored symbols (O16).
    """
    y = rotate_tokens(x)
    if mean_rot is not None:
        y = y - np.asarray(mean_rot, dtype=np.float64)
    S, n = y.shape
    M, C = table.levels, table.container
    o, s, u = affine_grid(y, M)
    nearest = grid_index(u, M)
    nearest[s == 0] = (M - 1) // 2

    m = nearest.copy()
    containers = np.zeros((S, C), dtype=np.uint8)
    lengths = np.zeros(S, dtype=np.int64)
    rounds = np.zeros(S, dtype=np.int64)
    done = np.zeros(S, dtype=bool)

    R = table.cost[m].sum(axis=-1)
    under = R <= table.budget_fx
    if np.any(under):
        idx = np.nonzero(under)[0]
        cont, ln = rans_encode(m[idx], table, C)
        fit = ln <= C
        containers[idx[fit]] = cont[fit]
        lengths[idx[fit]] = ln[fit]
        done[idx[fit]] = True

    while not np.all(done):
        act = np.nonzero(~done)[0]
        rounds[act] += 1
        if np.any(rounds[act] > 64):
            raise RuntimeError("drift did not converge")
        ui, mi = u[act], m[act]
        order, n_cand, dr_sorted = drift_candidates_u(ui, mi, table)
        Ri = table.cost[mi].sum(axis=-1)
        csum = np.concatenate([np.zeros((len(act), 1), np.int64), np.cumsum(dr_sorted, axis=1)], 1)
        ok_k = (Ri[:, None] - csum) <= table.budget_fx
        ok_k &= np.arange(n + 1)[None, :] <= n_cand[:, None]
        has_k0 = ok_k.any(axis=1)
        k = np.where(has_k0, np.argmax(ok_k, axis=1), n_cand)
        trying = has_k0.copy()
        fitted = np.zeros(len(act), dtype=bool)
        while np.any(trying):
            t = np.nonzero(trying)[0]
            mt = _apply_prefix(mi[t], order[t], table.inner, k[t])
            cont, ln = rans_encode(mt, table, C)
            fit = ln <= C
            g = act[t[fit]]
            containers[g] = cont[fit]
            lengths[g] = ln[fit]
            m[g] = mt[fit]
            done[g] = True
            fitted[t[fit]] = True
            trying[t[fit]] = False
            nf = t[~fit]
            k[nf] += 1
            trying[nf[k[nf] > n_cand[nf]]] = False
        nf = np.nonzero(~fitted)[0]
        if len(nf):
            if np.any(n_cand[nf] == 0):
                raise RuntimeError("stream cannot fit its container")
            m[act[nf]] = _apply_prefix(mi[nf], order[nf], table.inner, n_cand[nf])

    _, _, o16, s16 = refit(y, m)
    return TokenEncodeResult(containers=containers, o16=o16, s16=s16, symbols=m, nearest=nearest,
                             lengths=lengths, rounds=rounds, y=y, o=o, s=s, u=u)


def decode_tokens(containers: np.ndarray, table: Table):
    """Symbols [S, 1024] of each container and its integrity flag (final state
    L, no double renormalisation, no byte read past the container)."""
    sym, x, ptr, renorm_ok = rans_decode(containers, table, TOKEN_N)
    ok = (x == STATE_LOW) & renorm_ok & (ptr <= containers.shape[-1])
    return sym, ok


def reconstruct_tokens(symbols: np.ndarray, o16: np.ndarray, s16: np.ndarray,
                       mean_rot: np.ndarray | None = None) -> np.ndarray:
    """x_hat [S, 8, 128]: y_hat = o16 + s16 m (+ mean_rot), then each head's
    H y_hat / 128 (H H = 128 I)."""
    yhat = (np.asarray(o16, dtype=np.float64)[:, None]
            + np.asarray(s16, dtype=np.float64)[:, None] * symbols.astype(np.float64))
    if mean_rot is not None:
        yhat = yhat + np.asarray(mean_rot, dtype=np.float64)
    S = yhat.shape[0]
    return fwht(yhat.reshape(S, TOKEN_HEADS, 128)) / 128.0
