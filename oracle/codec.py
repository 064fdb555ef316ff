"""O2-O10 — the D-Quant cache-write codec and its decoder, in fp64 and exact ints.

TEST INFRASTRUCTURE ONLY (see the package header).

Paper anchors (D-Quant, arXiv 2609.19880):
* section 4.1: each token's key (or value) is rotated (Hadamard), normalised,
  quantised on an affine grid and entropy coded into a fixed-size container;
* section 3.1, the Enc/Dec equations of rANS:
      Enc(x, m) = floor(x / f_m) * 2^p + (x mod f_m) + c_m
      Dec(x, m) = f_m * floor(x / 2^p) + (x mod 2^p) - c_m
* section 4.2: the container constraint sum_i r(m_i) <= B with B = 8C - sigma;
* section 4.3 "Drift": minimise sum_i (x_i - x_hat(m_i))^2 subject to that
  constraint; only a few values move from an expensive symbol to a nearby
  cheaper one; section 1 solves it with a Lagrangian and bisection;
* appendix, paragraph "Drift makes only sparse, local corrections": the
  paper observes that every symbol drift changes lands on a neighbouring
  reconstruction level, never further away.

Readings: one stream is the 128 channels of one
(token, KV head); the per-token scale is the L2 norm stored as fp16; the
drift candidates are the one-level inward moves; the Lagrangian solution is
computed exactly as the minimal prefix of candidates sorted by
(distortion increase / rate decrease, channel index) - which is what a
bisection on the multiplier converges to; rANS details as in ``tables``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .tables import Table, STATE_LOW, STATE_BYTES, HEAD_DIM

# ----------------------------------------------------------------------------
# O2 rotation


def fwht(x: np.ndarray) -> np.ndarray:
    """y = H x with H the 128-point Sylvester Hadamard matrix (entries +-1).

    In-place butterflies for h = 1, 2, 4, ..., 64: every pair (i, i+h) with
    i mod 2h < h becomes (a + b, a - b). fp64, applied along the last axis.
    """
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < n:
        y = y.reshape(lead + (n // (2 * h), 2, h))
        a = y[..., 0, :]
        b = y[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2)
        h *= 2
    return y.reshape(lead + (n,))


# ----------------------------------------------------------------------------
# O3 normalisation


def tree_sum_squares(y: np.ndarray) -> np.ndarray:
    """S = sum_j y_j^2 by a fixed binary tree: s_j = y_j*y_j, then for
    w = 64, 32, ..., 1: s_j <- s_j + s_{j+w} for j < w. Returns s_0."""
    s = y * y
    w = y.shape[-1] // 2
    while w >= 1:
        s[..., :w] = s[..., :w] + s[..., w:2 * w]
        w //= 2
    return s[..., 0].copy()


def normalize(y: np.ndarray):
    """Per-stream norm and unit-RMS values.

    S = tree sum of y^2; rho = sqrt(S / 128) (the L2 norm of the unrotated
    row, since H^T H = 128 I); rho16 = rho rounded once to fp16 (nearest
    even); z = y / rho so that sum z^2 = 128. A zero row gives z = 0, rho16 = 0.
    Returns (rho float64 [S], rho16 float16 [S], z float64 [S, 128]).
    """
    S = tree_sum_squares(y)
    n = y.shape[-1]
    rho = np.sqrt(S / n)
    with np.errstate(over="ignore"):
        rho16 = rho.astype(np.float16)
    z = np.zeros_like(y)
    nz = S > 0
    z[nz] = y[nz] / rho[nz, None]
    return rho, rho16, z


# ----------------------------------------------------------------------------
# O4 nearest level, O5 cost


def nearest_level(z: np.ndarray, table: Table) -> np.ndarray:
    """Index of the nearest level; an exact midpoint goes to the inner level.

    m = #{j : z > b_j for b_j >= 0, z >= b_j for b_j < 0}. With M even, z = 0
    (the central midpoint) goes to index M/2 - 1.
    """
    m = np.zeros(z.shape, dtype=np.int64)
    for b in table.bounds:
        if b >= 0:
            m += (z > b)
        else:
            m += (z >= b)
    return m


def stream_cost(m: np.ndarray, table: Table) -> np.ndarray:
    """R = sum_i cost(m_i) in fixed-point units (exact)."""
    return table.cost[m].sum(axis=-1)


# ----------------------------------------------------------------------------
# O6 drift candidates


def drift_candidates(z: np.ndarray, m: np.ndarray, table: Table):
    """Candidate moves of one drift round, for a batch of streams.

    A symbol is a candidate when its level has an inward neighbour m' that is
    strictly cheaper: dr = cost(m) - cost(m') > 0. Its distortion increase is
    dd = (z - level(m'))^2 - (z - level(m))^2 and its key is dd / dr (fp64).
    Candidates are ordered by (key, channel index).

    Returns (order [S, n] int64: channel indices, candidates first in key order;
             n_cand [S]; dr_sorted [S, n] int64 (0 past n_cand); inner [S, n]).
    """
    inner = table.inner[m]
    has = inner >= 0
    inner_safe = np.where(has, inner, m)
    dr = np.where(has, table.cost[m] - table.cost[inner_safe], 0)
    cand = has & (dr > 0)
    lv_new = table.recon[inner_safe]
    lv_old = table.recon[m]
    dd = (z - lv_new) * (z - lv_new) - (z - lv_old) * (z - lv_old)
    key = np.full(z.shape, np.inf)
    key[cand] = dd[cand] / dr[cand].astype(np.float64)
    # stable sort on the key keeps equal keys in ascending channel order
    order = np.argsort(key, axis=-1, kind="stable")
    n_cand = cand.sum(axis=-1)
    dr_sorted = np.take_along_axis(np.where(cand, dr, 0), order, axis=-1)
    return order, n_cand, dr_sorted, inner


# ----------------------------------------------------------------------------
# O7 rANS encode, O9 rANS decode


def rans_enc_step(x, m, table: Table):
    """One rANS encode step (section 3.1): Enc(x, m) = floor(x/f_m) 2^p + (x mod f_m) + c_m.

    The caller has renormalised x into [f_m 2^(16-p), f_m 2^(24-p))."""
    f = table.freq[m]
    return (x // f) * (1 << table.prob_bits) + (x % f) + table.cum[m]


def rans_dec_step(x, table: Table):
    """One rANS decode step (section 3.1): the symbol m owning slot x mod 2^p,
    and Dec(x, m) = f_m floor(x / 2^p) + (x mod 2^p) - c_m. Returns (m, x')."""
    p = table.prob_bits
    slot = x & ((1 << p) - 1)
    m = table.sym[slot]
    return m, table.freq[m] * (x >> p) + slot - table.cum[m]


def rans_encode(m: np.ndarray, table: Table, capacity: int | None = None):
    """Encode each row of symbols into one rANS container.

    State x starts at L = 2^16. For i = n-1 down to 0 (so that the decoder
    emits channel 0 first): while x >= 2^(24-p) * f the low byte is emitted
    and x >>= 8 (at most once, because f >= 2^(p-8)); then x = Enc(x, m_i).
    The final state is flushed as 3 little-endian bytes at offset 0, followed
    by the emitted bytes in the order the decoder reads them, then zeros.

    Returns (containers uint8 [S, capacity], lengths int64 [S]). Rows whose
    length exceeds ``capacity`` are truncated (the caller checks lengths).
    """
    m = np.atleast_2d(m)
    S, n = m.shape
    p = table.prob_bits
    if capacity is None:
        capacity = STATE_BYTES + n
    x = np.full(S, STATE_LOW, dtype=np.int64)
    emitted = np.zeros((S, n), dtype=np.int64)
    count = np.zeros(S, dtype=np.int64)
    rows = np.arange(S)
    x_max_unit = (STATE_LOW >> p) << 8
    for i in range(n - 1, -1, -1):
        f = table.freq[m[:, i]]
        emit = x >= x_max_unit * f
        emitted[rows[emit], count[emit]] = x[emit] & 0xFF
        count += emit
        x = np.where(emit, x >> 8, x)
        x = rans_enc_step(x, m[:, i], table)
    lengths = STATE_BYTES + count
    out = np.zeros((S, max(capacity, STATE_BYTES + n)), dtype=np.uint8)
    out[:, 0] = x & 0xFF
    out[:, 1] = (x >> 8) & 0xFF
    out[:, 2] = (x >> 16) & 0xFF
    # bytes were emitted last-symbol first; the decoder wants them reversed
    for j in range(n):
        src = count - 1 - j
        ok = src >= 0
        out[rows[ok], STATE_BYTES + j] = emitted[rows[ok], src[ok]]
    return out[:, :capacity].copy(), lengths


def rans_decode(containers: np.ndarray, table: Table, n: int = HEAD_DIM):
    """Decode n symbols from each container (the inverse of ``rans_encode``).

    x = b0 | b1 << 8 | b2 << 16, then for each symbol: slot = x mod 2^p,
    m = the symbol owning slot, x = Dec(x, m), and while x < L one byte is
    shifted in. Returns (symbols [S, n], final state [S], bytes consumed [S],
    renorm_ok [S]: no step needed two renormalisation bytes).
    """
    b = np.atleast_2d(containers).astype(np.int64)
    S, cap = b.shape
    pad = np.zeros((S, cap + n + 1), dtype=np.int64)   # reads past the container see zeros
    pad[:, :cap] = b
    x = pad[:, 0] | (pad[:, 1] << 8) | (pad[:, 2] << 16)
    ptr = np.full(S, STATE_BYTES, dtype=np.int64)
    rows = np.arange(S)
    out = np.zeros((S, n), dtype=np.int64)
    ok = np.ones(S, dtype=bool)
    for i in range(n):
        s, x = rans_dec_step(x, table)
        need = x < STATE_LOW
        x = np.where(need, (x << 8) | pad[rows, ptr], x)
        ptr = ptr + need
        ok &= ~(x < STATE_LOW)
        out[:, i] = s
    return out, x, ptr, ok


# ----------------------------------------------------------------------------
# O4-O8 the whole cache write


@dataclass
class EncodeResult:
    containers: np.ndarray   # uint8 [S, C]
    rho16: np.ndarray        # float16 [S]
    symbols: np.ndarray      # int64 [S, n]: symbols actually stored
    nearest: np.ndarray      # int64 [S, n]: nearest-level symbols before drift
    lengths: np.ndarray      # int64 [S]: bytes used, <= C
    rounds: np.ndarray       # int64 [S]: drift rounds taken (0 = no drift needed)
    z: np.ndarray            # float64 [S, n]: unit-RMS rotated values
    rho: np.ndarray          # float64 [S]

    @property
    def changed(self) -> np.ndarray:
        """Per-stream count of symbols the drift changed."""
        return (self.symbols != self.nearest).sum(axis=-1)

    @property
    def fallback(self) -> np.ndarray:
        """Streams that needed more than one drift round."""
        return self.rounds > 1


def _apply_prefix(m, order, inner_of_level, k):
    """Move the first k candidates (in key order) of each row one level inward."""
    out = m.copy()
    S, n = m.shape
    sel = np.arange(n)[None, :] < k[:, None]
    r, j = np.nonzero(sel)
    idx = order[r, j]
    out[r, idx] = inner_of_level[m[r, idx]]
    return out


def encode_streams(x: np.ndarray, table: Table, mean_rot: np.ndarray | None = None) -> EncodeResult:
    """Encode rows x [S, 128] (values exactly representable in fp64) into
    fixed C-byte containers plus an fp16 norm each. With ``mean_rot`` [S, 128]
    (a key block's dequantised channel mean, O12) the rotated row minus that
    mean is what gets normalised and coded.

    Steps, per stream: y = H x (O2); S, rho, rho16, z (O3); nearest level (O4);
    R = sum of costs and B_fx = (8C - sigma) * 2^16 (O5). Then drift rounds
    (O6-O8): order the candidates by (key, index); start from the smallest
    prefix k0 with R - sum of its rate decreases <= B_fx; encode (O7) with the
    first k moves for k = k0, k0+1, ... until the container fits. If even all
    candidates fail (or k0 does not exist) the round ends with all of them
    moved and a new round starts from those symbols (a fallback that can move
    a symbol by more than one level; the table guarantees it terminates).
    """
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    S, n = x.shape
    C = table.container
    y = fwht(x)
    if mean_rot is not None:
        y = y - np.asarray(mean_rot, dtype=np.float64)
    rho, rho16, z = normalize(y)
    nearest = nearest_level(z, table)

    m = nearest.copy()
    containers = np.zeros((S, C), dtype=np.uint8)
    lengths = np.zeros(S, dtype=np.int64)
    rounds = np.zeros(S, dtype=np.int64)
    done = np.zeros(S, dtype=bool)

    # streams already within budget whose container fits need no drift
    R = stream_cost(m, table)
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
        zi, mi = z[act], m[act]
        order, n_cand, dr_sorted, _ = drift_candidates(zi, mi, table)
        Ri = stream_cost(mi, table)
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
        # rounds that did not fit: all candidates move, next round
        nf = np.nonzero(~fitted)[0]
        if len(nf):
            if np.any(n_cand[nf] == 0):
                raise RuntimeError("stream cannot fit its container")
            m[act[nf]] = _apply_prefix(mi[nf], order[nf], table.inner, n_cand[nf])

    return EncodeResult(containers=containers, rho16=rho16, symbols=m, nearest=nearest,
                        lengths=lengths, rounds=rounds, z=z, rho=rho)


def decode_streams(containers: np.ndarray, table: Table, n: int = HEAD_DIM):
    """O9: symbols of each container, with the integrity flags.

    Returns (symbols [S, n], ok [S]) where ok means the final state equals
    L, no step needed two bytes, and no byte past the container was read.
    """
    sym, x, ptr, renorm_ok = rans_decode(containers, table, n)
    ok = (x == STATE_LOW) & renorm_ok & (ptr <= containers.shape[-1])
    return sym, ok


def reconstruct(symbols: np.ndarray, rho16: np.ndarray, table: Table,
                mean_rot: np.ndarray | None = None) -> np.ndarray:
    """O10: x_hat = H (rho16 * level(m) [+ mean_rot]) / 128, back in the
    original domain.

    rho16 * level(m) approximates y = H x (the unnormalised rotation), or
    y minus a key block's channel mean (O12), which is then added back; since
    H H = 128 I the inverse rotation is H / 128.
    """
    yhat = np.asarray(rho16, dtype=np.float64)[..., None] * table.recon[symbols]
    if mean_rot is not None:
        yhat = yhat + np.asarray(mean_rot, dtype=np.float64)
    return fwht(yhat) / yhat.shape[-1]
