"""O1 — the static entropy table derived from the standard normal.

TEST INFRASTRUCTURE ONLY (see the package header).

Paper anchors (D-Quant, arXiv 2609.19880):
* section 3.1 "Entropy Coding": ideal cost r(m) = -log2 p_m and the rANS
  pair Enc/Dec built from integer frequencies f_m and cumulative starts c_m
  at precision 2^p;
* section 4.2: reconstruction levels x_hat = o + s*m on an affine grid;
* section 1 and section 3.2: the probability model comes straight from
  N(0,1) because rotated, normalised KV is close to standard normal;
* section 4.4 "Distribution sharpening": p'_m proportional to p_m^alpha,
  alpha > 1 (alpha = 1.4, section 5.1).

Readings where the paper is silent:
* grid: symmetric and uniform in unit-RMS units, level m at
  delta * (m - (M-1)/2); that is the paper's affine grid with o = -delta*(M-1)/2
  and s = delta, the per-token scale being the stored norm;
* p_m is the N(0,1) mass of level m's nearest-neighbour cell (boundaries
  halfway between adjacent levels);
* frequencies: round-half-even of q_m * 2^p for the lower half, floored at
  f_min = 2^(p-8), raised where needed so that a cell the model makes
  strictly more probable than its outer neighbour keeps a strictly larger
  frequency, mirrored, the (even) residual split equally over the two
  central levels (or given to the single central level when M is odd);
* costs are fixed point with 16 fractional bits, cost(m) = rint((p - log2 f_m) * 2^16);
* the rANS state lives in [2^16, 2^24) with byte renormalisation, flushed as
  3 bytes, so the fixed container overhead sigma of section 4.2 is 24 bits.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

STATE_LOW_BITS = 16
STATE_LOW = 1 << STATE_LOW_BITS       # L: lower end of the rANS state interval
STATE_BYTES = 3                       # the state [2^16, 2^24) is flushed as 3 bytes
FLUSH_BITS = 8 * STATE_BYTES          # sigma in B = 8C - sigma (section 4.2)
COST_FRAC_BITS = 16
COST_ONE = 1 << COST_FRAC_BITS        # one bit in fixed-point cost units
HEAD_DIM = 128

# Grid steps (unit-RMS units) that minimise the pooled post-drift NMSE of
# 20,000 i.i.d. N(0,1) streams of 128 values (seed 0) on a 0.01 grid, with
# alpha = 1.4 and p = 10. Written by oracle/sweep_step.py.
DEFAULT_STEP = {
    (8, 37): 0.92,
    (6, 37): 0.90,
    (8, 32): 1.12,
    (6, 32): 1.09,
    (8, 41): 0.79,
    (6, 27): 1.34,
}


def default_step(levels: int, container: int) -> float:
    """The frozen default grid step for (M, C); raises KeyError if none was swept."""
    return DEFAULT_STEP[(levels, container)]


def _phi(x: float) -> float:
    """Standard normal CDF via erfc (accurate in the lower tail)."""
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


@dataclass
class Table:
    """One static entropy table (keys and values each get their own)."""
    levels: int          # M
    container: int       # C, bytes per stream
    step: float          # delta
    alpha: float
    prob_bits: int       # p
    n: int               # symbols per stream
    recon: np.ndarray    # [M] float64, level value in unit-RMS units
    bounds: np.ndarray   # [M-1] float64, decision boundaries b_1..b_{M-1}
    mass: np.ndarray     # [M] float64, N(0,1) cell masses
    sharpened: np.ndarray  # [M] float64, p^alpha normalised
    freq: np.ndarray     # [M] int64, f_m, sums to 2^p
    cum: np.ndarray      # [M+1] int64, c_m = sum_{j<m} f_j
    cost: np.ndarray     # [M] int64, fixed-point cost of each symbol
    sym: np.ndarray      # [2^p] int64, slot -> symbol
    inner: np.ndarray    # [M] int64, drift target of each level (-1: none)
    f_min: int
    budget_fx: int       # (8C - sigma) * 2^16
    feasible: bool
    notes: list = field(default_factory=list)

    @property
    def total(self) -> int:
        return 1 << self.prob_bits


def make_table(levels: int, container: int, step: float | None = None, alpha: float = 1.4,
               prob_bits: int = 10, n: int = HEAD_DIM) -> Table:
    """Build the table for M levels and a C-byte container (O1)."""
    M, C, p = int(levels), int(container), int(prob_bits)
    if step is None:
        step = default_step(M, C)
    if M < 2:
        raise ValueError("need at least two levels")
    total = 1 << p
    f_min = 1 << (p - 8)

    # levels delta * (m - (M-1)/2), symmetric about zero
    half = (M - 1) / 2.0
    recon = np.array([step * (m - half) for m in range(M)], dtype=np.float64)
    bounds = np.array([(recon[j - 1] + recon[j]) / 2.0 for j in range(1, M)], dtype=np.float64)

    # N(0,1) mass of each level's nearest-neighbour cell. Lower half from the
    # CDF at negative boundaries (accurate), upper half by symmetry.
    mass = np.zeros(M)
    for m in range(M // 2):
        lo = 0.0 if m == 0 else _phi(bounds[m - 1])
        hi = 0.5 if (M % 2 == 0 and m == M // 2 - 1) else _phi(bounds[m])
        mass[m] = hi - lo
        mass[M - 1 - m] = mass[m]
    if M % 2 == 1:
        c = M // 2
        mass[c] = math.erf(-bounds[c - 1] / math.sqrt(2.0))  # 1 - 2*Phi(b) for the central cell

    # sharpening p' ~ p^alpha (section 4.4), normalised by a left-to-right sum
    w = [math.pow(float(mm), alpha) for mm in mass]
    s = 0.0
    for v in w:
        s += v
    sharpened = np.array([v / s for v in w])

    # integer frequencies at precision 2^p. Rounding and the floor must not
    # erase the model's order: going inward, a level whose cell is strictly
    # more probable than its outer neighbour's keeps at least one more unit.
    freq = np.zeros(M, dtype=np.int64)
    for m in range(M // 2):
        f = max(f_min, int(round(sharpened[m] * total)))   # round() is half-even
        if m > 0 and mass[m] > mass[m - 1]:
            f = max(f, int(freq[m - 1]) + 1)
        freq[m] = f
        freq[M - 1 - m] = f
    notes = []
    if M % 2 == 0:
        resid = total - int(freq.sum())
        freq[M // 2 - 1] += resid // 2
        freq[M // 2] += resid // 2
    else:
        freq[M // 2] = total - int(freq.sum())
    cum = np.zeros(M + 1, dtype=np.int64)
    cum[1:] = np.cumsum(freq)

    feasible = bool(np.all(freq >= f_min) and cum[-1] == total)
    if not feasible:
        notes.append("frequency below f_min after the residual")
    cost = np.array([int(round((p - math.log2(int(f))) * COST_ONE)) if f > 0 else 0 for f in freq],
                    dtype=np.int64)

    sym = np.zeros(total, dtype=np.int64)
    for m in range(M):
        sym[cum[m]:cum[m + 1]] = m

    # drift target: the nearest level toward zero whose cost is strictly lower
    # (section 4.3: expensive symbols drift to nearby cheaper ones). The
    # frequencies keep the model's strict order, so wherever the N(0,1) cells
    # get less probable outward (every configured table) this is the adjacent
    # inner level. The walk stops after the first level at or across zero; -1
    # means the level never drifts.
    inner = np.full(M, -1, dtype=np.int64)
    for m in range(M):
        d = -1 if recon[m] > 0 else (1 if recon[m] < 0 else 0)
        j = m + d
        while d != 0 and 0 <= j < M:
            if cost[j] < cost[m]:
                inner[m] = j
                break
            if recon[j] * recon[m] <= 0:
                break
            j += d

    budget_fx = (8 * C - FLUSH_BITS) * COST_ONE
    # Drift moves a symbol only to its (strictly cheaper) drift target, so
    # from level m it can at most reach the end of that chain. Every stream
    # must fit once all its symbols sit at such terminal levels, with a byte
    # of rANS slack. (Where costs grow outward every chain ends at a central
    # level.)
    worst = 0
    if feasible:
        for m in range(M):
            cur = m
            while inner[cur] >= 0:
                cur = int(inner[cur])
            worst = max(worst, int(cost[cur]))
    if feasible and n * worst + 8 * COST_ONE > budget_fx:
        feasible = False
        notes.append("a stream of drift-terminal levels does not fit the container")

    return Table(levels=M, container=C, step=float(step), alpha=float(alpha), prob_bits=p, n=n,
                 recon=recon, bounds=bounds, mass=mass, sharpened=sharpened, freq=freq, cum=cum,
                 cost=cost, sym=sym, inner=inner, f_min=f_min, budget_fx=budget_fx,
                 feasible=feasible, notes=notes)
