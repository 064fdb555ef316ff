"""Synthetic quality studies of the method, computed with the oracle alone.

TEST INFRASTRUCTURE ONLY: analyses of what the method computes, on seeded
i.i.d. N(0,1) rows of 128 values (``default_rng(0)``; after the rotation and
the normalisation the paper's preprocessed KV rows are close to this, section
3.2, Table 1). Nothing here runs on the product path.

1. Reconstruction error against the number of levels at fixed key and value
   budgets (the analysis of the paper's Table 2): for each M, the NMSE at the
   grid step that minimises it, with the fraction of drifted symbols, or "-"
   when no step gives a feasible table (one where every stream fits once all
   its symbols sit at the ends of their drift chains, with a byte of slack).
2. Largest alphabet against the container size (the analysis of Figure 6
   left): the largest M whose grid, at its MSE-optimal uniform step for
   N(0,1), has a mean coded length that fits the container (drift absorbs the
   spread), beside a fixed-width code of the same container charged the ideal
   log2 M bits per value (floor(2^(8C/128)) levels) and a power-of-two code
   width (2^floor(8C/128) levels).
3. Fixed-width comparator at the same container (section 5, fixed-width
   ablation): nearest-level rounding to floor(2^(8C/128)) levels on the same
   symmetric grid and norm, at its own best step, against the drifted
   entropy-coded stream.
4. Drift at the default configurations (Figure 6 right): fraction of symbols
   changed, the per-stream distribution of changed symbols and of the bytes
   left in the container, and the largest move in levels.

    python -m oracle.studies [--rows 20000] > oracle/studies_result.md
"""
from __future__ import annotations

import argparse

import numpy as np

from .codec import encode_streams, fwht, nearest_level, normalize, reconstruct
from .measures import nmse
from .tables import COST_ONE, make_table


def best_step(M: int, C: int, x: np.ndarray, lo: float = 0.15, hi: float = 3.0):
    """(step, NMSE, drifted fraction) minimising NMSE over a 0.05 grid refined
    to 0.01, or None when no step on the grid gives a feasible table."""
    def score(s: float):
        t = make_table(M, C, s)
        if not t.feasible:
            return None
        r = encode_streams(x, t)
        return nmse(x, reconstruct(r.symbols, r.rho16, t)), float(r.changed.sum() / r.symbols.size)

    coarse = [(float(s), score(float(s))) for s in np.round(np.arange(lo, hi + 1e-9, 0.05), 2)]
    coarse = [(s, v) for s, v in coarse if v is not None]
    if not coarse:
        return None
    s0 = min(coarse, key=lambda sv: sv[1][0])[0]
    fine = [(float(s), score(float(s))) for s in np.round(np.arange(s0 - 0.04, s0 + 0.041, 0.01), 2) if s > 0]
    fine = [(s, v) for s, v in fine if v is not None] + [(s0, dict(coarse)[s0])]
    s, (e, d) = min(fine, key=lambda sv: sv[1][0])
    return s, e, d


def uniform_step(M: int, z: np.ndarray) -> float:
    """MSE-minimising step (0.005 grid) of the symmetric M-level uniform grid
    under nearest-level rounding of the sample z."""
    best = None
    for s in np.arange(0.02, 2.5, 0.005):
        idx = np.clip(np.floor(z / s + M / 2.0), 0, M - 1)
        e = float(((z - s * (idx - (M - 1) / 2.0)) ** 2).mean())
        if best is None or e < best[1]:
            best = (float(s), e)
    return best[0]


def coded_rate(M: int, step: float) -> float:
    """Mean coded bits per value of a N(0,1) source on the table built for
    (M, step): sum over levels of the cell mass times the symbol's cost."""
    t = make_table(M, 64, step)
    return float((t.mass * t.cost).sum()) / COST_ONE


def fixed_width(M: int, C: int, x: np.ndarray):
    """Best-step NMSE of plain nearest-level rounding to M levels (no drift,
    no entropy coding); the container and norm are the same as D-Quant's."""
    y = fwht(x)
    _, rho16, z = normalize(y)
    best = None
    for s in np.round(np.arange(0.10, 3.0 + 1e-9, 0.01), 2):
        t = make_table(M, C, float(s))
        e = nmse(x, reconstruct(nearest_level(z, t), rho16, t))
        if best is None or e < best[1]:
            best = (float(s), e)
    return best


def drift_stats(M: int, C: int, x: np.ndarray) -> dict:
    t = make_table(M, C)
    r = encode_streams(x, t)
    ch = r.changed
    moved = np.abs(r.symbols - r.nearest)
    left = C - r.lengths
    edges = [0, 1, 3, 6, 11, 21, 129]
    hist = np.histogram(ch, bins=edges)[0] / ch.size
    ledges = [0, 1, 2, 4, 8, C + 1]
    lhist = np.histogram(left, bins=ledges)[0] / left.size
    return {"changed": float(ch.sum() / r.symbols.size), "streams_drifted": float((ch > 0).mean()),
            "max_move": int(moved.max()), "fallback": int(r.fallback.sum()),
            "nmse": nmse(x, reconstruct(r.symbols, r.rho16, t)),
            "hist": hist, "edges": edges, "left_hist": lhist, "left_edges": ledges}


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--rows", type=int, default=20000)
    args = ap.parse_args()
    x = np.random.default_rng(0).standard_normal((args.rows, 128))
    print("# Synthetic quality studies (oracle, fp64)\n")
    print(f"{args.rows} i.i.d. N(0,1) rows of 128 values, `default_rng(0)`; alpha = 1.4, p = 10. "
          "Command: `python -m oracle.studies`.\n")

    budgets = [("key", 41), ("value", 27)]
    levels = [4, 5, 6, 7, 8, 9, 10, 11, 12, 14]
    print("## 1. NMSE against the number of levels at a fixed container\n")
    print("Best-step NMSE (drifted symbols) per level count; 41-byte key and 27-byte value containers "
          "(2.69 and 1.81 bits per value with the fp16 norm). '-': no step gives a table every stream fits.\n")
    print("| Container | " + " | ".join(f"M={M}" for M in levels) + " |")
    print("|---|" + "---|" * len(levels))
    for name, C in budgets:
        cells = []
        for M in levels:
            r = best_step(M, C, x)
            cells.append("-" if r is None else f"{100 * r[1]:.2f}% ({100 * r[2]:.1f}%, step {r[0]:.2f})")
        print(f"| {name} {C} B | " + " | ".join(cells) + " |", flush=True)

    print("\n## 2. Largest alphabet against the container size\n")
    print("An M-level grid is placed at its MSE-optimal uniform step for N(0,1); it is supported by a "
          "C-byte entropy-coded container when its mean coded length fits, 128 x rate + 24 <= 8C "
          "(drift absorbs the spread around the mean). Fixed-width codes of the same container hold "
          "floor(2^(8C/128)) levels charged the ideal log2 M, or 2^floor(8C/128) as integer-width codes.\n")
    zs = x.reshape(-1)[:400000]
    rates = {}
    for M in range(2, 65):
        rates[M] = coded_rate(M, uniform_step(M, zs))
    print("| C (bytes) | payload bits/value | entropy-coded max M | fixed width, ideal log2 M | fixed width, integer code |")
    print("|---|---|---|---|---|")
    for C in range(12, 66, 4):
        mmax = max([M for M, r in rates.items() if 128 * r + 24 <= 8 * C], default=0)
        b = 8 * C / 128
        print(f"| {C} | {b:.3f} | {mmax} | {int(np.floor(2 ** b))} | {2 ** int(np.floor(b))} |", flush=True)

    print("\n## 3. Fixed-width comparator at the same container\n")
    print("| Container | D-Quant (M, NMSE) | fixed width (M = floor(2^(8C/128)), NMSE, step) |")
    print("|---|---|---|")
    for (name, C), M in ((("key", 41), 8), (("value", 27), 6), (("both", 37), 8), (("both", 37), 6),
                         (("both", 32), 8), (("both", 32), 6)):
        t = make_table(M, C)
        r = encode_streams(x, t)
        e = nmse(x, reconstruct(r.symbols, r.rho16, t))
        Mf = int(np.floor(2 ** (8 * C / 128)))
        s, ef = fixed_width(Mf, C, x)
        print(f"| {name} {C} B | M={M}: {100 * e:.2f}% | M={Mf}: {100 * ef:.2f}% (step {s:.2f}) |", flush=True)

    print("\n## 4. Drift at the default configurations\n")
    print("| (M, C) | symbols changed | streams drifted | largest move (levels) | fallback rounds | NMSE |")
    print("|---|---|---|---|---|---|")
    stats = {}
    for M, C in ((8, 37), (6, 37), (8, 32), (6, 32), (8, 41), (6, 27)):
        d = drift_stats(M, C, x)
        stats[(M, C)] = d
        print(f"| ({M}, {C}) | {100 * d['changed']:.2f}% | {100 * d['streams_drifted']:.1f}% | {d['max_move']} | "
              f"{d['fallback']} | {100 * d['nmse']:.2f}% |", flush=True)
    d0 = next(iter(stats.values()))
    print("\nPer-stream changed symbols (fraction of streams):\n")
    heads = [f"{a}" if b - a == 1 else f"{a}-{b - 1}" for a, b in zip(d0["edges"][:-1], d0["edges"][1:])]
    print("| (M, C) | " + " | ".join(heads) + " |")
    print("|---|" + "---|" * len(heads))
    for (M, C), d in stats.items():
        print(f"| ({M}, {C}) | " + " | ".join(f"{100 * v:.1f}%" for v in d["hist"]) + " |")
    print("\nBytes left unused in the container (fraction of streams):\n")
    print("| (M, C) | 0 | 1 | 2-3 | 4-7 | 8+ |")
    print("|---|---|---|---|---|---|")
    for (M, C), d in stats.items():
        print(f"| ({M}, {C}) | " + " | ".join(f"{100 * v:.1f}%" for v in d["left_hist"]) + " |")


if __name__ == "__main__":
    main()
