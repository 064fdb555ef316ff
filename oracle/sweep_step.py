"""Choose the default grid step per (levels, container) with the oracle alone.

TEST INFRASTRUCTURE ONLY. For each (M, C), every step on a 0.01 grid is
scored by the pooled post-drift NMSE of 20,000 i.i.d. N(0,1) rows of 128
values (``default_rng(0)``), alpha = 1.4, p = 10; the minimiser is printed as
the entry to freeze in ``oracle/tables.py`` (DEFAULT_STEP) and in the C
header's documented defaults.

    python -m oracle.sweep_step [--lo 0.70 --hi 1.40] [--pairs 8:37,6:37]
"""
from __future__ import annotations

import argparse

import numpy as np

from .tables import make_table
from .codec import encode_streams, reconstruct
from .measures import nmse


def score(M: int, C: int, step: float, x: np.ndarray) -> tuple[float, float]:
    t = make_table(M, C, step)
    if not t.feasible:
        return float("inf"), float("nan")
    r = encode_streams(x, t)
    return nmse(x, reconstruct(r.symbols, r.rho16, t)), r.changed.sum() / r.symbols.size


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--lo", type=float, default=0.70)
    ap.add_argument("--hi", type=float, default=1.40)
    ap.add_argument("--rows", type=int, default=20000)
    ap.add_argument("--pairs", default="8:37,6:37,8:32,6:32,8:41,6:27",
                    help="comma-separated levels:container pairs to sweep")
    args = ap.parse_args()
    x = np.random.default_rng(0).standard_normal((args.rows, 128))
    steps = np.round(np.arange(args.lo, args.hi + 1e-9, 0.01), 2)
    best = {}
    pairs = [tuple(int(v) for v in pc.split(":")) for pc in args.pairs.split(",")]
    for M, C in pairs:
        res = [(s, *score(M, C, float(s), x)) for s in steps]
        s_best, e_best, d_best = min(res, key=lambda r: r[1])
        best[(M, C)] = float(s_best)
        print(f"M={M} C={C}: step {s_best:.2f}  NMSE {e_best:.5f}  drifted symbols {d_best:.4f}", flush=True)
        for s, e, d in res:
            print(f"    {s:.2f} {e:.5f} {d:.4f}", flush=True)
    print("DEFAULT_STEP =", best)


if __name__ == "__main__":
    main()
