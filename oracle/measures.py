"""Rate and distortion measures the paper defines (D-Quant section 3.1, 3.2).

TEST INFRASTRUCTURE ONLY (see the package header).

* ideal cost of a symbol: r(m) = -log2 p_m; its expectation is the entropy H;
* Coding Gain = log2 M - H (saving of entropy coding over fixed width);
* Normal Gap = CE - H, the excess of coding with an N(0,1)-derived model
  instead of the empirical one (CE = cross-entropy);
* NMSE = ||x - x_hat||^2 / ||x||^2 (pooled over the rows given).
"""
from __future__ import annotations

import numpy as np


def entropy(p: np.ndarray) -> float:
    p = np.asarray(p, dtype=np.float64)
    p = p[p > 0]
    return float(-(p * np.log2(p)).sum())


def histogram(symbols: np.ndarray, levels: int) -> np.ndarray:
    """Empirical symbol distribution."""
    h = np.bincount(np.asarray(symbols).ravel(), minlength=levels).astype(np.float64)
    return h / h.sum()


def cross_entropy(p_emp: np.ndarray, model: np.ndarray) -> float:
    """-sum_m p_emp(m) log2 model(m)."""
    p_emp = np.asarray(p_emp, dtype=np.float64)
    model = np.asarray(model, dtype=np.float64)
    nz = p_emp > 0
    return float(-(p_emp[nz] * np.log2(model[nz])).sum())


def coding_gain(p_emp: np.ndarray) -> float:
    return float(np.log2(len(p_emp)) - entropy(p_emp))


def normal_gap(p_emp: np.ndarray, model: np.ndarray) -> float:
    return cross_entropy(p_emp, model) - entropy(p_emp)


def nmse(x: np.ndarray, xhat: np.ndarray) -> float:
    x = np.asarray(x, dtype=np.float64)
    xhat = np.asarray(xhat, dtype=np.float64)
    return float(((x - xhat) ** 2).sum() / (x ** 2).sum())
