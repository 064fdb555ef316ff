"""O11 — fp64 GQA decode attention over reconstructed keys and values.

TEST INFRASTRUCTURE ONLY (see the package header).

The paper folds the decoded levels straight into the attention contraction
(D-Quant section 4.5 "Decoding") and evaluates grouped-query models (Qwen3-8B,
Llama-3.1-8B; GQA, Ainslie et al. 2023). The plain definition used here:
for sequence b and query head h, KV head g = floor(h / (Hq / Hkv)),

    s_t = scale * (q_h . k_hat_{b,g,t}),  p = softmax(s),  o_h = sum_t p_t v_hat_{b,g,t}

over the first T_b tokens, in fp64, in the original (unrotated) domain.
"""
from __future__ import annotations

import numpy as np

from .codec import fwht


def _softmax(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - s.max())
    return e / e.sum()


def attention(q: np.ndarray, khat, vhat, lens=None, scale: float | None = None) -> np.ndarray:
    """q [B][Hq][D]; khat/vhat: per sequence an array [Hkv][T_b][D] (a list,
    or one array [B][Hkv][T][D] with ``lens`` giving T_b). Returns fp64 [B][Hq][D]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        kb = np.asarray(khat[b], dtype=np.float64)
        vb = np.asarray(vhat[b], dtype=np.float64)
        Hkv = kb.shape[0]
        T = kb.shape[1] if lens is None else int(lens[b])
        group = Hq // Hkv
        for h in range(Hq):
            g = h // group
            s = scale * (kb[g, :T] @ q[b, h])
            out[b, h] = _softmax(s) @ vb[g, :T]
    return out


def attention_rotated(q: np.ndarray, yk, yv, lens=None, scale: float | None = None) -> np.ndarray:
    """The same attention evaluated in the rotated domain.

    yk / yv hold rotated reconstructions (rho16 * level, approximating H x).
    With q_rot = H q, q . x_hat = q_rot . y_hat / 128 and o = H o_rot / 128.
    Used only to check that the two domains agree.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    qr = fwht(q)
    out = np.zeros((B, Hq, D))
    for b in range(B):
        kb = np.asarray(yk[b], dtype=np.float64)
        vb = np.asarray(yv[b], dtype=np.float64)
        Hkv = kb.shape[0]
        T = kb.shape[1] if lens is None else int(lens[b])
        group = Hq // Hkv
        for h in range(Hq):
            g = h // group
            s = scale * (kb[g, :T] @ qr[b, h]) / D
            out[b, h] = _softmax(s) @ vb[g, :T]
    return fwht(out) / D
