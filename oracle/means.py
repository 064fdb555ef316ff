"""O12: windowed INT8 channel-mean removal for keys.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The paper removes the channel-wise mean of the rotated keys, which a
token-level offset cannot capture (section 3.2, Table 1 "+ mean removal"),
using windowed INT8 channel means (section 5, fixed-width ablation). The
pages fix neither the window nor the INT8 encoding; the readings taken here:

* the window is a block of 128 consecutive tokens of one sequence and KV
  head (blocks start at token positions that are multiples of 128: a block
  is what leaves the 128-token BF16 window of recent tokens when it is
  compressed);
* the mean is taken in the rotated domain y = H x (the Sylvester rotation of
  the codec, O2): mu = (sum over t = 0..127 of y_t, added in token order in
  fp64) / 128;
* INT8 with one scale per block and head: s16 = fp16(max_c |mu_c| / 127)
  (one round to nearest even), q_c = rint(mu_c / s16) clamped to [-127, 127]
  (rint rounds half to even), mu_hat = q * s16; a zero scale gives q = 0;
* the key stream encodes the residual y_t - mu_hat (normalised by its own
  norm, O3), and the reconstruction adds mu_hat back before the inverse
  rotation; values are unchanged.
"""
from __future__ import annotations

import numpy as np

from .codec import fwht

BLOCK = 128


def block_means(x: np.ndarray):
    """x [..., 128 tokens, 128 channels]: one block of original-domain key rows
    per leading index. Returns (q int8 [..., 128], s16 float16 [...],
    mu_hat float64 [..., 128], mu float64 [..., 128])."""
    x = np.asarray(x, dtype=np.float64)
    if x.shape[-2] != BLOCK:
        raise ValueError("a block holds 128 tokens")
    y = fwht(x)
    acc = np.zeros(x.shape[:-2] + (x.shape[-1],))
    for t in range(BLOCK):            # token order, one fp64 addition per token
        acc = acc + y[..., t, :]
    mu = acc / float(BLOCK)           # exact: a power of two
    s = np.abs(mu).max(axis=-1) / 127.0
    with np.errstate(over="ignore"):
        s16 = s.astype(np.float16)
    sd = s16.astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(sd[..., None] > 0, np.rint(mu / np.where(sd > 0, sd, 1.0)[..., None]), 0.0)
    q = np.clip(r, -127, 127).astype(np.int8)
    mu_hat = q.astype(np.float64) * sd[..., None]
    return q, s16, mu_hat, mu


def dequantize(q: np.ndarray, s16: np.ndarray) -> np.ndarray:
    """mu_hat = q * s16 in fp64 (exact)."""
    return np.asarray(q, dtype=np.float64) * np.asarray(s16, dtype=np.float64)[..., None]
