"""Pins of O12, the windowed INT8 key channel-mean removal (section 3.2,
Table 1 "+ mean removal"; section 5, fixed-width ablation), against closed
forms, an exact special case that reduces to the plain codec, the rounding
bound of the INT8 encoding, and the effect the paper reports (removing a
channel mean restores the key reconstruction error)."""
import numpy as np
import pytest

import oracle
from oracle.means import block_means, dequantize


def _h(n=128):
    from scipy.linalg import hadamard
    return hadamard(n).astype(np.float64)


def test_constant_block_closed_form():
    """Every row equal to v: the rotated mean is H v exactly (integer data,
    exact sums). With H v = 127 e_5 the scale is exactly 1 and the INT8 code
    is H v itself."""
    Hm = _h()
    target = np.zeros(128)
    target[5] = 127.0
    v = Hm @ target / 128.0                      # H v = target (H H = 128 I)
    x = np.broadcast_to(v, (128, 128)).copy()
    q, s16, mu_hat, mu = block_means(x)
    assert np.array_equal(mu, target)
    assert float(s16) == 1.0
    assert np.array_equal(q.astype(np.float64), target)
    assert np.array_equal(mu_hat, target)


def test_opposite_pairs_give_zero_mean_and_plain_codec():
    """Rows in (r, -r) pairs sum to exactly zero token by token: q = 0, a zero
    scale, and the key streams encode exactly as without mean removal."""
    rng = np.random.default_rng(3)
    r = rng.standard_normal((64, 128))
    x = np.empty((128, 128))
    x[0::2], x[1::2] = r, -r
    q, s16, mu_hat, mu = block_means(x)
    assert not np.any(mu) and not np.any(q) and float(s16) == 0.0 and not np.any(mu_hat)
    t = oracle.make_table(8, 37)
    a = oracle.encode_streams(x, t)
    b = oracle.encode_streams(x, t, mean_rot=np.broadcast_to(mu_hat, x.shape))
    assert np.array_equal(a.containers, b.containers) and np.array_equal(a.rho16, b.rho16)


def test_int8_rounding_bound_and_scale():
    """|mu_hat - mu| <= s16 / 2 on every channel that is not clamped, the
    largest |q| is 127 (or 126..127 after the fp16 rounding of the scale), and
    the scale is the fp16 rounding of max |mu| / 127."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 128, 128)) + rng.standard_normal((6, 1, 128)) * 3.0
    q, s16, mu_hat, mu = block_means(x)
    sd = s16.astype(np.float64)
    assert np.array_equal(s16, (np.abs(mu).max(-1) / 127.0).astype(np.float16))
    unclamped = np.abs(mu / sd[:, None]) <= 127.0
    err = np.abs(mu_hat - mu)
    assert np.all(err[unclamped] <= sd[:, None].repeat(128, 1)[unclamped] / 2 * (1 + 1e-12))
    assert np.all(np.abs(q).max(-1) >= 126)
    assert np.array_equal(dequantize(q, s16), mu_hat)


def test_mean_is_taken_in_token_order():
    """The block mean is a token-order fp64 sum divided by 128: a sum whose
    value depends on the order (1, 2^53, -2^53, ...) comes out as that order
    gives it."""
    Hm = _h()
    y = np.zeros((128, 128))
    y[0, 0], y[1, 0], y[2, 0] = 1.0, 2.0 ** 53, -(2.0 ** 53)      # token order: (1 + 2^53) rounds to 2^53
    x = y @ Hm.T / 128.0                          # rows whose rotation is y (H H = 128 I)
    assert np.array_equal(oracle.fwht(x), y)
    _, _, _, mu = block_means(x)
    assert mu[0] == 0.0                           # a pairwise or exact sum would give 1/128


@pytest.mark.parametrize("M,C", [(8, 37), (8, 41)])
def test_mean_removal_restores_key_error(M, C):
    """Keys with a strong per-channel offset: without mean removal the
    reconstruction error grows several-fold; with it, it is back within 10% of
    the offset-free error (the paper's Table 1 effect). A dropped term or a
    wrong sign in the removal or in the reconstruction fails this."""
    rng = np.random.default_rng(5)
    base = rng.standard_normal((128, 128))
    offset = rng.standard_normal(128) * 2.0
    x = base + offset
    t = oracle.make_table(M, C)

    def err(rows, mean=None):
        r = oracle.encode_streams(rows, t, mean_rot=mean)
        xh = oracle.reconstruct(r.symbols, r.rho16, t, mean_rot=mean)
        return float(((rows - xh) ** 2).sum() / ((rows - rows.mean(0)) ** 2).sum())

    e_clean = err(base)
    e_raw = err(x)
    _, _, mu_hat, _ = block_means(x)
    e_mean = err(x, np.broadcast_to(mu_hat, x.shape))
    assert e_raw > 3 * e_clean
    assert e_mean < 1.1 * e_clean
