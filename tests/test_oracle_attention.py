"""Pins for the oracle's fp64 decode attention (O11) and reconstruction (O10).

Closed forms: one token returns its value row; equal logits average the
values; the rotated-domain evaluation agrees with the original domain;
softmax matches scipy; grouped-query heads read their own KV head.
"""
import numpy as np
import scipy.special

import oracle
from oracle.attention import _softmax


def test_single_token_returns_value():
    rng = np.random.default_rng(40)
    q = rng.standard_normal((1, 2, 128))
    k = rng.standard_normal((1, 1, 1, 128))
    v = rng.standard_normal((1, 1, 1, 128))
    o = oracle.attention(q, k, v)
    assert np.array_equal(o[0, 0], v[0, 0, 0]) and np.array_equal(o[0, 1], v[0, 0, 0])


def test_equal_keys_and_zero_query_average_values():
    rng = np.random.default_rng(41)
    v = rng.standard_normal((1, 1, 50, 128))
    k = np.broadcast_to(rng.standard_normal(128), (1, 1, 50, 128))
    o = oracle.attention(rng.standard_normal((1, 1, 128)), k, v)
    assert np.allclose(o[0, 0], v[0, 0].mean(axis=0), atol=1e-14)
    k2 = rng.standard_normal((1, 1, 50, 128))
    o2 = oracle.attention(np.zeros((1, 1, 128)), k2, v)
    assert np.allclose(o2[0, 0], v[0, 0].mean(axis=0), atol=1e-14)


def test_softmax_matches_scipy():
    s = np.random.default_rng(42).standard_normal(1000) * 20
    assert np.allclose(_softmax(s), scipy.special.softmax(s), rtol=1e-13, atol=0)


def test_gqa_mapping():
    rng = np.random.default_rng(43)
    B, Hq, Hkv, T = 2, 8, 2, 30
    q = rng.standard_normal((B, Hq, 128))
    k = rng.standard_normal((B, Hkv, T, 128))
    v = rng.standard_normal((B, Hkv, T, 128))
    o = oracle.attention(q, k, v)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            single = oracle.attention(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1])
            assert np.array_equal(o[b, h], single[0, 0])


def test_ragged_lengths_ignore_tail():
    rng = np.random.default_rng(44)
    q = rng.standard_normal((2, 1, 128))
    k = rng.standard_normal((2, 1, 40, 128))
    v = rng.standard_normal((2, 1, 40, 128))
    lens = [17, 40]
    o = oracle.attention(q, k, v, lens=lens)
    k2 = k.copy(); k2[0, :, 17:] = 1e9; v2 = v.copy(); v2[0, :, 17:] = np.nan
    assert np.array_equal(oracle.attention(q, k2, v2, lens=lens), o)


def test_rotated_domain_agrees_and_reconstruction_is_rotation_inverse():
    rng = np.random.default_rng(45)
    tk = oracle.make_table(8, 37)
    tv = oracle.make_table(6, 37)
    T = 64
    xk = rng.standard_normal((T, 128))
    xv = rng.standard_normal((T, 128))
    rk = oracle.encode_streams(xk, tk)
    rv = oracle.encode_streams(xv, tv)
    kh = oracle.reconstruct(rk.symbols, rk.rho16, tk)
    vh = oracle.reconstruct(rv.symbols, rv.rho16, tv)
    # rotated reconstructions, and the inverse rotation check
    yk = rk.rho16.astype(np.float64)[:, None] * tk.recon[rk.symbols]
    yv = rv.rho16.astype(np.float64)[:, None] * tv.recon[rv.symbols]
    assert np.allclose(oracle.fwht(kh), yk, atol=1e-12)
    q = rng.standard_normal((1, 4, 128))
    o1 = oracle.attention(q, kh[None, None], vh[None, None])
    o2 = oracle.attention_rotated(q, yk[None, None], yv[None, None])
    assert np.allclose(o1, o2, rtol=0, atol=1e-12)
    # reconstruction error is in the range the 2.26-bit budget allows
    assert oracle.measures.nmse(xk, kh) < 0.1 and oracle.measures.nmse(xv, vh) < 0.1


def test_two_token_closed_form_with_scale():
    # q . k1 = sqrt(128) ln 3 and q . k2 = 0 -> logits (ln 3, 0) -> weights (3/4, 1/4)
    q = np.zeros((1, 1, 128)); q[0, 0, 0] = 1.0
    k = np.zeros((1, 1, 2, 128)); k[0, 0, 0, 0] = np.sqrt(128.0) * np.log(3.0)
    v = np.random.default_rng(46).standard_normal((1, 1, 2, 128))
    o = oracle.attention(q, k, v)
    assert np.allclose(o[0, 0], 0.75 * v[0, 0, 0] + 0.25 * v[0, 0, 1], rtol=0, atol=1e-15)
    # an explicit scale of 1 / (sqrt(128) ln 3) turns the same logits into (1, 0)
    o2 = oracle.attention(q, k, v, scale=1.0 / (np.sqrt(128.0) * np.log(3.0)))
    w = np.exp(1.0) / (np.exp(1.0) + 1.0)
    assert np.allclose(o2[0, 0], w * v[0, 0, 0] + (1 - w) * v[0, 0, 1], rtol=0, atol=1e-15)
