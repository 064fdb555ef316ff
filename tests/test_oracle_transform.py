"""Pins for the oracle's rotation (O2) and normalisation (O3).

Rotation: D-Quant section 3.2 / 4.1 (Hadamard rotation). The oracle's fast
transform is checked against scipy's Sylvester Hadamard matrix, against the
algebraic identities H H^T = 128 I and ||H x|| = sqrt(128) ||x||, and the
norm against numpy's L2 norm of the unrotated row.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle.codec import tree_sum_squares
from decode_attention_dq_amd import synth

H = scipy.linalg.hadamard(128).astype(np.float64)


def test_hadamard_matrix_identity():
    # H H^T = 128 I exactly (integer entries), built column by column by the oracle
    Hm = oracle.fwht(np.eye(128))
    assert np.array_equal(Hm, H)
    assert np.array_equal(Hm @ Hm.T, 128.0 * np.eye(128))


def test_fwht_matches_matrix_exact_for_bf16_inputs():
    x = synth.round_to_bf16(np.random.default_rng(3).standard_normal((64, 128)).astype(np.float32))
    x = x.astype(np.float64)
    # sums of bf16 values of N(0,1) size fit in fp64 exactly: both paths are exact
    assert np.array_equal(oracle.fwht(x), x @ H)


def test_fwht_matches_matrix_fp32_inputs():
    x = np.random.default_rng(4).standard_normal((64, 128)).astype(np.float32).astype(np.float64)
    y = oracle.fwht(x)
    ref = x @ H
    assert np.max(np.abs(y - ref) / np.abs(ref).max(axis=1, keepdims=True)) < 1e-15


def test_fwht_involution_and_norm():
    x = np.random.default_rng(5).standard_normal((16, 128))
    y = oracle.fwht(x)
    assert np.allclose(oracle.fwht(y) / 128.0, x, rtol=0, atol=1e-13)
    assert np.allclose(np.linalg.norm(y, axis=1), np.sqrt(128) * np.linalg.norm(x, axis=1), rtol=1e-14)


def test_fwht_butterfly_order_small_case():
    # e_j maps to column j of H; a planted error in the pair order would permute columns
    for j in [0, 1, 2, 5, 64, 127]:
        e = np.zeros(128)
        e[j] = 1.0
        assert np.array_equal(oracle.fwht(e), H[:, j])


def test_tree_sum_is_the_fixed_tree():
    # y0^2 = y64^2 = 2^-50 meet first (level w = 64) and make 2^-49 = ulp(9); then
    # y32^2 = 9 joins at w = 32: S = 9 + 2^-49 exactly. Summing in index order
    # (or numpy's pairwise blocks) adds each 2^-50 to 9 separately: a tie that
    # rounds back to 9, so any other order gives a different fp64 value.
    y = np.zeros(128)
    y[0] = y[64] = 2.0 ** -25
    y[32] = 3.0
    assert tree_sum_squares(y[None])[0] == 9.0 + 2.0 ** -49
    assert float(np.sum(y * y)) == 9.0


def test_normalize_unit_rms_and_norm():
    x = np.random.default_rng(6).standard_normal((200, 128)) * np.exp(np.random.default_rng(7).normal(0, 3, (200, 1)))
    y = oracle.fwht(x)
    rho, rho16, z = oracle.normalize(y)
    assert np.allclose((z * z).sum(axis=1), 128.0, rtol=1e-12)
    nrm = np.linalg.norm(x, axis=1)
    assert np.allclose(rho, nrm, rtol=1e-14)
    # the stored norm is the L2 norm of the original row rounded once to fp16
    assert np.array_equal(rho16, nrm.astype(np.float16))


def test_normalize_zero_row():
    y = np.zeros((2, 128))
    rho, rho16, z = oracle.normalize(y)
    assert np.all(z == 0) and np.all(rho16 == 0)


@pytest.mark.parametrize("M,C", [(8, 37), (6, 37), (8, 32), (6, 32)])
def test_zero_row_encodes_to_central_symbols(M, C):
    t = oracle.make_table(M, C)
    r = oracle.encode_streams(np.zeros((1, 128)), t)
    central = (M - 1) // 2          # the central midpoint goes to the lower central level
    assert np.all(r.symbols == central)
    assert np.all(oracle.reconstruct(r.symbols, r.rho16, t) == 0)
