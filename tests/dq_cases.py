"""Helpers shared by the parity tests (not collected by pytest).

Expected values always come from the CPU oracle (``oracle/``) applied to
the same seeded inputs the device sees; this module only lays the oracle's
containers out in the paged cache format and compares results.
"""
from __future__ import annotations

import numpy as np

import oracle

TOL = 2e-3          # max relative error per (sequence, query head) row


def tables(kM=8, kC=37, vM=6, vC=37, kstep=None, vstep=None, p=10):
    return (oracle.make_table(kM, kC, kstep, 1.4, p), oracle.make_table(vM, vC, vstep, 1.4, p))


def oracle_encode(rows: np.ndarray, table):
    """rows [..., 128] (values exactly representable in fp64) -> EncodeResult
    over the flattened streams, in row-major order."""
    return oracle.encode_streams(np.asarray(rows, dtype=np.float64).reshape(-1, 128), table)


def rho16_bits(r) -> np.ndarray:
    return np.asarray(r.rho16, dtype=np.float16).view(np.uint16)


def paged_layout(conts, norms, page_size, perm_seed=None):
    """Lay per-sequence containers out as the paged cache.

    conts: list over sequences of uint8 [T_b][Hkv][C]; norms: list of uint16
    [T_b][Hkv]. Returns (cache [pages][Hkv][P][C] uint8, norm [pages][Hkv][P]
    uint16, block_table [B][max_pages] int32). Pages are handed out in order,
    then relabelled by a seeded permutation when ``perm_seed`` is given.
    """
    P = page_size
    B = len(conts)
    hkv, C = conts[0].shape[1], conts[0].shape[2]
    npages = [max(1, -(-c.shape[0] // P)) for c in conts]
    total = sum(npages)
    perm = np.arange(total) if perm_seed is None else np.random.default_rng(perm_seed).permutation(total)
    maxp = max(npages)
    bt = np.zeros((B, maxp), dtype=np.int32)
    cache = np.zeros((total, hkv, P, C), dtype=np.uint8)
    nrm = np.zeros((total, hkv, P), dtype=np.uint16)
    nxt = 0
    for b in range(B):
        T = conts[b].shape[0]
        for lp in range(npages[b]):
            phys = int(perm[nxt]); nxt += 1
            bt[b, lp] = phys
            lo, hi = lp * P, min(T, (lp + 1) * P)
            if hi > lo:
                cache[phys, :, :hi - lo, :] = conts[b][lo:hi].transpose(1, 0, 2)
                nrm[phys, :, :hi - lo] = norms[b][lo:hi].T
    return cache, nrm, bt


def row_rel_err(out: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per (b, h) row: max |out - ref| / max |ref|."""
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(out - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return num / np.where(den > 0, den, 1.0)


def sequence_case(tk, tv, k_rows, v_rows):
    """Oracle side of one sequence: rows [T][Hkv][128] -> (containers, norms,
    reconstructed keys/values [Hkv][T][128]) for K and V."""
    T, hkv = k_rows.shape[:2]
    rk = oracle_encode(k_rows, tk)
    rv = oracle_encode(v_rows, tv)
    kc = rk.containers.reshape(T, hkv, -1)
    vc = rv.containers.reshape(T, hkv, -1)
    kn = rho16_bits(rk).reshape(T, hkv)
    vn = rho16_bits(rv).reshape(T, hkv)
    kh = oracle.reconstruct(rk.symbols, rk.rho16, tk).reshape(T, hkv, 128).transpose(1, 0, 2)
    vh = oracle.reconstruct(rv.symbols, rv.rho16, tv).reshape(T, hkv, 128).transpose(1, 0, 2)
    return kc, vc, kn, vn, kh, vh
