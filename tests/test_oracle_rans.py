"""Pins for the oracle's rANS coder (O7, O9).

D-Quant section 3.1 gives Enc/Dec. Pins: hand-worked examples
(tests/golden/rans_hand_examples.txt), the exhaustive inverse property of a
single step, brute force over every short symbol sequence, hypothesis on
full-length streams, and the at-most-one-byte renormalisation bound.
"""
import itertools
import os
from types import SimpleNamespace

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "rans_hand_examples.txt")


def toy_table(freqs, p):
    freq = np.array(freqs, dtype=np.int64)
    cum = np.concatenate([[0], np.cumsum(freq)]).astype(np.int64)
    sym = np.zeros(1 << p, dtype=np.int64)
    for m in range(len(freq)):
        sym[cum[m]:cum[m + 1]] = m
    return SimpleNamespace(freq=freq, cum=cum, sym=sym, prob_bits=p)


def load_golden():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        name, p, fr, sy, by = [s.strip() for s in line.split("|")]
        rows.append((name, int(p), [int(v) for v in fr.split()], [int(v) for v in sy.split()],
                     [int(v, 16) for v in by.split()]))
    return rows


@pytest.mark.parametrize("row", load_golden(), ids=lambda r: r[0])
def test_hand_worked_examples(row):
    name, p, freqs, symbols, expected = row
    t = toy_table(freqs, p)
    cont, ln = oracle.rans_encode(np.array([symbols]), t, capacity=len(expected))
    assert ln[0] == len(expected)
    assert cont[0].tolist() == expected
    sym, x, ptr, ok = oracle.rans_decode(cont, t, n=len(symbols))
    assert sym[0].tolist() == symbols and x[0] == oracle.STATE_LOW and ptr[0] == len(expected)


@pytest.mark.parametrize("M,C", [(8, 37), (6, 32)])
def test_step_inverse_exhaustive(M, C):
    t = oracle.make_table(M, C)
    p = t.prob_bits
    for m in range(M):
        f = int(t.freq[m])
        # every state the encoder can hold before Enc(., m)
        x = np.arange(f << (16 - p), f << (24 - p), dtype=np.int64)
        y = oracle.rans_enc_step(x, np.full_like(x, m), t)
        assert y.min() >= oracle.STATE_LOW and y.max() < 1 << 24
        ms, back = oracle.rans_dec_step(y, t)
        assert np.all(ms == m)
        assert np.array_equal(back, x)


@pytest.mark.parametrize("M,n", [(8, 5), (6, 6), (3, 9)])
def test_brute_force_roundtrip(M, n):
    t = oracle.make_table(M, 37, step=0.9)
    seqs = np.array(list(itertools.product(range(M), repeat=n)), dtype=np.int64)
    cont, ln = oracle.rans_encode(seqs, t)      # unbounded container
    sym, x, ptr, ok = oracle.rans_decode(cont, t, n=n)
    assert np.array_equal(sym, seqs)
    assert np.all(x == oracle.STATE_LOW) and np.array_equal(ptr, ln) and ok.all()


@settings(max_examples=60, deadline=None)
@given(st.lists(st.integers(0, 7), min_size=128, max_size=128))
def test_roundtrip_full_length_hypothesis(symbols):
    t = oracle.make_table(8, 37)
    m = np.array([symbols])
    cont, ln = oracle.rans_encode(m, t)
    sym, x, ptr, ok = oracle.rans_decode(cont, t)
    assert np.array_equal(sym, m) and x[0] == oracle.STATE_LOW and ptr[0] == ln[0] and ok[0]


def test_worst_case_stream_uses_one_byte_per_step():
    t = oracle.make_table(8, 37)
    # all outermost symbols: 8 bits each, the maximum
    m = np.zeros((1, 128), dtype=np.int64)
    cont, ln = oracle.rans_encode(m, t)
    assert ln[0] == 3 + 128
    sym, x, ptr, ok = oracle.rans_decode(cont, t)
    assert ok[0] and np.array_equal(sym, m)


def test_corrupt_container_is_detected():
    t = oracle.make_table(8, 37)
    x = np.random.default_rng(11).standard_normal((64, 128))
    r = oracle.encode_streams(x, t)
    bad = r.containers.copy()
    bad[:, 1] ^= 0x5A          # flip bits of the flushed state
    _, ok = oracle.decode_streams(bad, t)
    assert not ok.all()
