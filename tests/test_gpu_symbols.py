"""The device rANS decoder (the routine the attention kernel runs) against
the oracle: symbols byte-identical, integrity flag exactly when the oracle's
decoder flags a stream."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_dq_amd import synth
from dq_cases import oracle_encode

pytestmark = pytest.mark.gpu


def _decode(dq, tabs, which, conts):
    c = torch.from_numpy(np.ascontiguousarray(conts)).cuda()
    out = torch.empty((conts.shape[0], 128), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_decode_symbols(tabs, which, c, out, err)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(err.item())


@pytest.mark.parametrize("kC,vC", [(37, 37), (32, 32)])
def test_symbols_of_encoded_streams(gpu_lib, kC, vC):
    dq = gpu_lib
    tk, tv = oracle.make_table(8, kC), oracle.make_table(6, vC)
    tabs = dq.dq_tables_init(dq.make_params(8, kC), dq.make_params(6, vC))
    k, v, _ = synth.tiny_check_inputs(0, tokens=1000)      # 1000 streams: 15 full tiles and a ragged one
    for which, rows, t in ((dq.DQ_KEYS, k, tk), (dq.DQ_VALUES, v, tv)):
        r = oracle_encode(rows, t)
        got, err = _decode(dq, tabs, which, r.containers)
        assert err == 0
        assert np.array_equal(got, r.symbols)


def test_symbols_of_random_sequences(gpu_lib):
    """Arbitrary symbol sequences (model-distributed and uniform), encoded by the
    oracle's rANS coder into 64-byte containers."""
    dq = gpu_lib
    M, C = 8, 64
    t = oracle.make_table(M, C, 0.92)
    tabs = dq.dq_tables_init(dq.make_params(M, C, 0.92), dq.make_params(6, 37))
    rng = np.random.default_rng(3)
    probs = t.freq / t.freq.sum()
    a = rng.choice(M, size=(3000, 128), p=probs)
    b = rng.integers(0, M, size=(3000, 128))
    b[:, ::2] = rng.choice(M, size=(3000, 64), p=probs)
    syms = np.concatenate([a, b])
    cont, ln = oracle.rans_encode(syms, t, C)
    keep = ln <= C
    assert keep.sum() > 3000
    got, err = _decode(dq, tabs, dq.DQ_KEYS, cont[keep])
    assert err == 0
    assert np.array_equal(got, syms[keep])


def _bytes_per_block(cont, t, n=128):
    """Bytes the oracle's decoder takes in each 4-step block of each stream."""
    S = cont.shape[0]
    x = cont[:, 0].astype(np.int64) | (cont[:, 1].astype(np.int64) << 8) | (cont[:, 2].astype(np.int64) << 16)
    taken = np.zeros((S, n // 4), dtype=np.int64)
    pos = np.full(S, 3, dtype=np.int64)
    rows = np.arange(S)
    for i in range(n):
        _, x = oracle.rans_dec_step(x, t)
        low = x < (1 << 16)
        x = np.where(low, (x << 8) | cont[rows, np.minimum(pos, cont.shape[1] - 1)], x)
        pos += low
        taken[:, i // 4] += low
    return taken


def test_symbols_of_byte_bursts(gpu_lib):
    """Runs of the rarest levels (f = 2^(p-8): every step takes a byte, 4 bytes
    between two window refills) between runs of the most probable ones (windows
    that stay in place over several refills), so the carried window refill moves
    its aligned start by a whole dword and by none, many times per stream. The
    decoder's odd and even waves run its two forms (with and without the
    aligned start held)."""
    dq = gpu_lib
    M, C = 8, 64
    t = oracle.make_table(M, C, 0.92)
    assert t.freq.min() == 1 << (t.prob_bits - 8)
    tabs = dq.dq_tables_init(dq.make_params(M, C, 0.92), dq.make_params(6, 37))
    rng = np.random.default_rng(29)
    rare = np.flatnonzero(t.freq == t.freq.min())
    common = np.flatnonzero(t.freq == t.freq.max())
    syms = np.empty((4000, 128), dtype=np.int64)
    for s in range(syms.shape[0]):
        row, use_rare = [], bool(rng.integers(0, 2))
        while len(row) < 128:
            k = int(rng.integers(4, 13)) if use_rare else int(rng.integers(6, 31))
            row += list(rng.choice(rare if use_rare else common, size=k))
            use_rare = not use_rare
        syms[s] = row[:128]
    cont, ln = oracle.rans_encode(syms, t, C)
    keep = ln <= C
    assert keep.sum() >= 1000
    cont, syms = cont[keep], syms[keep]
    taken = _bytes_per_block(cont, t)
    assert (taken == 4).sum() > 1000 and (taken == 0).sum() > 1000
    got, err = _decode(dq, tabs, dq.DQ_KEYS, cont)
    assert err == 0
    assert np.array_equal(got, syms)


def test_integrity_flag(gpu_lib):
    dq = gpu_lib
    t = oracle.make_table(8, 37)
    tabs = dq.dq_tables_init(dq.make_params(8, 37), dq.make_params(6, 37))
    k, _, _ = synth.tiny_check_inputs(1, tokens=40)
    r = oracle_encode(k, t)
    rng = np.random.default_rng(11)
    flagged = 0
    for i in range(40):
        c = r.containers[i:i + 1].copy()
        pos = rng.integers(0, 12)
        c[0, pos] ^= np.uint8(1 << rng.integers(0, 8))
        _, ok = oracle.decode_streams(c, t)
        _, err = _decode(dq, tabs, dq.DQ_KEYS, c)
        assert bool(err & dq.DQ_DEVERR_DECODE) == (not ok[0])
        flagged += not ok[0]
    assert flagged > 0
