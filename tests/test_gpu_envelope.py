"""Corners of the supported envelope on the device: 2 to 9 levels,
probability precision p = 9 and 10, containers from 8 to 128 bytes (padded and
unpadded LDS strides, and containers over 64 bytes, which take two 16-byte
staging units per lane). At each corner: the cache write is bit-exact to the
oracle, the symbol decode is exact, and attention over the encoded cache
meets the 2e-3 bar against the oracle's fp64 attention."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_dq_amd import synth
from dq_cases import TOL, row_rel_err
from test_gpu_attention import _case, _run
from test_gpu_encode import _check

pytestmark = pytest.mark.gpu

#            M   C    p   step
CORNERS = [(3, 8, 10, 3.0), (2, 24, 9, 1.0), (5, 16, 9, 1.6), (9, 45, 9, 0.9), (8, 72, 10, 0.7),
           (9, 100, 10, 0.6), (9, 128, 9, 0.5)]


def _tables(dq, M, C, p, step):
    t = oracle.make_table(M, C, step, 1.4, p)
    assert t.feasible
    tabs = dq.dq_tables_init(dq.make_params(M, C, step, prob_bits=p), dq.make_params(M, C, step, prob_bits=p))
    return t, tabs


@pytest.mark.parametrize("M,C,p,step", CORNERS)
def test_corner_encode_and_symbols(gpu_lib, M, C, p, step):
    dq = gpu_lib
    t, tabs = _tables(dq, M, C, p, step)
    k = synth.gaussian_kv(500 + C, synth.T_K, 96, 4, outliers=2)
    v = synth.gaussian_kv(500 + C, synth.T_V, 96, 4)
    _check(dq, tabs, t, t, k, v, torch.from_numpy(k).cuda(), torch.from_numpy(v).cuda(), C=(C, C))
    r = oracle.encode_streams(k.reshape(-1, 128).astype(np.float64), t)
    cont = torch.from_numpy(np.ascontiguousarray(r.containers)).cuda()
    sym = torch.zeros((cont.shape[0], 128), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_decode_symbols(tabs, dq.DQ_KEYS, cont, sym, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(sym.cpu().numpy(), r.symbols.astype(np.uint8))


@pytest.mark.parametrize("M,C,p,step", CORNERS)
def test_corner_attention(gpu_lib, M, C, p, step):
    dq = gpu_lib
    t, tabs = _tables(dq, M, C, p, step)
    lens = [1, 100, 300]
    q, kc, vc, kn, vn, bt, ref = _case(t, t, lens, 2, 8, 16, True, seed=600 + C, perm_seed=C)
    out, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, lens, 2, 16, max(lens))
    assert err == 0
    assert row_rel_err(out, ref).max() <= TOL
