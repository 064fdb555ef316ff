"""dq_decode_attention_noalloc (the variant for callers that cannot allocate)
against dq_decode_attention on the same inputs, through the C ABI: identical
outputs on two calls in a row, the second with a smaller input, both within
the oracle's tolerance; sizes beyond the fixed scratch are refused before any
launch."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_dq_amd import synth
from dq_cases import TOL, paged_layout, row_rel_err, sequence_case

pytestmark = pytest.mark.gpu


def _case(tk, tv, lens, hkv, hq, P, seed):
    ck, cv, nk, nv, kh, vh = [], [], [], [], [], []
    for b, T in enumerate(lens):
        k = synth.gaussian_kv(300 + seed, synth.T_K, T, hkv, part=b)
        v = synth.gaussian_kv(300 + seed, synth.T_V, T, hkv, part=b)
        a, bb, c, d, e, f = sequence_case(tk, tv, k, v)
        ck.append(a); cv.append(bb); nk.append(c); nv.append(d); kh.append(e); vh.append(f)
    kc, kn, bt = paged_layout(ck, nk, P, seed)
    vc, vn, _ = paged_layout(cv, nv, P, seed)
    q = synth.queries(300 + seed, len(lens), hq, bf16=True)
    ref = np.stack([oracle.attention(q[b:b + 1], [kh[b]], [vh[b]])[0] for b in range(len(lens))])
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return dict(q=dev(q).to(torch.bfloat16), kc=dev(kc), vc=dev(vc), kn=dev(kn.view(np.int16)),
                vn=dev(vn.view(np.int16)), bt=dev(bt), lens=dev(np.asarray(lens, np.int32))), ref


def _both(dq, tabs, d, hkv, P, max_ctx):
    B, hq = d["q"].shape[:2]
    args = (tabs, d["q"], d["kc"], d["vc"], d["kn"], d["vn"], d["bt"], d["lens"], hkv, P, max_ctx)
    ws = torch.full((dq.dq_workspace_size(B, hq, hkv, max_ctx),), 0xFF, dtype=torch.uint8, device="cuda")
    a = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    b = torch.full_like(a, float("nan"))
    ea = torch.zeros(1, dtype=torch.int32, device="cuda")
    eb = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_decode_attention(*args, a, ws, err_word=ea)
    dq.dq_decode_attention_noalloc(*args, b, err_word=eb)
    torch.cuda.synchronize()
    assert int(ea.item()) == 0 and int(eb.item()) == 0
    return a.cpu().numpy(), b.cpu().numpy()


def test_noalloc_matches_workspace_call(gpu_lib):
    dq = gpu_lib
    tk, tv = oracle.make_table(8, 37), oracle.make_table(6, 37)
    tabs = dq.dq_tables_init(dq.make_params(8, 37), dq.make_params(6, 37))
    # a larger call, then a smaller one: the second must not see the first's partials
    for lens, hkv, hq, P, seed in (([2100, 700, 1, 1500], 2, 8, 16, 1), ([300, 40], 1, 4, 32, 2)):
        d, ref = _case(tk, tv, lens, hkv, hq, P, seed)
        a, b = _both(dq, tabs, d, hkv, P, max(lens))
        assert np.array_equal(a, b)
        assert row_rel_err(b, ref).max() <= TOL


def test_noalloc_refuses_sizes_beyond_its_scratch(gpu_lib):
    dq = gpu_lib
    tabs = dq.dq_tables_init(dq.make_params(8, 37), dq.make_params(6, 37))
    B, hq, hkv, ctx = 1024, 32, 8, 8192
    assert dq.dq_workspace_size(B, hq, hkv, ctx) > dq.DQ_NOALLOC_SCRATCH
    z = lambda *s, dt=torch.uint8: torch.zeros(s, dtype=dt, device="cuda")
    q = z(B, hq, 128, dt=torch.bfloat16)
    out = z(B, hq, 128, dt=torch.float32)
    with pytest.raises(dq.DQError) as ei:
        dq.dq_decode_attention_noalloc(tabs, q, z(16), z(16), z(8, dt=torch.int16), z(8, dt=torch.int16),
                                       z(B, ctx // 256, dt=torch.int32), z(B, dt=torch.int32), hkv, 256, ctx, out)
    assert ei.value.code == dq.DQ_ERR_WORKSPACE
