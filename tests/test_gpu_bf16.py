"""The uncompressed bf16 reference kernel (dq_bf16_decode_attention) against
the oracle's fp64 attention over the same bf16 rows. Inputs are exact in bf16,
so only fp32 accumulation separates the two: the bar is 1e-4."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_dq_amd import synth, workloads
from dq_cases import paged_layout, row_rel_err

pytestmark = pytest.mark.gpu
TOL_BF16 = 1e-4


def _rows(seed, tensor, T, hkv, b):
    x = synth.gaussian_kv(300 + seed, tensor, max(T, 1), hkv, part=b)[:T]
    return synth.f32_to_bf16_bits(x)          # uint16 [T][hkv][128]


def _case(dq, lens, hkv, hq, P, seed, perm_seed=None, splits=0):
    B = len(lens)
    kb = [_rows(seed, synth.T_K, T, hkv, b) for b, T in enumerate(lens)]
    vb = [_rows(seed, synth.T_V, T, hkv, b) for b, T in enumerate(lens)]
    as_bytes = lambda r: r.view(np.uint8).reshape(r.shape[0], hkv, 256)
    zn = [np.zeros((T, hkv), np.uint16) for T in lens]
    kc, _, bt = paged_layout([as_bytes(r) for r in kb], zn, P, perm_seed=perm_seed)
    vc, _, _ = paged_layout([as_bytes(r) for r in vb], zn, P, perm_seed=perm_seed)
    used, _, _ = paged_layout([np.ones((T, hkv, 256), np.uint8) for T in lens], zn, P, perm_seed=perm_seed)
    kc[used == 0] = 0xFF                       # rows past each end hold NaN bit patterns
    vc[used == 0] = 0xFF
    q = synth.queries(300 + seed, B, hq, bf16=True)
    f = lambda r: synth.bf16_bits_to_f32(r).transpose(1, 0, 2).astype(np.float64)
    ref = np.zeros((B, hq, 128))
    for b, T in enumerate(lens):              # an empty sequence attends to nothing: zeros
        if T:
            ref[b] = oracle.attention(q[b:b + 1], [f(kb[b])], [f(vb[b])])[0]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bf = lambda a: dev(a).view(torch.bfloat16)
    kcd = bf(kc).view(kc.shape[0], hkv, P, 128)
    vcd = bf(vc).view(vc.shape[0], hkv, P, 128)
    max_ctx = max(1, max(lens))
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    # NaN bytes: a partial the kernel leaves unwritten reaches the merge as NaN
    ws = torch.full((dq.dq_workspace_size(B, hq, hkv, max_ctx, splits),), 0xFF, dtype=torch.uint8, device="cuda")
    dq.dq_bf16_decode_attention(bf(synth.f32_to_bf16_bits(q)), kcd, vcd, dev(bt),
                                dev(np.asarray(lens, dtype=np.int32)), hkv, P, max_ctx, out, ws,
                                num_splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy(), ref


@pytest.mark.parametrize("G", [1, 2, 4])
def test_bf16_ragged_paged(gpu_lib, G):
    lens = [1, 31, 32, 33, 300, 1000]
    out, ref = _case(gpu_lib, lens, 2, 2 * G, 16, seed=G, perm_seed=5)
    assert row_rel_err(out, ref).max() <= TOL_BF16


def test_bf16_splits_and_empty(gpu_lib):
    lens = [0, 700, 2049]
    for splits in (1, 3, 9):
        out, ref = _case(gpu_lib, lens, 1, 4, 64, seed=7, splits=splits)
        assert np.all(out[0] == 0)
        assert row_rel_err(out[1:], ref[1:]).max() <= TOL_BF16, splits


@pytest.mark.parametrize("splits", [0, 3, 7])
def test_bf16_every_job_class(gpu_lib, splits):
    """Lengths around every tile and split boundary (see the compressed path's
    test of the same name): each job class taken once, every partial written."""
    lens = [0, 1, 255, 257, 511, 1024, 1537, 2047, 3300]
    out, ref = _case(gpu_lib, lens, 2, 4, 16, seed=9, perm_seed=3, splits=splits)
    assert np.all(out[0] == 0)
    assert row_rel_err(out[1:], ref[1:]).max() <= TOL_BF16


def test_bf16_full_qwen3_layer_sampled(gpu_lib):
    """The Qwen3-8B decode layer (B=128, 8192 tokens) in bf16, in the launch
    configuration the benchmark times."""
    dq = gpu_lib
    w = workloads.WORKLOADS["decode_qwen3_8b"]
    kc, vc, bt, lens = workloads.build_bf16_cache(w)
    q = workloads.query_rows(w)
    B, hq, hkv = w.batch, w.num_q_heads, w.num_kv_heads
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_workspace_size(B, hq, hkv, w.context), dtype=torch.uint8, device="cuda")
    dq.dq_bf16_decode_attention(q, kc, vc, bt, lens, hkv, w.page_size, w.context, out, ws)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    qh = q.float().cpu().numpy()
    G = hq // hkv
    for b, g in [(0, 0), (77, 4), (127, 7)]:
        T = int(lens[b])
        k = workloads.kv_rows(w, 0, synth.T_K, b, T)[:, g].to(torch.bfloat16).double().cpu().numpy()
        v = workloads.kv_rows(w, 0, synth.T_V, b, T)[:, g].to(torch.bfloat16).double().cpu().numpy()
        ref = oracle.attention(qh[b:b + 1, g * G:(g + 1) * G], [k[None]], [v[None]])[0]
        assert row_rel_err(out[b, g * G:(g + 1) * G], ref).max() <= TOL_BF16, (b, g)
    del kc, vc
