"""Decode attention with an uncompressed bf16 window of recent tokens merged by
log-sum-exp with the compressed cache (the paper keeps the most recent tokens
in BF16, section 5.1), and unequal key/value container budgets (section 4.4
"Separate K/V configurations"). Expected values: the oracle's fp64 attention
over its reconstructions of the compressed tokens followed by the exact bf16
window rows."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_dq_amd import synth
from dq_cases import TOL, paged_layout, row_rel_err, sequence_case

pytestmark = pytest.mark.gpu


def _window_case(dq, kM, kC, kstep, vM, vC, vstep, comp_lens, win_lens, cap, hkv, hq, P, seed):
    # a step of 0 selects the library's default; the oracle's default is step=None
    tk, tv = oracle.make_table(kM, kC, kstep or None), oracle.make_table(vM, vC, vstep or None)
    tabs = dq.dq_tables_init(dq.make_params(kM, kC, kstep), dq.make_params(vM, vC, vstep))
    B = len(comp_lens)
    conts_k, conts_v, nk, nv, kh, vh = [], [], [], [], [], []
    wk = np.zeros((B, hkv, cap, 128), dtype=np.float32)
    wv = np.zeros_like(wk)
    for b, (T, W) in enumerate(zip(comp_lens, win_lens)):
        k = synth.gaussian_kv(200 + seed, synth.T_K, T + W, hkv, part=b)
        v = synth.gaussian_kv(200 + seed, synth.T_V, T + W, hkv, part=b)
        wk[b, :, :W] = synth.round_to_bf16(k[T:]).transpose(1, 0, 2)
        wv[b, :, :W] = synth.round_to_bf16(v[T:]).transpose(1, 0, 2)
        if T:
            a, bb, c, d, e, f = sequence_case(tk, tv, k[:T], v[:T])
        else:
            a = np.zeros((0, hkv, kC), np.uint8); bb = np.zeros((0, hkv, vC), np.uint8)
            c = np.zeros((0, hkv), np.uint16); d = np.zeros((0, hkv), np.uint16)
            e = np.zeros((hkv, 0, 128)); f = np.zeros((hkv, 0, 128))
        conts_k.append(a); conts_v.append(bb); nk.append(c); nv.append(d)
        kh.append(np.concatenate([e, wk[b, :, :W].astype(np.float64)], axis=1))
        vh.append(np.concatenate([f, wv[b, :, :W].astype(np.float64)], axis=1))
    kc, kn, bt = paged_layout(conts_k, nk, P, perm_seed=seed)
    vc, vn, _ = paged_layout(conts_v, nv, P, perm_seed=seed)
    q = synth.queries(200 + seed, B, hq, bf16=True)
    ref = np.zeros((B, hq, 128))
    for b in range(B):
        if comp_lens[b] + win_lens[b]:
            ref[b] = oracle.attention(q[b:b + 1], [kh[b]], [vh[b]])[0]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
    max_ctx = max(1, max(comp_lens))
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_workspace_size(B, hq, hkv, max_ctx), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_decode_attention_window(tabs, dev(q).to(torch.bfloat16), dev(kc), dev(vc), dev(kn.view(np.int16)),
                                  dev(vn.view(np.int16)), dev(bt), dev(np.array(comp_lens, np.int32)), bf(wk), bf(wv),
                                  dev(np.array(win_lens, np.int32)), hkv, P, max_ctx, out, ws, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    return out.cpu().numpy(), ref


def test_window_with_compressed_cache(gpu_lib):
    out, ref = _window_case(gpu_lib, 8, 37, 0.0, 6, 37, 0.0, [300, 1, 0, 1000, 64], [128, 128, 77, 5, 0],
                            128, 2, 8, 16, seed=1)
    assert row_rel_err(out, ref).max() <= TOL


def test_window_only_and_empty(gpu_lib):
    out, ref = _window_case(gpu_lib, 8, 37, 0.0, 6, 37, 0.0, [0, 0, 0], [1, 256, 0], 256, 1, 4, 16, seed=2)
    assert np.all(out[2] == 0)
    assert row_rel_err(out[:2], ref[:2]).max() <= TOL


def test_unequal_kv_budgets_with_window(gpu_lib):
    """Keys 41 bytes / values 27 bytes per stream (with the fp16 norms, 2.69 and 1.81
    bits per value: a key/value split of the same 2.25-bit average)."""
    out, ref = _window_case(gpu_lib, 8, 41, 0.0, 6, 27, 0.0, [2000, 517, 4096], [128, 0, 64], 128, 2, 8, 32,
                            seed=3)
    assert row_rel_err(out, ref).max() <= TOL
