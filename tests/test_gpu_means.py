"""Windowed INT8 key channel-mean removal on the device (sections 3.2 and 5):
the block cache write (dq_encode_kv_blocks) bit-exact against the oracle's
O12 + codec (containers, fp16 norms, INT8 means and their fp16 scales), and
decode attention with the means (dq_decode_attention_ext) within the 2e-3
bar against the oracle's fp64 attention over the reconstructions."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_dq_amd import synth
from dq_cases import TOL, row_rel_err

pytestmark = pytest.mark.gpu
BLK = 128


def _rows(seed, tensor, T, hkv, b, offset):
    x = synth.gaussian_kv(400 + seed, tensor, T, hkv, part=b).astype(np.float64)
    if offset is not None:
        x = x + offset[None]                       # a per-(head, channel) key mean
    return x.astype(np.float32)


def _layout(lens, P, perm_seed):
    """Slots of every token, pages handed out per sequence (then relabelled)."""
    npages = [-(-T // P) for T in lens]
    total = sum(npages)
    perm = np.arange(total) if perm_seed is None else np.random.default_rng(perm_seed).permutation(total)
    bt = np.zeros((len(lens), max(npages)), np.int32)
    slots, nxt = [], 0
    for b, T in enumerate(lens):
        for lp in range(npages[b]):
            bt[b, lp] = perm[nxt]; nxt += 1
        t = np.arange(T)
        slots.append((bt[b, t // P] * P + t % P).astype(np.int32))
    return bt, total, slots


def _encode_case(dq, lens, hkv, P, seed, perm_seed=None, kC=37, vC=37):
    rng = np.random.default_rng(seed)
    offset = rng.standard_normal((hkv, 128)) * 2.0
    tk, tv = oracle.make_table(8, kC), oracle.make_table(6, vC)
    tabs = dq.dq_tables_init(dq.make_params(8, kC), dq.make_params(6, vC))
    bt, total, slots = _layout(lens, P, perm_seed)
    R = dq.mean_rows_per_page(P)
    kx = [_rows(seed, synth.T_K, T, hkv, b, offset) for b, T in enumerate(lens)]
    vx = [_rows(seed, synth.T_V, T, hkv, b, None) for b, T in enumerate(lens)]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc = torch.zeros((total, hkv, P, kC), dtype=torch.uint8, device="cuda")
    vc = torch.zeros((total, hkv, P, vC), dtype=torch.uint8, device="cuda")
    kn = torch.zeros((total, hkv, P), dtype=torch.int16, device="cuda")
    vn = torch.zeros_like(kn)
    km = torch.zeros((total, hkv, R, 128), dtype=torch.int8, device="cuda")
    ks = torch.zeros((total, hkv, R), dtype=torch.int16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_encode_kv_blocks(tabs, dev(np.concatenate(kx)), dev(np.concatenate(vx)), dev(np.concatenate(slots)),
                           kc, vc, kn, vn, km, ks, P, err_word=err)
    torch.cuda.synchronize()
    return dict(tk=tk, tv=tv, tabs=tabs, bt=bt, slots=slots, kx=kx, vx=vx, kc=kc, vc=vc, kn=kn, vn=vn, km=km,
                ks=ks, err=int(err.item()), R=R)


def _expected(c, b, hkv, P):
    """Oracle containers, norms and means of sequence b, per token and head."""
    T = c["kx"][b].shape[0]
    out = {"kc": [], "kn": [], "vc": [], "vn": [], "q": [], "s16": [], "mu": []}
    for h in range(hkv):
        kb = c["kx"][b][:, h].astype(np.float64).reshape(T // BLK, BLK, 128)
        q, s16, mu_hat, _ = oracle.block_means(kb)
        mean_rows = np.repeat(mu_hat, BLK, axis=0)
        rk = oracle.encode_streams(c["kx"][b][:, h], c["tk"], mean_rot=mean_rows)
        rv = oracle.encode_streams(c["vx"][b][:, h], c["tv"])
        out["kc"].append(rk.containers); out["kn"].append(rk.rho16)
        out["vc"].append(rv.containers); out["vn"].append(rv.rho16)
        out["q"].append(q); out["s16"].append(s16); out["mu"].append(mean_rows)
        out.setdefault("ksym", []).append(rk.symbols); out.setdefault("vsym", []).append(rv.symbols)
    return out


@pytest.mark.parametrize("P,perm", [(16, 7), (256, None), (128, 3)])
def test_encode_blocks_bit_exact(gpu_lib, P, perm):
    dq = gpu_lib
    lens, hkv = [256, 128, 384], 2
    c = _encode_case(dq, lens, hkv, P, seed=1, perm_seed=perm)
    assert c["err"] == 0
    kc, vc = c["kc"].cpu().numpy(), c["vc"].cpu().numpy()
    kn, vn = c["kn"].cpu().numpy().view(np.uint16), c["vn"].cpu().numpy().view(np.uint16)
    km, ks = c["km"].cpu().numpy(), c["ks"].cpu().numpy().view(np.uint16)
    for b, T in enumerate(lens):
        e = _expected(c, b, hkv, P)
        slots = c["slots"][b]
        pg, off = slots // P, slots % P
        for h in range(hkv):
            assert np.array_equal(kc[pg, h, off], e["kc"][h]), (b, h)
            assert np.array_equal(vc[pg, h, off], e["vc"][h]), (b, h)
            assert np.array_equal(kn[pg, h, off], e["kn"][h].view(np.uint16)), (b, h)
            assert np.array_equal(vn[pg, h, off], e["vn"][h].view(np.uint16)), (b, h)
            first = slots[::BLK]
            rows_pg, rows_i = first // P, (first % P) // BLK
            assert np.array_equal(km[rows_pg, h, rows_i], e["q"][h]), (b, h)
            assert np.array_equal(ks[rows_pg, h, rows_i], e["s16"][h].view(np.uint16)), (b, h)


def test_attention_with_means(gpu_lib):
    dq = gpu_lib
    lens, hkv, hq, P = [256, 128, 384], 2, 8, 16
    c = _encode_case(dq, lens, hkv, P, seed=2, perm_seed=11)
    assert c["err"] == 0
    ctx = [200, 128, 301]                        # partial last blocks attend to their first tokens
    kh, vh = [], []
    for b, T in enumerate(lens):
        e = _expected(c, b, hkv, P)
        kh.append(np.stack([oracle.reconstruct(e["ksym"][h], e["kn"][h], c["tk"], mean_rot=e["mu"][h])
                            for h in range(hkv)])[:, :ctx[b]])
        vh.append(np.stack([oracle.reconstruct(e["vsym"][h], e["vn"][h], c["tv"]) for h in range(hkv)])[:, :ctx[b]])
    q = synth.queries(402, len(lens), hq, bf16=True)
    ref = oracle.attention(q, kh, vh)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    B = len(lens)
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_workspace_size(B, hq, hkv, max(ctx)), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_decode_attention_ext(c["tabs"], dev(q).to(torch.bfloat16), c["kc"], c["vc"], c["kn"], c["vn"], dev(c["bt"]),
                               dev(np.array(ctx, np.int32)), hkv, P, max(ctx), out, ws, k_mean=c["km"],
                               k_mean_scale=c["ks"], err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert row_rel_err(out.cpu().numpy(), ref).max() <= TOL
    # without the means the keys are off by their channel mean: far outside the bar
    dq.dq_decode_attention(c["tabs"], dev(q).to(torch.bfloat16), c["kc"], c["vc"], c["kn"], c["vn"], dev(c["bt"]),
                           dev(np.array(ctx, np.int32)), hkv, P, max(ctx), out, ws)
    torch.cuda.synchronize()
    assert row_rel_err(out.cpu().numpy(), ref).max() > 10 * TOL


def test_means_with_window(gpu_lib):
    """Compressed blocks with means plus a bf16 window of the newest tokens."""
    dq = gpu_lib
    lens, hkv, hq, P = [256, 128], 1, 4, 256
    c = _encode_case(dq, lens, hkv, P, seed=3)
    W = [40, 128]
    rng = np.random.default_rng(9)
    wk = synth.round_to_bf16(rng.standard_normal((2, hkv, 128, 128)).astype(np.float32))
    wv = synth.round_to_bf16(rng.standard_normal((2, hkv, 128, 128)).astype(np.float32))
    kh, vh = [], []
    for b, T in enumerate(lens):
        e = _expected(c, b, hkv, P)
        kr = np.stack([oracle.reconstruct(e["ksym"][h], e["kn"][h], c["tk"], mean_rot=e["mu"][h]) for h in range(hkv)])
        vr = np.stack([oracle.reconstruct(e["vsym"][h], e["vn"][h], c["tv"]) for h in range(hkv)])
        kh.append(np.concatenate([kr, wk[b, :, :W[b]].astype(np.float64)], axis=1))
        vh.append(np.concatenate([vr, wv[b, :, :W[b]].astype(np.float64)], axis=1))
    q = synth.queries(403, 2, hq, bf16=True)
    ref = oracle.attention(q, kh, vh)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
    out = torch.full((2, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_workspace_size(2, hq, hkv, 256), dtype=torch.uint8, device="cuda")
    dq.dq_decode_attention_ext(c["tabs"], dev(q).to(torch.bfloat16), c["kc"], c["vc"], c["kn"], c["vn"], dev(c["bt"]),
                               dev(np.array(lens, np.int32)), hkv, P, 256, out, ws, window_k=bf(wk), window_v=bf(wv),
                               window_lens=dev(np.array(W, np.int32)), k_mean=c["km"], k_mean_scale=c["ks"])
    torch.cuda.synchronize()
    assert row_rel_err(out.cpu().numpy(), ref).max() <= TOL


def test_misaligned_block_is_flagged(gpu_lib):
    """A block whose first slot is not at a block start is refused on the
    device: DQ_DEVERR_MEAN_SLOT, its key streams unwritten, values written."""
    dq = gpu_lib
    hkv, P = 1, 256
    tabs = dq.dq_tables_init(dq.make_params(8, 37), dq.make_params(6, 37))
    slots = (np.arange(128) + 64).astype(np.int32)          # starts mid-block
    x = synth.gaussian_kv(405, synth.T_K, 128, hkv)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    kc = torch.zeros((1, hkv, P, 37), dtype=torch.uint8, device="cuda"); vc = torch.zeros_like(kc)
    kn = torch.zeros((1, hkv, P), dtype=torch.int16, device="cuda"); vn = torch.zeros_like(kn)
    km = torch.zeros((1, hkv, 2, 128), dtype=torch.int8, device="cuda")
    ks = torch.zeros((1, hkv, 2), dtype=torch.int16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_encode_kv_blocks(tabs, dev(x), dev(x), dev(slots), kc, vc, kn, vn, km, ks, P, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) & dq.DQ_DEVERR_MEAN_SLOT
    assert not kc.any() and not kn.any() and not km.any()
    assert vc[0, 0, 64:192].any()
