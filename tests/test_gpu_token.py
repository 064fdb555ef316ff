"""The per-token format on the device (one 1024-value stream per token over
the 8 KV heads, min-max affine grid, least-squares refit; sections 4.2, 4.5,
5.1): the cache write bit-exact against the oracle (containers, fp16 (o, s),
drift statistics), the symbol decode exact, and decode attention over oracle
containers within the 2e-3 bar against the oracle's fp64 attention over its
reconstructions. Expected values come from the oracle only."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_dq_amd import synth
from dq_cases import TOL, row_rel_err

pytestmark = pytest.mark.gpu
K_CFG, V_CFG = (8, 331), (6, 231)


@pytest.fixture(scope="module")
def setup(gpu_lib):
    dq = gpu_lib
    tk, tv = oracle.make_token_table(*K_CFG), oracle.make_token_table(*V_CFG)
    tabs = dq.dq_token_tables_init(dq.make_params(*K_CFG), dq.make_params(*V_CFG))
    return dq, tk, tv, tabs


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _tokens(seed, tensor, n, part=0, bf16=False):
    """[n][8][128] float32 rows (K with 4 outlier channels per head)."""
    return synth.gaussian_kv(700 + seed, tensor, n, 8, part=part, outliers=4 if tensor == synth.T_K else 0,
                             bf16=bf16)


def _to_pages(conts, P):
    """Per-slot containers [pages * P][C] -> the cache layout [pages][C4][P][4]
    (dword j of slot s at [page][j][s], zero padding to whole dwords)."""
    n, C = conts.shape
    C4 = -(-C // 4)
    pad = np.zeros((n, 4 * C4), np.uint8)
    pad[:, :C] = conts
    return np.ascontiguousarray(pad.reshape(n // P, P, C4, 4).transpose(0, 2, 1, 3))


def _from_pages(cache, C):
    """The inverse of _to_pages: [pages][C4][P][4] -> [pages * P][4 C4]."""
    pages, C4, P, _ = cache.shape
    return cache.transpose(0, 2, 1, 3).reshape(pages * P, 4 * C4)


def _layout(lens, P, perm_seed):
    """Block table and the slot of every token, pages handed out per sequence."""
    npages = [max(1, -(-T // P)) for T in lens]
    total = sum(npages)
    perm = np.random.default_rng(perm_seed).permutation(total)
    bt = np.zeros((len(lens), max(npages)), np.int32)
    slots, nxt = [], 0
    for b, T in enumerate(lens):
        for lp in range(npages[b]):
            bt[b, lp] = perm[nxt]
            nxt += 1
        t = np.arange(T)
        slots.append((bt[b, t // P] * P + t % P).astype(np.int32))
    return bt, total, slots


@pytest.mark.parametrize("bf16", [False, True])
def test_token_encode_bit_exact(setup, bf16):
    """Containers, (o16, s16) and drift statistics equal the oracle's; a
    constant token and a zero token included; a slot of -1 writes nothing."""
    dq, tk, tv, tabs = setup
    n, P = 300, 16
    k = _tokens(1, synth.T_K, n, bf16=bf16)
    v = _tokens(1, synth.T_V, n, bf16=bf16)
    k[7] = 0.0
    v[7] = 0.0
    k[8] = 0.0
    k[8, :, 0] = 3.0                      # rotates to a constant 3 in every channel
    slots = np.random.default_rng(2).permutation(n + 20)[:n].astype(np.int32)
    slots[11] = -1
    pages = -(-(n + 20) // P)
    kc = torch.zeros(dq.token_cache_shape(pages, P, K_CFG[1]), dtype=torch.uint8, device="cuda")
    vc = torch.zeros(dq.token_cache_shape(pages, P, V_CFG[1]), dtype=torch.uint8, device="cuda")
    km = torch.zeros((pages, P, 2), dtype=torch.int16, device="cuda")
    vm = torch.zeros_like(km)
    ds = torch.zeros((n, 2), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    kd, vd = _dev(k), _dev(v)
    if bf16:
        kd, vd = kd.to(torch.bfloat16), vd.to(torch.bfloat16)   # exact: the rows hold bf16 values
    dq.dq_encode_tokens(tabs, kd, vd, _dev(slots), kc, vc, km, vm, P, drift_stats=ds, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    rk = oracle.encode_tokens(k.astype(np.float64), tk)
    rv = oracle.encode_tokens(v.astype(np.float64), tv)
    kc, vc = _from_pages(kc.cpu().numpy(), K_CFG[1]), _from_pages(vc.cpu().numpy(), V_CFG[1])
    assert not kc[:, K_CFG[1]:].any() and not vc[:, V_CFG[1]:].any()       # padding bytes are zero
    kc, vc = kc[:, :K_CFG[1]], vc[:, :V_CFG[1]]
    km, vm = km.cpu().numpy().view(np.uint16).reshape(-1, 2), vm.cpu().numpy().view(np.uint16).reshape(-1, 2)
    ds = ds.cpu().numpy().view(np.uint32)
    live = slots >= 0
    s = slots[live]
    assert np.array_equal(kc[s], rk.containers[live]) and np.array_equal(vc[s], rv.containers[live])
    assert np.array_equal(km[s, 0], rk.o16[live].view(np.uint16))
    assert np.array_equal(km[s, 1], rk.s16[live].view(np.uint16))
    assert np.array_equal(vm[s, 0], rv.o16[live].view(np.uint16))
    assert np.array_equal(vm[s, 1], rv.s16[live].view(np.uint16))
    assert np.array_equal(ds[live, 0] & 0xFFFF, rk.changed[live]) and np.array_equal(ds[live, 0] >> 16, rk.rounds[live])
    assert np.array_equal(ds[live, 1] & 0xFFFF, rv.changed[live]) and np.array_equal(ds[live, 1] >> 16, rv.rounds[live])
    unused = np.setdiff1d(np.arange(pages * P), s)
    assert not kc[unused].any() and not km[unused].any()


def test_token_encode_later_rounds(gpu_lib):
    """Key streams whose first drift round cannot bring the rate under a tight
    budget (several rounds, the per-stream procedure) next to value streams that
    fit in the first round, in the same waves: all bit-exact."""
    dq = gpu_lib
    kcfg = (8, 200)
    tk, tv = oracle.make_token_table(*kcfg), oracle.make_token_table(*V_CFG)
    tabs = dq.dq_token_tables_init(dq.make_params(*kcfg), dq.make_params(*V_CFG))
    n, P = 96, 16
    k = _tokens(5, synth.T_K, n)
    v = _tokens(5, synth.T_V, n)
    rk = oracle.encode_tokens(k.astype(np.float64), tk)
    rv = oracle.encode_tokens(v.astype(np.float64), tv)
    assert (rk.rounds > 1).sum() > n // 2 and (rv.rounds <= 1).all(), "case no longer exercises both paths"
    slots = np.random.default_rng(4).permutation(n).astype(np.int32)
    pages = n // P
    kc = torch.zeros(dq.token_cache_shape(pages, P, kcfg[1]), dtype=torch.uint8, device="cuda")
    vc = torch.zeros(dq.token_cache_shape(pages, P, V_CFG[1]), dtype=torch.uint8, device="cuda")
    km = torch.zeros((pages, P, 2), dtype=torch.int16, device="cuda")
    vm = torch.zeros_like(km)
    ds = torch.zeros((n, 2), dtype=torch.int32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_encode_tokens(tabs, _dev(k), _dev(v), _dev(slots), kc, vc, km, vm, P, drift_stats=ds, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    kc = _from_pages(kc.cpu().numpy(), kcfg[1])[:, :kcfg[1]]
    vc = _from_pages(vc.cpu().numpy(), V_CFG[1])[:, :V_CFG[1]]
    km, vm = km.cpu().numpy().view(np.uint16).reshape(-1, 2), vm.cpu().numpy().view(np.uint16).reshape(-1, 2)
    ds = ds.cpu().numpy().view(np.uint32)
    assert np.array_equal(kc[slots], rk.containers) and np.array_equal(vc[slots], rv.containers)
    assert np.array_equal(km[slots, 0], rk.o16.view(np.uint16)) and np.array_equal(km[slots, 1], rk.s16.view(np.uint16))
    assert np.array_equal(vm[slots, 0], rv.o16.view(np.uint16)) and np.array_equal(vm[slots, 1], rv.s16.view(np.uint16))
    assert np.array_equal(ds[:, 0] & 0xFFFF, rk.changed) and np.array_equal(ds[:, 0] >> 16, rk.rounds)
    assert np.array_equal(ds[:, 1] & 0xFFFF, rv.changed) and np.array_equal(ds[:, 1] >> 16, rv.rounds)


def test_token_encode_large_containers(gpu_lib):
    """The largest containers (1024-byte keys, 900-byte values): fewer streams
    share a wave so that their rows and emission buffers fit the LDS; bit-exact."""
    dq = gpu_lib
    kcfg, vcfg = (8, 1024), (6, 900)
    tk, tv = oracle.make_token_table(*kcfg), oracle.make_token_table(*vcfg)
    tabs = dq.dq_token_tables_init(dq.make_params(*kcfg), dq.make_params(*vcfg))
    n, P = 45, 16
    k = _tokens(6, synth.T_K, n)
    v = _tokens(6, synth.T_V, n)
    slots = np.random.default_rng(6).permutation(48)[:n].astype(np.int32)
    pages = 3
    kc = torch.zeros(dq.token_cache_shape(pages, P, kcfg[1]), dtype=torch.uint8, device="cuda")
    vc = torch.zeros(dq.token_cache_shape(pages, P, vcfg[1]), dtype=torch.uint8, device="cuda")
    km = torch.zeros((pages, P, 2), dtype=torch.int16, device="cuda")
    vm = torch.zeros_like(km)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_encode_tokens(tabs, _dev(k), _dev(v), _dev(slots), kc, vc, km, vm, P, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    rk = oracle.encode_tokens(k.astype(np.float64), tk)
    rv = oracle.encode_tokens(v.astype(np.float64), tv)
    kc = _from_pages(kc.cpu().numpy(), kcfg[1])[:, :kcfg[1]]
    vc = _from_pages(vc.cpu().numpy(), vcfg[1])[:, :vcfg[1]]
    km, vm = km.cpu().numpy().view(np.uint16).reshape(-1, 2), vm.cpu().numpy().view(np.uint16).reshape(-1, 2)
    assert np.array_equal(kc[slots], rk.containers) and np.array_equal(vc[slots], rv.containers)
    assert np.array_equal(km[slots, 0], rk.o16.view(np.uint16)) and np.array_equal(km[slots, 1], rk.s16.view(np.uint16))
    assert np.array_equal(vm[slots, 0], rv.o16.view(np.uint16)) and np.array_equal(vm[slots, 1], rv.s16.view(np.uint16))


def test_token_decode_symbols(setup):
    """Oracle containers decode to the oracle's symbols; a corrupted container
    sets the decode flag."""
    dq, tk, tv, tabs = setup
    for tab, cfg, t, tensor in ((tk, K_CFG, dq.DQ_KEYS, synth.T_K), (tv, V_CFG, dq.DQ_VALUES, synth.T_V)):
        r = oracle.encode_tokens(_tokens(3, tensor, 64).astype(np.float64), tab)
        cont = _dev(r.containers)
        sym = torch.zeros((64, 1024), dtype=torch.uint8, device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        dq.dq_token_decode_symbols(tabs, t, cont, sym, err_word=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert np.array_equal(sym.cpu().numpy(), r.symbols.astype(np.uint8))
        bad = r.containers.copy()
        bad[5, 0] ^= 0x5A                   # a different initial state
        dq.dq_token_decode_symbols(tabs, t, _dev(bad), sym, err_word=err)
        torch.cuda.synchronize()
        assert int(err.item()) & dq.DQ_DEVERR_DECODE


def _attention_case(setup, lens, G, P=16, seed=5, perm_seed=3):
    dq, tk, tv, tabs = setup
    bt, pages, slots = _layout(lens, P, perm_seed)
    kc = np.zeros((pages * P, K_CFG[1]), np.uint8)
    vc = np.zeros((pages * P, V_CFG[1]), np.uint8)
    km = np.zeros((pages * P, 2), np.uint16)
    vm = np.zeros((pages * P, 2), np.uint16)
    kh, vh = [], []
    for b, T in enumerate(lens):
        if T == 0:
            kh.append(np.zeros((8, 0, 128)))
            vh.append(np.zeros((8, 0, 128)))
            continue
        rk = oracle.encode_tokens(_tokens(seed, synth.T_K, T, part=b).astype(np.float64), tk)
        rv = oracle.encode_tokens(_tokens(seed, synth.T_V, T, part=b).astype(np.float64), tv)
        s = slots[b]
        kc[s], vc[s] = rk.containers, rv.containers
        km[s, 0], km[s, 1] = rk.o16.view(np.uint16), rk.s16.view(np.uint16)
        vm[s, 0], vm[s, 1] = rv.o16.view(np.uint16), rv.s16.view(np.uint16)
        kh.append(oracle.reconstruct_tokens(rk.symbols, rk.o16, rk.s16).transpose(1, 0, 2))
        vh.append(oracle.reconstruct_tokens(rv.symbols, rv.o16, rv.s16).transpose(1, 0, 2))
    hq = 8 * G
    q = synth.queries(800 + seed, len(lens), hq, bf16=True)
    ref = np.zeros((len(lens), hq, 128))
    for b, T in enumerate(lens):
        if T:
            ref[b] = oracle.attention(q[b:b + 1], [kh[b]], [vh[b]])[0]
    dev = dict(q=_dev(q).to(torch.bfloat16), kc=_dev(_to_pages(kc, P)), vc=_dev(_to_pages(vc, P)),
               km=_dev(km.view(np.int16).reshape(pages, P, 2)), vm=_dev(vm.view(np.int16).reshape(pages, P, 2)),
               bt=_dev(bt), lens=_dev(np.asarray(lens, np.int32)))
    return dq, tabs, dev, ref, P


def _run(dq, tabs, d, lens, P, splits=0):
    B, hq = d["q"].shape[:2]
    max_ctx = max(1, max(lens))
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((dq.dq_token_workspace_size(B, hq, max_ctx, splits),), 0xFF, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_token_decode_attention(tabs, d["q"], d["kc"], d["vc"], d["km"], d["vm"], d["bt"], d["lens"], P, max_ctx,
                                 out, ws, num_splits=splits, err_word=err)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(err.item())


@pytest.mark.parametrize("G", [1, 2, 4])
def test_token_attention_ragged_paged(setup, G):
    lens = [1, 63, 64, 65, 300, 700, 0]
    dq, tabs, d, ref, P = _attention_case(setup, lens, G)
    out, err = _run(dq, tabs, d, lens, P)
    assert err == 0
    assert np.all(out[6] == 0)
    assert row_rel_err(out[:6], ref[:6]).max() <= TOL


@pytest.mark.parametrize("splits", [1, 3, 7])
def test_token_attention_split_counts(setup, splits):
    lens = [1500, 257, 1024]
    dq, tabs, d, ref, P = _attention_case(setup, lens, 4, seed=6, perm_seed=9)
    out, err = _run(dq, tabs, d, lens, P, splits)
    assert err == 0
    assert row_rel_err(out, ref).max() <= TOL


def test_token_attention_flags_corrupt_stream(setup):
    lens = [100]
    dq, tabs, d, ref, P = _attention_case(setup, lens, 1, seed=7)
    d["kc"][0, 0, 3, 0] ^= 0x5A                # first byte (state) of slot 3 of page 0
    out, err = _run(dq, tabs, d, lens, P)
    assert err & dq.DQ_DEVERR_DECODE


def test_token_attention_context_length_outside_range_is_flagged(setup):
    """A length above max_context is attended as max_context and sets
    DQ_DEVERR_CONTEXT."""
    lens = [90, 200]
    dq, tabs, d, ref, P = _attention_case(setup, lens, 2, seed=11, perm_seed=4)
    d["lens"] = _dev(np.asarray([90, 260], np.int32))
    B, hq = d["q"].shape[:2]
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((dq.dq_token_workspace_size(B, hq, 200, 0),), 0xFF, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_token_decode_attention(tabs, d["q"], d["kc"], d["vc"], d["km"], d["vm"], d["bt"], d["lens"], P, 200,
                                 out, ws, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == dq.DQ_DEVERR_CONTEXT
    assert row_rel_err(out.cpu().numpy(), ref).max() <= TOL


def test_token_encode_then_attend(setup):
    """The device cache write feeding the device attention: the same output as
    attention over the oracle's containers, within the bar of the oracle."""
    dq, tk, tv, tabs = setup
    lens, P, G = [200, 333], 32, 4
    bt, pages, slots = _layout(lens, P, 4)
    kc = torch.zeros(dq.token_cache_shape(pages, P, K_CFG[1]), dtype=torch.uint8, device="cuda")
    vc = torch.zeros(dq.token_cache_shape(pages, P, V_CFG[1]), dtype=torch.uint8, device="cuda")
    km = torch.zeros((pages, P, 2), dtype=torch.int16, device="cuda")
    vm = torch.zeros_like(km)
    kh, vh = [], []
    for b, T in enumerate(lens):
        k, v = _tokens(9, synth.T_K, T, part=b), _tokens(9, synth.T_V, T, part=b)
        dq.dq_encode_tokens(tabs, _dev(k), _dev(v), _dev(slots[b]), kc, vc, km, vm, P)
        rk, rv = oracle.encode_tokens(k.astype(np.float64), tk), oracle.encode_tokens(v.astype(np.float64), tv)
        kh.append(oracle.reconstruct_tokens(rk.symbols, rk.o16, rk.s16).transpose(1, 0, 2))
        vh.append(oracle.reconstruct_tokens(rv.symbols, rv.o16, rv.s16).transpose(1, 0, 2))
    q = synth.queries(809, 2, 8 * G, bf16=True)
    ref = oracle.attention(q, kh, vh)
    d = dict(q=_dev(q).to(torch.bfloat16), kc=kc, vc=vc, km=km, vm=vm, bt=_dev(bt), lens=_dev(np.asarray(lens, np.int32)))
    out, err = _run(dq, tabs, d, lens, P)
    assert err == 0
    assert row_rel_err(out, ref).max() <= TOL


def test_token_qwen3_layer_sampled(setup):
    """The benchmark's per-token layer (128 x 8192 tokens, 256-token pages,
    the library's split rule), built by the device cache write: the containers
    and (o16, s16) of two sampled sequences equal the oracle's byte for byte,
    and their attention rows (all 32 query heads) meet the bar."""
    from decode_attention_dq_amd import workloads
    dq, tk, tv, tabs = setup
    w = workloads.WORKLOADS["token_qwen3_8b"]
    cache = workloads.build_token_cache(dq, tabs, w)
    q = workloads.query_rows(w)
    B, hq, P = w.batch, w.num_q_heads, w.page_size
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_token_workspace_size(B, hq, w.context), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_token_decode_attention(tabs, q, cache.k_cache, cache.v_cache, cache.k_norm, cache.v_norm,
                                 cache.block_table, cache.context_lens, P, w.context, out, ws, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    out = out.cpu().numpy()
    qh = q.float().cpu().numpy()
    bt = cache.block_table.cpu().numpy()
    for b in (5, 101):
        T = int(cache.lens[b])
        k = workloads.kv_rows(w, 0, synth.T_K, b, T).float().cpu().numpy().astype(np.float64)
        v = workloads.kv_rows(w, 0, synth.T_V, b, T).float().cpu().numpy().astype(np.float64)
        rk, rv = oracle.encode_tokens(k, tk), oracle.encode_tokens(v, tv)
        slots = workloads.slot_mapping(bt[b:b + 1], cache.lens[b:b + 1], P)
        pg = torch.as_tensor(slots // P, device="cuda", dtype=torch.long)
        off = torch.as_tensor(slots % P, device="cuda", dtype=torch.long)
        for c, r, C, meta in ((cache.k_cache, rk, w.container, cache.k_norm), (cache.v_cache, rv, w.cv, cache.v_norm)):
            got = c.permute(0, 2, 1, 3)[pg, off].reshape(T, -1).cpu().numpy()
            assert np.array_equal(got[:, :C], r.containers) and not got[:, C:].any(), b
            mt = meta[pg, off].cpu().numpy().view(np.uint16)
            assert np.array_equal(mt[:, 0], r.o16.view(np.uint16)) and np.array_equal(mt[:, 1], r.s16.view(np.uint16))
        kh = oracle.reconstruct_tokens(rk.symbols, rk.o16, rk.s16).transpose(1, 0, 2)
        vh = oracle.reconstruct_tokens(rv.symbols, rv.o16, rv.s16).transpose(1, 0, 2)
        ref = oracle.attention(qh[b:b + 1], [kh], [vh])[0]
        e = row_rel_err(out[b], ref)
        assert e.max() <= TOL, (b, e.max())


def test_token_attention_with_bf16_window(setup):
    """The paper's serving layout on the per-token format: compressed tokens
    plus a bf16 window of the newest ones (section 5.1), merged by log-sum-exp;
    window with compressed tokens, window only, and an empty sequence."""
    dq, tk, tv, tabs = setup
    lens, wl, G, cap = [300, 0, 100, 0], [64, 128, 0, 0], 4, 128
    dq_, tabs_, d, _, P = _attention_case(setup, lens, G, seed=11, perm_seed=6)
    rng = np.random.default_rng(12)
    wk = synth.round_to_bf16(rng.standard_normal((4, 8, cap, 128)).astype(np.float32))
    wv = synth.round_to_bf16(rng.standard_normal((4, 8, cap, 128)).astype(np.float32))
    q = d["q"].float().cpu().numpy()
    ref = np.zeros((4, 8 * G, 128))
    for b, T in enumerate(lens):
        if T + wl[b] == 0:
            continue
        kh = np.zeros((8, 0, 128)); vh = np.zeros((8, 0, 128))
        if T:
            rk = oracle.encode_tokens(_tokens(11, synth.T_K, T, part=b).astype(np.float64), tk)
            rv = oracle.encode_tokens(_tokens(11, synth.T_V, T, part=b).astype(np.float64), tv)
            kh = oracle.reconstruct_tokens(rk.symbols, rk.o16, rk.s16).transpose(1, 0, 2)
            vh = oracle.reconstruct_tokens(rv.symbols, rv.o16, rv.s16).transpose(1, 0, 2)
        kh = np.concatenate([kh, wk[b, :, :wl[b]].astype(np.float64)], axis=1)
        vh = np.concatenate([vh, wv[b, :, :wl[b]].astype(np.float64)], axis=1)
        ref[b] = oracle.attention(q[b:b + 1], [kh], [vh])[0]
    bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
    B, hq = q.shape[:2]
    max_ctx = max(lens)
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((dq.dq_token_workspace_size(B, hq, max_ctx),), 0xFF, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_token_decode_attention(tabs, d["q"], d["kc"], d["vc"], d["km"], d["vm"], d["bt"], d["lens"], P, max_ctx,
                                 out, ws, err_word=err, window_k=bf(wk), window_v=bf(wv),
                                 window_lens=_dev(np.asarray(wl, np.int32)))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert int(err.item()) == 0
    assert np.all(out[3] == 0)
    assert row_rel_err(out[:3], ref[:3]).max() <= TOL


BLK = 128


def _mean_rows(seed, tensor, T, b, offset):
    """[T][8][128] rows; keys get a per-(head, channel) offset that also moves
    from one 128-token block to the next: the mean the block removal takes
    out, different enough between blocks that a missing share shows."""
    x = _tokens(seed, tensor, T, part=b).astype(np.float64)
    if offset is not None:
        drift = np.random.default_rng([seed, b]).standard_normal((-(-T // BLK), 8, 128))
        x = x + offset[None] + np.repeat(drift, BLK, axis=0)[:T]
    return synth.round_to_bf16(x.astype(np.float32))


def _oracle_block_means(k):
    """Oracle means of [128 nb][8][128] key rows: q [nb][8][128], s16 [nb][8]
    and the per-token rotated mean [128 nb][1024] (head-major)."""
    nb = k.shape[0] // BLK
    kb = k.astype(np.float64).reshape(nb, BLK, 8, 128).transpose(0, 2, 1, 3)
    q, s16, mu_hat, _ = oracle.block_means(kb)
    return q, s16, np.repeat(mu_hat.reshape(nb, 1024), BLK, axis=0)


def _means_cache(dq, tabs, enc_lens, P, seed, perm_seed):
    """Device cache of whole 128-token blocks per sequence, written by one
    dq_encode_tokens_blocks call; returns the device buffers and the rows."""
    bt, pages, slots = _layout(enc_lens, P, perm_seed)
    R = dq.mean_rows_per_page(P)
    offset = np.random.default_rng(seed).standard_normal((8, 128)) * 2.0
    kx = [_mean_rows(seed, synth.T_K, T, b, offset) for b, T in enumerate(enc_lens)]
    vx = [_mean_rows(seed, synth.T_V, T, b, None) for b, T in enumerate(enc_lens)]
    d = dict(kc=torch.zeros(dq.token_cache_shape(pages, P, K_CFG[1]), dtype=torch.uint8, device="cuda"),
             vc=torch.zeros(dq.token_cache_shape(pages, P, V_CFG[1]), dtype=torch.uint8, device="cuda"),
             km=torch.zeros((pages, P, 2), dtype=torch.int16, device="cuda"),
             vm=torch.zeros((pages, P, 2), dtype=torch.int16, device="cuda"),
             kmu=torch.zeros((pages, 8, R, 128), dtype=torch.int8, device="cuda"),
             ksc=torch.zeros((pages, 8, R), dtype=torch.int16, device="cuda"),
             bt=_dev(bt))
    return d, bt, pages, slots, kx, vx


@pytest.mark.parametrize("P,bf16", [(64, False), (256, True), (128, False)])
def test_token_encode_blocks_bit_exact(setup, P, bf16):
    """Key block means on the per-token format: the INT8 means, their fp16
    scales, the key containers and (o16, s16) of the residual streams, and the
    untouched value streams equal the oracle's; a block whose first slot is
    missing sets the mean flag and leaves its key streams unwritten."""
    dq, tk, tv, tabs = setup
    lens = [256, 128, 384, 128]
    d, bt, pages, slots, kx, vx = _means_cache(dq, tabs, lens, P, seed=21, perm_seed=5)
    slots[3] = slots[3].copy()
    slots[3][0] = -1                                  # the last block has no mean row
    k, v = np.concatenate(kx), np.concatenate(vx)
    kd, vd = _dev(k), _dev(v)
    if bf16:
        kd, vd = kd.to(torch.bfloat16), vd.to(torch.bfloat16)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    ds = torch.zeros((k.shape[0], 2), dtype=torch.int32, device="cuda")
    dq.dq_encode_tokens_blocks(tabs, kd, vd, _dev(np.concatenate(slots)), d["kc"], d["vc"], d["km"], d["vm"],
                               d["kmu"], d["ksc"], P, drift_stats=ds, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == dq.DQ_DEVERR_MEAN_SLOT
    kc, vc = _from_pages(d["kc"].cpu().numpy(), K_CFG[1]), _from_pages(d["vc"].cpu().numpy(), V_CFG[1])
    km = d["km"].cpu().numpy().view(np.uint16).reshape(-1, 2)
    vm = d["vm"].cpu().numpy().view(np.uint16).reshape(-1, 2)
    kmu, ksc = d["kmu"].cpu().numpy(), d["ksc"].cpu().numpy().view(np.uint16)
    ds = ds.cpu().numpy().view(np.uint32)
    row0 = 0
    for b, T in enumerate(lens):
        q, s16, mrot = _oracle_block_means(kx[b])
        rk = oracle.encode_tokens(kx[b].astype(np.float64), tk, mean_rot=mrot)
        rv = oracle.encode_tokens(vx[b].astype(np.float64), tv)
        s = slots[b]
        live = s >= 0
        assert np.array_equal(vc[s[live], :V_CFG[1]], rv.containers[live]), b
        assert np.array_equal(vm[s[live], 0], rv.o16[live].view(np.uint16))
        assert np.array_equal(vm[s[live], 1], rv.s16[live].view(np.uint16))
        if b == 3:
            assert not kc[s[1:]].any() and not km[s[1:]].any()    # key streams of the flagged block
            row0 += T
            continue
        assert np.array_equal(kc[s, :K_CFG[1]], rk.containers), b
        assert not kc[s, K_CFG[1]:].any()
        assert np.array_equal(km[s, 0], rk.o16.view(np.uint16)) and np.array_equal(km[s, 1], rk.s16.view(np.uint16))
        st = ds[row0:row0 + T, 0]
        assert np.array_equal(st & 0xFFFF, rk.changed) and np.array_equal(st >> 16, rk.rounds)
        first = s[::BLK]
        rp, ri = first // P, (first % P) // BLK
        for h in range(8):
            assert np.array_equal(kmu[rp, h, ri], q[:, h]), (b, h)
            assert np.array_equal(ksc[rp, h, ri], s16[:, h].view(np.uint16)), (b, h)
        row0 += T


@pytest.mark.parametrize("P,G,window", [(64, 4, False), (256, 2, True), (128, 1, False), (16, 4, True)])
def test_token_attention_with_key_means(setup, P, G, window):
    """The paper's full per-token configuration: per-token streams of the key
    residuals after block-mean removal, the means' share added to every logit,
    and (with `window`) a bf16 window of the newest tokens. Context lengths end
    inside a block (its tokens use the block's mean row all the same); the
    reference is the oracle's fp64 attention over its reconstructions plus the
    dequantised means."""
    dq, tk, tv, tabs = setup
    lens = [3 * BLK + 50, BLK, 77, 0, 5 * BLK]
    enc = [max(BLK, -(-T // BLK) * BLK) for T in lens]
    d, bt, pages, slots, kx, vx = _means_cache(dq, tabs, enc, P, seed=23, perm_seed=8)
    dq.dq_encode_tokens_blocks(tabs, _dev(np.concatenate(kx)), _dev(np.concatenate(vx)), _dev(np.concatenate(slots)),
                               d["kc"], d["vc"], d["km"], d["vm"], d["kmu"], d["ksc"], P)
    B, hq, cap = len(lens), 8 * G, 128
    q = synth.queries(830, B, hq, bf16=True)
    rng = np.random.default_rng(24)
    wl = [40, 0, 128, 9, 0] if window else [0] * B
    wk = synth.round_to_bf16(rng.standard_normal((B, 8, cap, 128)).astype(np.float32))
    wv = synth.round_to_bf16(rng.standard_normal((B, 8, cap, 128)).astype(np.float32))
    ref = np.zeros((B, hq, 128))
    for b, T in enumerate(lens):
        _, _, mrot = _oracle_block_means(kx[b])
        rk = oracle.encode_tokens(kx[b].astype(np.float64), tk, mean_rot=mrot)
        rv = oracle.encode_tokens(vx[b].astype(np.float64), tv)
        kh = oracle.reconstruct_tokens(rk.symbols, rk.o16, rk.s16, mean_rot=mrot).transpose(1, 0, 2)[:, :T]
        vh = oracle.reconstruct_tokens(rv.symbols, rv.o16, rv.s16).transpose(1, 0, 2)[:, :T]
        kh = np.concatenate([kh, wk[b, :, :wl[b]].astype(np.float64)], axis=1)
        vh = np.concatenate([vh, wv[b, :, :wl[b]].astype(np.float64)], axis=1)
        if kh.shape[1]:
            ref[b] = oracle.attention(q[b:b + 1], [kh], [vh])[0]
    bf = lambda a: torch.from_numpy(synth.f32_to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)
    kw = dict(window_k=bf(wk), window_v=bf(wv), window_lens=_dev(np.asarray(wl, np.int32))) if window else {}
    max_ctx = max(lens)
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.full((dq.dq_token_workspace_size(B, hq, max_ctx),), 0xFF, dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_token_decode_attention(tabs, _dev(q).to(torch.bfloat16), d["kc"], d["vc"], d["km"], d["vm"], d["bt"],
                                 _dev(np.asarray(lens, np.int32)), P, max_ctx, out, ws, err_word=err,
                                 k_mean=d["kmu"], k_mean_scale=d["ksc"], **kw)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert int(err.item()) == 0
    live = [b for b in range(B) if lens[b] + wl[b] > 0]
    dead = [b for b in range(B) if lens[b] + wl[b] == 0]
    assert all(np.all(out[b] == 0) for b in dead)
    e = row_rel_err(out[live], ref[live])
    assert e.max() <= TOL, e.max()


def test_token_attention_needs_both_mean_buffers(setup):
    """k_mean without k_mean_scale (or the reverse) is an argument error."""
    import ctypes
    dq, tk, tv, tabs = setup
    lens = [10]
    dq_, tabs_, d, _, P = _attention_case(setup, lens, 1, seed=13)
    dummy = torch.zeros(16, dtype=torch.int8, device="cuda")
    out = torch.zeros((1, 8, 128), dtype=torch.float32, device="cuda")
    ws = torch.zeros((dq.dq_token_workspace_size(1, 8, 10),), dtype=torch.uint8, device="cuda")
    for a, b in ((dummy.data_ptr(), None), (None, dummy.data_ptr())):
        ex = dq.dq_attention_extras(None, None, None, 0, a, b)
        rc = dq._lib.dq_token_decode_attention_ext(tabs.handle, d["q"].data_ptr(), dq.DQ_DTYPE_BF16,
                                                   d["kc"].data_ptr(), d["vc"].data_ptr(), d["km"].data_ptr(),
                                                   d["vm"].data_ptr(), d["bt"].data_ptr(), d["lens"].data_ptr(), 1, 8,
                                                   d["bt"].shape[1], P, 10, 0.0, 0, ctypes.byref(ex), out.data_ptr(),
                                                   ws.data_ptr(), ws.numel(), None, None)
        assert rc == dq.DQ_ERR_INVALID_ARG


def test_token_full_config_layer_sampled(setup):
    """The paper's full per-token configuration on the benchmark's layer
    (128 x 8192: key block means, the newest 128 tokens in bf16, the library's
    split rule), built by the device cache write: for a sampled sequence the
    containers, (o16, s16), INT8 means and scales equal the oracle's byte for
    byte, and its 32 attention rows meet the bar."""
    from decode_attention_dq_amd import workloads
    dq, tk, tv, tabs = setup
    w = workloads.WORKLOADS["token_full_qwen3_8b"]
    cache = workloads.build_token_cache(dq, tabs, w)
    q = workloads.query_rows(w)
    B, hq, P = w.batch, w.num_q_heads, w.page_size
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_token_workspace_size(B, hq, w.context), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_token_decode_attention(tabs, q, cache.k_cache, cache.v_cache, cache.k_norm, cache.v_norm,
                                 cache.block_table, cache.context_lens, P, w.context, out, ws, err_word=err,
                                 window_k=cache.win_k, window_v=cache.win_v, window_lens=cache.win_lens,
                                 k_mean=cache.k_mean, k_mean_scale=cache.k_mean_scale)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    out = out.cpu().numpy()
    qh = q.float().cpu().numpy()
    bt = cache.block_table.cpu().numpy()
    b = 77
    T = int(cache.lens[b])
    full = T + w.window
    k = workloads.kv_rows(w, 0, synth.T_K, b, full).float().cpu().numpy().astype(np.float64)
    v = workloads.kv_rows(w, 0, synth.T_V, b, full).float().cpu().numpy().astype(np.float64)
    qm, s16, mrot = _oracle_block_means(k[:T])
    rk, rv = oracle.encode_tokens(k[:T], tk, mean_rot=mrot), oracle.encode_tokens(v[:T], tv)
    slots = workloads.slot_mapping(bt[b:b + 1], cache.lens[b:b + 1], P)
    pg = torch.as_tensor(slots // P, device="cuda", dtype=torch.long)
    off = torch.as_tensor(slots % P, device="cuda", dtype=torch.long)
    for c, r, C, meta in ((cache.k_cache, rk, w.container, cache.k_norm), (cache.v_cache, rv, w.cv, cache.v_norm)):
        got = c.permute(0, 2, 1, 3)[pg, off].reshape(T, -1).cpu().numpy()
        assert np.array_equal(got[:, :C], r.containers) and not got[:, C:].any()
        mt = meta[pg, off].cpu().numpy().view(np.uint16)
        assert np.array_equal(mt[:, 0], r.o16.view(np.uint16)) and np.array_equal(mt[:, 1], r.s16.view(np.uint16))
    first = slots[::BLK]
    kmu, ksc = cache.k_mean.cpu().numpy(), cache.k_mean_scale.cpu().numpy().view(np.uint16)
    R = dq.mean_rows_per_page(P)
    rp, ri = first // P, (first % P) // BLK
    assert R == P // BLK
    for h in range(8):
        assert np.array_equal(kmu[rp, h, ri], qm[:, h]) and np.array_equal(ksc[rp, h, ri], s16[:, h].view(np.uint16))
    # the window holds the sequence's newest rows in bf16
    wk = synth.round_to_bf16(k[T:].astype(np.float32)).astype(np.float64).transpose(1, 0, 2)
    wv = synth.round_to_bf16(v[T:].astype(np.float32)).astype(np.float64).transpose(1, 0, 2)
    kh = np.concatenate([oracle.reconstruct_tokens(rk.symbols, rk.o16, rk.s16, mean_rot=mrot).transpose(1, 0, 2), wk],
                        axis=1)
    vh = np.concatenate([oracle.reconstruct_tokens(rv.symbols, rv.o16, rv.s16).transpose(1, 0, 2), wv], axis=1)
    ref = oracle.attention(qh[b:b + 1], [kh], [vh])[0]
    e = row_rel_err(out[b], ref)
    assert e.max() <= TOL, e.max()
