"""Fused decode attention against the oracle's fp64 attention over its own
reconstructions of the same seeded K/V: max relative error per (sequence,
query head) row <= 2e-3. Cases: the tiny check, GQA with ragged lengths and
shuffled 16-token pages, split-count invariance, an empty context, extreme
value norms, context lengths outside the range, and sampled units of every
full-size workload (the Qwen3-8B layer, 4 x 64K and 1 x 128K contexts at two
split counts each, every sequence of the ragged 1.96-bit batch, the
bf16-window layer) in the benchmark's launch configuration."""
import numpy as np
import pytest
import torch

import oracle
from decode_attention_dq_amd import synth, workloads
from dq_cases import TOL, oracle_encode, paged_layout, row_rel_err, rho16_bits, sequence_case

pytestmark = pytest.mark.gpu


def _run(dq, tabs, q, kc, vc, kn, vn, bt, lens, hkv, P, max_ctx, splits=0):
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    B, hq = q.shape[:2]
    out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    # NaN bytes: a partial the kernels leave unwritten reaches the merge as NaN
    ws = torch.full((max(1, dq.dq_workspace_size(B, hq, hkv, max_ctx, splits)),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_decode_attention(tabs, q, dev(kc), dev(vc), dev(kn.view(np.int16)), dev(vn.view(np.int16)),
                           dev(bt), dev(np.asarray(lens, dtype=np.int32)), hkv, P, max_ctx, out, ws,
                           num_splits=splits, err_word=err)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(err.item())


def _case(tk, tv, lens, hkv, hq, P, q_bf16, seed, perm_seed=None, v_scale=None):
    """Oracle containers and expected output for a batch of sequences."""
    conts_k, conts_v, nk, nv, kh, vh = [], [], [], [], [], []
    for b, T in enumerate(lens):
        k = synth.gaussian_kv(100 + seed, synth.T_K, max(T, 1), hkv, part=b)[:T]
        v = synth.gaussian_kv(100 + seed, synth.T_V, max(T, 1), hkv, part=b)[:T]
        if v_scale is not None:
            v = (v * v_scale(T)[:, None, None]).astype(np.float32)
        if T == 0:
            C = tk.container
            conts_k.append(np.zeros((0, hkv, C), np.uint8)); conts_v.append(np.zeros((0, hkv, tv.container), np.uint8))
            nk.append(np.zeros((0, hkv), np.uint16)); nv.append(np.zeros((0, hkv), np.uint16))
            kh.append(np.zeros((hkv, 0, 128))); vh.append(np.zeros((hkv, 0, 128)))
            continue
        a, bb, c, d, e, f = sequence_case(tk, tv, k, v)
        conts_k.append(a); conts_v.append(bb); nk.append(c); nv.append(d); kh.append(e); vh.append(f)
    kc, kn, bt = paged_layout(conts_k, nk, P, perm_seed)
    vc, vn, bt2 = paged_layout(conts_v, nv, P, perm_seed)
    assert np.array_equal(bt, bt2)
    q = synth.queries(100 + seed, len(lens), hq, bf16=q_bf16)
    ref = np.zeros((len(lens), hq, 128))
    for b, T in enumerate(lens):
        if T:
            ref[b] = oracle.attention(q[b:b + 1], [kh[b]], [vh[b]])[0]
    qd = torch.from_numpy(q).cuda()
    if q_bf16:
        qd = qd.to(torch.bfloat16)   # exact: q already holds bf16 values
    return qd, kc, vc, kn, vn, bt, ref


def _tables(dq, kC=37, vC=37):
    return (oracle.make_table(8, kC), oracle.make_table(6, vC),
            dq.dq_tables_init(dq.make_params(8, kC), dq.make_params(6, vC)))


def test_attention_tiny_check(gpu_lib):
    """1 sequence, 1 KV head, 1 query head, 256 tokens, fp32 rows from seed 0."""
    dq = gpu_lib
    tk, tv, tabs = _tables(dq)
    k, v, q = synth.tiny_check_inputs(0)
    kc_, vc_, kn_, vn_, kh, vh = sequence_case(tk, tv, k, v)
    kc, kn, bt = paged_layout([kc_], [kn_], 16)
    vc, vn, _ = paged_layout([vc_], [vn_], 16)
    ref = oracle.attention(q, [kh], [vh])
    out, err = _run(dq, tabs, torch.from_numpy(q).cuda(), kc, vc, kn, vn, bt, [256], 1, 16, 256)
    assert err == 0
    e = row_rel_err(out, ref)
    assert e.max() <= TOL, e


@pytest.mark.parametrize("C", [37, 32])
def test_attention_gqa_ragged_paged(gpu_lib, C):
    dq = gpu_lib
    tk, tv, tabs = _tables(dq, C, C)
    lens = [1, 63, 64, 65, 300, 1000]
    q, kc, vc, kn, vn, bt, ref = _case(tk, tv, lens, 2, 8, 16, True, seed=C, perm_seed=7)
    out, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, lens, 2, 16, max(lens))
    assert err == 0
    e = row_rel_err(out, ref)
    assert e.max() <= TOL, e


@pytest.mark.parametrize("G", [1, 2, 3])
def test_attention_group_sizes(gpu_lib, G):
    dq = gpu_lib
    tk, tv, tabs = _tables(dq)
    lens = [200, 517]
    q, kc, vc, kn, vn, bt, ref = _case(tk, tv, lens, 2, 2 * G, 32, False, seed=10 + G)
    out, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, lens, 2, 32, max(lens))
    assert err == 0
    assert row_rel_err(out, ref).max() <= TOL


def test_page_size_not_power_of_two_is_unsupported(gpu_lib):
    """The kernel locates a token's page by shift and mask: a 48-token page is
    refused on the host before any launch."""
    dq = gpu_lib
    _, _, tabs = _tables(dq)
    z = lambda n, dt=torch.uint8: torch.zeros(n, dtype=dt, device="cuda")
    q = torch.zeros((1, 4, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((1, 4, 128), dtype=torch.float32, device="cuda")
    ws = z(dq.dq_workspace_size(1, 4, 1, 48))
    with pytest.raises(dq.DQError) as ei:
        dq.dq_decode_attention(tabs, q, z(48 * 37), z(48 * 37), z(48, torch.int16), z(48, torch.int16),
                               torch.zeros((1, 1), dtype=torch.int32, device="cuda"),
                               torch.full((1,), 48, dtype=torch.int32, device="cuda"), 1, 48, 48, out, ws)
    assert ei.value.code == dq.DQ_ERR_UNSUPPORTED


def test_split_invariance(gpu_lib):
    dq = gpu_lib
    tk, tv, tabs = _tables(dq)
    lens = [3000, 1700, 256]
    q, kc, vc, kn, vn, bt, ref = _case(tk, tv, lens, 1, 4, 64, True, seed=3)
    outs = []
    for s in (1, 2, 3, 12):
        out, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, lens, 1, 64, 3000, splits=s)
        assert err == 0
        assert row_rel_err(out, ref).max() <= TOL, s
        outs.append(out)
    # split counts change the running maxima the fp16 p.v weights are scaled by, so results
    # differ at the level of that rounding (2^-11 relative per weight), far inside TOL
    for o in outs[1:]:
        assert row_rel_err(o, outs[0]).max() <= 5e-4


@pytest.mark.parametrize("splits", [0, 2, 3, 7, 13])
def test_every_job_class(gpu_lib, splits):
    """Lengths on both sides of every 256-token tile and split boundary, so
    that the longest-first job order draws jobs from every tile class (full
    splits, last splits of 1 .. K tiles, empty sequences) at several split
    lengths; every partial the merge reads must have been written."""
    dq = gpu_lib
    tk, tv, tabs = _tables(dq)
    lens = [0, 1, 255, 256, 257, 511, 769, 1024, 1535, 1536, 1537, 2047, 3072, 3300]
    q, kc, vc, kn, vn, bt, ref = _case(tk, tv, lens, 2, 4, 16, True, seed=8, perm_seed=8)
    out, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, lens, 2, 16, max(lens), splits=splits)
    assert err == 0
    assert np.all(out[0] == 0)
    assert row_rel_err(out[1:], ref[1:]).max() <= TOL


def test_empty_context_gives_zeros(gpu_lib):
    dq = gpu_lib
    tk, tv, tabs = _tables(dq)
    lens = [0, 70, 0]
    q, kc, vc, kn, vn, bt, ref = _case(tk, tv, lens, 1, 2, 16, True, seed=4)
    out, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, lens, 1, 16, 70)
    assert err == 0
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert row_rel_err(out[1:2], ref[1:2]).max() <= TOL


def test_extreme_value_norms(gpu_lib):
    """Value rows whose norms span 1e-5 .. 1e3 inside one sequence."""
    dq = gpu_lib
    tk, tv, tabs = _tables(dq)
    lens = [700]
    scale = lambda T: 10.0 ** np.random.default_rng(1).uniform(-5, 3, T)
    q, kc, vc, kn, vn, bt, ref = _case(tk, tv, lens, 1, 4, 16, True, seed=5, v_scale=scale)
    out, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, lens, 1, 16, 700)
    assert err == 0
    assert row_rel_err(out, ref).max() <= TOL


def test_corrupt_container_sets_error(gpu_lib):
    dq = gpu_lib
    tk, tv, tabs = _tables(dq)
    lens = [128]
    q, kc, vc, kn, vn, bt, ref = _case(tk, tv, lens, 1, 1, 16, True, seed=6)
    kc = kc.copy()
    kc[bt[0, 2], 0, 5, :3] = 0     # state below 2^16
    _, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, lens, 1, 16, 128)
    assert err & dq.DQ_DEVERR_DECODE


def _oracle_unit(tk, tv, k, v, T, kdev, vdev, q_rows):
    """Oracle side of one (sequence, KV head) unit of a full-size layer:
    containers compared with the device's, and the fp64 attention rows of its
    query heads. k, v: [T + W][1][128] host rows; the last W enter attention as
    their bf16 values (the window)."""
    kc_, vc_, kn_, vn_, kh, vh = sequence_case(tk, tv, k[:T], v[:T])
    W = k.shape[0] - T
    if W:
        kh = np.concatenate([kh, synth.round_to_bf16(k[T:]).transpose(1, 0, 2).astype(np.float64)], axis=1)
        vh = np.concatenate([vh, synth.round_to_bf16(v[T:]).transpose(1, 0, 2).astype(np.float64)], axis=1)
    same = np.array_equal(kdev, kc_[:, 0]) and np.array_equal(vdev, vc_[:, 0])
    return same, oracle.attention(q_rows, [kh], [vh])[0]


def _full_size_sampled(dq, w, samples, splits=(0,)):
    """The full layer in the benchmark's launch configuration (and at each
    extra split count), checked on sampled (sequence, KV head) units: their
    containers byte for byte, and the attention rows of their query heads
    within TOL of the oracle's fp64 attention. The oracle side of the units
    runs in a thread pool (NumPy releases the GIL in its array operations)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    tk, tv = oracle.make_table(w.k_levels, w.container), oracle.make_table(w.v_levels, w.cv)
    tabs = dq.dq_tables_init(dq.make_params(w.k_levels, w.container), dq.make_params(w.v_levels, w.cv))
    cache = workloads.build_cache(dq, tabs, w)
    q = workloads.query_rows(w)
    B, hq, hkv = w.batch, w.num_q_heads, w.num_kv_heads
    outs = {}
    for ns in splits:
        out = torch.full((B, hq, 128), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.full((dq.dq_workspace_size(B, hq, hkv, w.context, ns),), 0xFF, dtype=torch.uint8,
                        device="cuda")
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        if w.window:
            dq.dq_decode_attention_window(tabs, q, cache.k_cache, cache.v_cache, cache.k_norm, cache.v_norm,
                                          cache.block_table, cache.context_lens, cache.win_k, cache.win_v,
                                          cache.win_lens, hkv, w.page_size, w.context, out, ws, num_splits=ns,
                                          err_word=err)
        else:
            dq.dq_decode_attention(tabs, q, cache.k_cache, cache.v_cache, cache.k_norm, cache.v_norm,
                                   cache.block_table, cache.context_lens, hkv, w.page_size, w.context, out, ws,
                                   num_splits=ns, err_word=err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0, ns
        outs[ns] = out.cpu().numpy()
    qh = q.float().cpu().numpy()
    bt = cache.block_table.cpu().numpy()
    G = hq // hkv
    tasks = []
    for b, g in samples:
        T = int(cache.lens[b])
        W = int(cache.win_lens[b]) if w.window else 0
        k = workloads.kv_rows(w, 0, synth.T_K, b, T + W)[:, g:g + 1].float().cpu().numpy()
        v = workloads.kv_rows(w, 0, synth.T_V, b, T + W)[:, g:g + 1].float().cpu().numpy()
        slots = workloads.slot_mapping(bt[b:b + 1], cache.lens[b:b + 1], w.page_size)
        pg = torch.as_tensor(slots // w.page_size, device="cuda", dtype=torch.long)
        off = torch.as_tensor(slots % w.page_size, device="cuda", dtype=torch.long)
        tasks.append((tk, tv, k, v, T, cache.k_cache[pg, g, off].cpu().numpy(),
                      cache.v_cache[pg, g, off].cpu().numpy(), qh[b:b + 1, g * G:(g + 1) * G]))
    del cache
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        results = list(ex.map(lambda t: _oracle_unit(*t), tasks))
    for (b, g), (same, ref) in zip(samples, results):
        assert same, ("containers differ", b, g)
        for ns, out in outs.items():
            e = row_rel_err(out[b, g * G:(g + 1) * G], ref)
            assert e.max() <= TOL, (b, g, ns, e)


def test_full_qwen3_layer_sampled(gpu_lib):
    """Eight (sequence, KV head) units over the batch and every KV head."""
    dq = gpu_lib
    _full_size_sampled(dq, workloads.WORKLOADS["decode_qwen3_8b"],
                       [(0, 0), (17, 1), (33, 2), (57, 3), (70, 4), (91, 5), (110, 6), (127, 7)])


def test_long_context_4x64k_sampled(gpu_lib):
    """Batch 4 at 65,536 tokens: two units of every sequence, at the library's
    split count and at a forced 13 (a count that leaves a short last split)."""
    dq = gpu_lib
    _full_size_sampled(dq, workloads.WORKLOADS["long_llama_b4"],
                       [(0, 0), (0, 5), (1, 1), (1, 6), (2, 2), (2, 7), (3, 3), (3, 4)], splits=(0, 13))


def test_long_context_128k_sampled(gpu_lib):
    """One sequence of 131,072 tokens, two KV heads, at the library's split
    count (128 splits, 129 partials per merge) and at a forced 37."""
    dq = gpu_lib
    _full_size_sampled(dq, workloads.WORKLOADS["long_llama_b1"], [(0, 5), (0, 2)], splits=(0, 37))


def test_ragged_low_budget_sampled(gpu_lib):
    """Every sequence of the ragged 1.96-bit batch, the KV head rotating with
    the sequence."""
    dq = gpu_lib
    w = workloads.WORKLOADS["ragged_1p96"]
    _full_size_sampled(dq, w, [(b, b % w.num_kv_heads) for b in range(w.batch)])


def test_window_split_budget_layer_sampled(gpu_lib):
    """A Qwen3-8B layer at batch 128 with the 128 newest tokens in bf16 and
    41/27-byte key/value containers."""
    dq = gpu_lib
    _full_size_sampled(dq, workloads.WORKLOADS["window_split_qwen3_8b"], [(0, 0), (90, 5), (127, 7)])


def test_decode_step_with_append(gpu_lib):
    """One decode step of a ragged paged batch at the 1.96-bit budget: the device
    writes each sequence's newest token into its slot (dq_encode_kv), then attends
    over all tokens including it."""
    dq = gpu_lib
    tk, tv, tabs = _tables(dq, 32, 32)
    lens, hkv, hq, P, seed = [17, 200, 1, 64, 333], 2, 8, 16, 21
    q, kc, vc, kn, vn, bt, ref = _case(tk, tv, lens, hkv, hq, P, True, seed=seed, perm_seed=3)
    B = len(lens)
    last = np.array(lens) - 1
    slots = (bt[np.arange(B), last // P] * P + last % P).astype(np.int32)
    new_k = np.stack([synth.gaussian_kv(100 + seed, synth.T_K, T, hkv, part=b)[T - 1] for b, T in enumerate(lens)])
    new_v = np.stack([synth.gaussian_kv(100 + seed, synth.T_V, T, hkv, part=b)[T - 1] for b, T in enumerate(lens)])
    kc0, vc0, kn0, vn0 = kc.copy(), vc.copy(), kn.copy(), vn.copy()
    for arr in (kc0, vc0, kn0, vn0):
        arr[slots // P, :, slots % P] = 0          # the newest tokens are not in the cache yet
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dkc, dvc, dkn, dvn = dev(kc0), dev(vc0), dev(kn0.view(np.int16)), dev(vn0.view(np.int16))
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    dq.dq_encode_kv(tabs, dev(new_k), dev(new_v), dev(slots), dkc, dvc, dkn, dvn, P, err_word=err)
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_workspace_size(B, hq, hkv, max(lens)), dtype=torch.uint8, device="cuda")
    dq.dq_decode_attention(tabs, q, dkc, dvc, dkn, dvn, dev(bt), dev(np.array(lens, dtype=np.int32)), hkv, P,
                           max(lens), out, ws, err_word=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert np.array_equal(dkc.cpu().numpy(), kc) and np.array_equal(dvc.cpu().numpy(), vc)
    assert np.array_equal(dkn.cpu().numpy().view(np.uint16), kn) and np.array_equal(dvn.cpu().numpy().view(np.uint16), vn)
    assert row_rel_err(out.cpu().numpy(), ref).max() <= TOL


def test_context_length_outside_range_is_flagged(gpu_lib):
    """A length above max_context is attended as max_context, a negative one
    as 0, and either sets DQ_DEVERR_CONTEXT; lengths inside the range do not."""
    dq = gpu_lib
    tk, tv, tabs = _tables(dq)
    q, kc, vc, kn, vn, bt, ref = _case(tk, tv, [100, 200], 1, 4, 16, True, seed=9, perm_seed=9)
    out, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, [100, 200], 1, 16, 200)
    assert err == 0 and row_rel_err(out, ref).max() <= TOL
    out, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, [100, 300], 1, 16, 200)
    assert err == dq.DQ_DEVERR_CONTEXT
    assert row_rel_err(out, ref).max() <= TOL
    out, err = _run(dq, tabs, q, kc, vc, kn, vn, bt, [-3, 200], 1, 16, 200)
    assert err == dq.DQ_DEVERR_CONTEXT
    assert np.all(out[0] == 0) and row_rel_err(out[1:], ref[1:]).max() <= TOL
