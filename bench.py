#!/usr/bin/env python3
"""Benchmark of the fused D-Quant decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one decode step of the Qwen3-8B-shaped workload over all 36 layer
caches (batch 128, 8192-token context, 32 query / 8 KV heads, 37-byte
containers, 8 key / 6 value levels): 36 calls of dq_decode_attention, each
reading one layer's compressed cache straight from HBM. Caches are built
beforehand by the library's encoder from seeded synthetic N(0,1) rows and
stay resident in HBM.

Prints one JSON line: compressed-KV GB/s (the value), its fraction of the
8 TB/s HBM peak (the roofline entry), attention-only tokens/s, what binds the
decode kernel instead (its measured VALU-issue and LDS-active fractions, and
the integer work per symbol against the 39.3 T lane-op/s of 256 CUs x 64 lanes
x 2.4 GHz), the paper's published H20 figures as context, and the CPU oracle
timed on bounded samples (one thread and a process pool) before the GPU work.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
VALU_PEAK_TOPS = 256 * 64 * 2.4e9 / 1e12      # int32 lane-ops per second, in T
OPS_PER_SYMBOL = 8                            # least lane-ops of one rANS decode step: slot mask, x >> p, one
                                              # 24-bit multiply-add, renorm compare, shift-in, select, pointer
                                              # advance, one field extraction
METRIC = "decode-attn compressed-KV GB/s (% HBM peak) and tokens/s at B=128, 8K ctx"


def algorithmic_bytes(w, lens, window_lens=None) -> int:
    """Bytes one attention call must read: K and V containers plus their fp16
    norms for every compressed (token, KV head), 128 INT8 means and a scale per
    128-token key block when the workload has them, and 2 x 256 bytes per bf16
    window token."""
    per_stream_pair = (w.container + 2) + (w.cv + 2)
    n = int(np.sum(lens)) * w.num_kv_heads * per_stream_pair
    if getattr(w, "means", False):
        n += int(np.sum(-(-np.asarray(lens) // 128))) * w.num_kv_heads * (128 + 2)
    if window_lens is not None:
        n += int(np.sum(window_lens)) * w.num_kv_heads * 2 * 256
    return n


def host_info() -> dict:
    """The host the CPU baseline runs on: logical CPUs, CPU model, BLAS
    thread settings."""
    model = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [{k: d.get(k) for k in ("user_api", "internal_api", "num_threads")} for d in threadpool_info()]
    except Exception:   # threadpoolctl missing: report the environment only
        blas = []
    return {"cpu_count": os.cpu_count(), "cpu_model": model, "blas_threadpools": blas,
            "OMP_NUM_THREADS": os.environ.get("OMP_NUM_THREADS")}


# The CPU baseline: the oracle as it stands, on two slices of the benchmark's
# workloads, drawn by the host generators with the workloads' shapes and
# distributions: (i) the cache write of one Llama-shaped sequence (8192 tokens x
# 8 KV heads, bf16 rows with 4 outlier channels per head, K and V), (ii) decode
# + reconstruction + fp64 attention of one Qwen3-shaped sequence (8192 tokens x
# 8 KV heads, 32 query heads). Workers are forked before the process touches
# the GPU.
CPU_T = 8192


def _cpu_worker_init():
    from threadpoolctl import threadpool_limits
    global _CPU_LIMIT
    _CPU_LIMIT = threadpool_limits(1)


def _cpu_decode_unit(task):
    """One (sequence, KV head) of the Qwen3-shaped layer: the oracle encodes
    its K and V streams (not timed), then decodes, reconstructs and runs fp64
    attention for the head's 4 query heads `repeats` times (timed). Returns
    (timed seconds, compressed bytes handled, streams decoded)."""
    import oracle
    from decode_attention_dq_amd import synth
    b, g, repeats = task
    tk, tv = oracle.make_table(8, 37), oracle.make_table(6, 37)
    k = synth.gaussian_kv(3, synth.T_K, CPU_T, 8, part=b)[:, g].astype(np.float64)
    v = synth.gaussian_kv(3, synth.T_V, CPU_T, 8, part=b)[:, g].astype(np.float64)
    q = synth.queries(3, b + 1, 32)[b:b + 1, 4 * g:4 * g + 4]
    rk, rv = oracle.encode_streams(k, tk), oracle.encode_streams(v, tv)
    t0 = time.perf_counter()
    for _ in range(repeats):
        sk, _ = oracle.decode_streams(rk.containers, tk)
        sv, _ = oracle.decode_streams(rv.containers, tv)
        kh = oracle.reconstruct(sk, rk.rho16, tk)
        vh = oracle.reconstruct(sv, rv.rho16, tv)
        oracle.attention(q, [kh[None]], [vh[None]])
    return time.perf_counter() - t0, repeats * CPU_T * 2 * (37 + 2), repeats * CPU_T * 2


def _cpu_encode_unit(task):
    """The oracle's cache write of one (tensor, KV head) of a Llama-shaped
    sequence: 8192 streams of bf16 rows with the workload's outlier channels.
    Returns (timed seconds, streams)."""
    import oracle
    from decode_attention_dq_amd import synth
    b, tensor, g = task
    x = synth.gaussian_kv(2, tensor, CPU_T, 8, part=b, outliers=4, bf16=True)[:, g].astype(np.float64)
    t = oracle.make_table(8 if tensor == synth.T_K else 6, 37)
    t0 = time.perf_counter()
    oracle.encode_streams(x, t)
    return time.perf_counter() - t0, CPU_T


def cpu_baseline(workers: int, decode_repeats: int = 4) -> dict:
    """The CPU oracle timed on the host, one thread and a pool of `workers`
    processes (one BLAS thread each), on the two slices above, extrapolated to
    the full workloads. A baseline, not a target. Runs before any GPU work."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    from decode_attention_dq_amd import synth
    head_bytes = 128 * 8192 * 8 * 2 * (37 + 2)          # one Qwen3-8B layer-step of containers + norms
    enc_streams = 16 * 8192 * 8 * 2                    # the Llama-shaped cache write
    res = {"kind": "oracle", "host": host_info()}
    t_start = time.perf_counter()
    with threadpool_limits(1):
        dec = [_cpu_decode_unit((0, g, decode_repeats)) for g in range(8)]
        enc = [_cpu_encode_unit((0, tensor, g)) for tensor in (synth.T_K, synth.T_V) for g in range(8)]
    t1 = sum(d[0] for d in dec)
    single = {"decode_attention": {"GBps": round(sum(d[1] for d in dec) / t1 / 1e9, 6),
                                   "streams_per_s": round(sum(d[2] for d in dec) / t1, 1),
                                   "seconds_per_layer_step": round(head_bytes / (sum(d[1] for d in dec) / t1), 2)},
              "encode": {"streams_per_s": round(sum(e[1] for e in enc) / sum(e[0] for e in enc), 1),
                         "seconds_per_write": round(enc_streams * sum(e[0] for e in enc) / sum(e[1] for e in enc),
                                                    2)}}
    # pool: every worker busy at once; the aggregate rate is the work over the slowest worker's time
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_cpu_worker_init) as pool:
        dec = pool.map(_cpu_decode_unit, [(i // 8, i % 8, decode_repeats) for i in range(workers)], chunksize=1)
        enc = pool.map(_cpu_encode_unit, [(i // 16, (synth.T_K, synth.T_V)[(i // 8) % 2], i % 8)
                                          for i in range(workers)], chunksize=1)
    td, te = max(d[0] for d in dec), max(e[0] for e in enc)
    pool_res = {"decode_attention": {"GBps": round(sum(d[1] for d in dec) / td / 1e9, 6),
                                     "streams_per_s": round(sum(d[2] for d in dec) / td, 1),
                                     "seconds_per_layer_step": round(head_bytes / (sum(d[1] for d in dec) / td), 2)},
                "encode": {"streams_per_s": round(sum(e[1] for e in enc) / te, 1),
                           "seconds_per_write": round(enc_streams * te / sum(e[1] for e in enc), 2)}}
    res.update({
        "value": pool_res["decode_attention"]["GBps"], "unit": "GB/s", "cores": workers,
        "sample": (f"CPU oracle, baseline only. Decode slice: {workers} (sequence, KV head) units of the Qwen3-8B "
                   f"layer shape ({CPU_T} tokens each, host-drawn N(0,1) rows), each {decode_repeats}x rANS decode "
                   f"of K and V, reconstruction and fp64 attention for 4 query heads; encode slice: {workers} "
                   f"(tensor, KV head) units of 8192 Llama-shaped bf16 rows with outlier channels. value = the pool's "
                   f"decode slice in compressed GB/s (bytes over the slowest worker's time)"),
        "single_thread": single, "pool": {"workers": workers, **pool_res},
        "wall_s": round(time.perf_counter() - t_start, 1)})
    return res


def encode_measurement(dq, torch, workloads, reps: int = 3) -> dict:
    """Cache write of the Llama-3.1-8B-shaped workload (16 x 8192 tokens, 8 KV
    heads, bf16 rows with x10 outlier channels, 37-byte containers), inputs
    resident in HBM, timed with HIP events; drift statistics from the
    encoder's own per-stream counts."""
    from decode_attention_dq_amd import synth
    w = workloads.WORKLOADS["encode_llama"]
    tables = dq.dq_tables_init(dq.make_params(w.k_levels, w.container), dq.make_params(w.v_levels, w.container))
    lens = workloads.context_lengths(w)
    bt, total = workloads.page_plan(w, lens)
    H, P, C = w.num_kv_heads, w.page_size, w.container
    k = torch.cat([workloads.kv_rows(w, 0, synth.T_K, b, int(lens[b])) for b in range(w.batch)])
    v = torch.cat([workloads.kv_rows(w, 0, synth.T_V, b, int(lens[b])) for b in range(w.batch)])
    slots = torch.as_tensor(workloads.slot_mapping(bt, lens, P), device="cuda")
    kc = torch.zeros((total, H, P, C), dtype=torch.uint8, device="cuda")
    vc = torch.zeros_like(kc)
    kn = torch.zeros((total, H, P), dtype=torch.int16, device="cuda")
    vn = torch.zeros_like(kn)
    st = torch.zeros((k.shape[0], H, 2), dtype=torch.int16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    dq.dq_encode_kv(tables, k, v, slots, kc, vc, kn, vn, P, drift_stats=st, err_word=err, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dq.dq_encode_kv(tables, k, v, slots, kc, vc, kn, vn, P, drift_stats=st, err_word=err, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / reps / 1e3
    s = st.cpu().numpy().view(np.uint16)
    n_streams = 2 * k.shape[0] * H
    changed, rounds = s & 255, s >> 8
    nmse = write_nmse(dq, torch, tables, w, k, v, kc, vc, kn, vn, bt, lens)
    return {"workload": w.name, "streams": n_streams, "ms": round(t * 1e3, 3),
            "streams_per_s": round(n_streams / t, 1),
            "input_GBps": round((k.numel() + v.numel()) * k.element_size() / t / 1e9, 2),
            "output_GBps": round(n_streams * (C + 2) / t / 1e9, 2),
            "drift_rate_symbols": {"K": round(float(changed[..., 0].sum()) / (k.shape[0] * H * 128), 5),
                                   "V": round(float(changed[..., 1].sum()) / (k.shape[0] * H * 128), 5)},
            "drifted_streams": {"K": round(float((changed[..., 0] > 0).mean()), 5),
                                "V": round(float((changed[..., 1] > 0).mean()), 5)},
            "fallback_streams": int((rounds > 1).sum()), "device_errors": int(err.item()),
            "nmse": nmse}


def write_nmse(dq, torch, tables, w, k, v, kc, vc, kn, vn, bt, lens) -> dict:
    """Pooled NMSE sum |x - x_hat|^2 / sum |x|^2 of the written cache, per K and
    V: the library's symbol decoder reads the containers back, and x_hat =
    H (rho16 * step * (m - (M-1)/2)) / 128 (a measurement in torch, not a path
    step)."""
    H = torch.ones((1, 1), dtype=torch.float64, device="cuda")
    while H.shape[0] < 128:
        H = torch.cat([torch.cat([H, H], 1), torch.cat([H, -H], 1)], 0)
    P, hkv = w.page_size, w.num_kv_heads
    out, row0 = {}, np.concatenate([[0], np.cumsum(lens)])
    for name, which, x_all, cache, norm in (("K", dq.DQ_KEYS, k, kc, kn), ("V", dq.DQ_VALUES, v, vc, vn)):
        info = tables.info(which)
        half = (info["levels"] - 1) / 2.0
        num = den = 0.0
        for b in range(w.batch):
            slots = torch.as_tensor(workloads_slots(bt, lens, P, b), device="cuda", dtype=torch.long)
            pg, off = slots // P, slots % P
            cont = cache[pg, :, off].reshape(-1, cache.shape[-1]).contiguous()
            sym = torch.empty((cont.shape[0], 128), dtype=torch.uint8, device="cuda")
            dq.dq_decode_symbols(tables, which, cont, sym)
            rho = norm[pg, :, off].view(torch.float16).reshape(-1, 1).double()
            r = rho * (info["step"] * (sym.double() - half))
            xh = (r @ H) / 128.0
            x = x_all[int(row0[b]):int(row0[b + 1])].reshape(-1, 128).double()
            num += float(((x - xh) ** 2).sum())
            den += float((x ** 2).sum())
        out[name] = round(num / den, 5)
    return out


def workloads_slots(bt, lens, P, b):
    t = np.arange(int(lens[b]))
    return bt[b, t // P] * P + (t % P)


def warm_up(torch, call, copies: int, seconds: float = 0.5) -> None:
    """Back-to-back calls for about `seconds` before a workload is timed. The
    cache builds before it leave the GPU idle, and the first calls after an
    idle spell run at lower clocks (a workload timed right after its build
    measured 3-10% slower than the same calls a few hundred ms later)."""
    t0 = time.perf_counter()
    i = 0
    while True:
        for _ in range(8 * copies):
            call(i % copies)
            i += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return


def config_measurement(dq, torch, workloads, name: str, copies: int, reps: int = 5) -> dict:
    """One decode-attention call per step on another workload, rotating through
    `copies` distinct caches (their total above the 256 MB MALL). For a ragged
    batch the step also re-encodes each sequence's newest token into its slot
    first (the cache write that precedes attention in a decode step)."""
    from decode_attention_dq_amd import synth
    w = workloads.WORKLOADS[name]
    tables = dq.dq_tables_init(dq.make_params(w.k_levels, w.container), dq.make_params(w.v_levels, w.cv))
    caches = [workloads.build_cache(dq, tables, w, layer=l) for l in range(copies)]
    qs = [workloads.query_rows(w, l) for l in range(copies)]
    B, hq, hkv, P = w.batch, w.num_q_heads, w.num_kv_heads, w.page_size
    lens = caches[0].lens
    wl = caches[0].win_lens.cpu().numpy() if w.window else None
    append = w.ragged is not None
    if append:
        bt = caches[0].block_table.cpu().numpy()
        last = lens - 1
        new_slots = torch.as_tensor((bt[np.arange(B), last // P] * P + last % P).astype(np.int32), device="cuda")
        new_k = [torch.stack([workloads.kv_rows(w, l, synth.T_K, b, int(lens[b]))[-1] for b in range(B)])
                 for l in range(copies)]
        new_v = [torch.stack([workloads.kv_rows(w, l, synth.T_V, b, int(lens[b]))[-1] for b in range(B)])
                 for l in range(copies)]
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_workspace_size(B, hq, hkv, w.context), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(l, with_append=False):
        c = caches[l]
        if with_append:
            dq.dq_encode_kv(tables, new_k[l], new_v[l], new_slots, c.k_cache, c.v_cache, c.k_norm, c.v_norm, P,
                            err_word=err, stream=stream)
        if w.means:
            dq.dq_decode_attention_ext(tables, qs[l], c.k_cache, c.v_cache, c.k_norm, c.v_norm, c.block_table,
                                       c.context_lens, hkv, P, w.context, out, ws, k_mean=c.k_mean,
                                       k_mean_scale=c.k_mean_scale, err_word=err, stream=stream)
        elif w.window:
            dq.dq_decode_attention_window(tables, qs[l], c.k_cache, c.v_cache, c.k_norm, c.v_norm, c.block_table,
                                          c.context_lens, c.win_k, c.win_v, c.win_lens, hkv, P, w.context, out, ws,
                                          err_word=err, stream=stream)
        else:
            dq.dq_decode_attention(tables, qs[l], c.k_cache, c.v_cache, c.k_norm, c.v_norm, c.block_table,
                                   c.context_lens, hkv, P, w.context, out, ws, err_word=err, stream=stream)

    # Runs of reps x copies back-to-back calls, each run between one pair of
    # events (as the headline's timed region; an event pair around every call
    # adds its own gaps); the median run.
    def run(with_append=False, scale=1) -> float:
        n = reps * copies * scale
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            call(i % copies, with_append)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n

    warm_up(torch, call, copies)
    attn = float(np.median([run() for _ in range(3)]))
    nbytes = algorithmic_bytes(w, lens, wl)
    res = {"batch": B, "context": "ragged %d..%d" % w.ragged if append else w.context,
           "container_bytes": [w.container, w.cv], "page_size": P, "cache_copies": copies,
           **({"bf16_window": w.window} if w.window else {}),
           **({"key_block_means": True} if w.means else {}),
           "us_per_call": round(attn * 1e6, 2), "GBps": round(nbytes / attn / 1e9, 2),
           "hbm_frac": round(nbytes / attn / 1e9 / HBM_PEAK_GBS, 4)}
    if append:
        res["appended_streams"] = 2 * B * hkv
        # what the cache write of each sequence's newest token adds to a decode
        # step: runs with and without it, timed the same way, four times longer
        # and alternated (a difference of two runs is what is reported)
        plain_runs, both_runs = [], []
        for _ in range(5):
            plain_runs.append(run(False, 4))
            both_runs.append(run(True, 4))
        plain = float(np.median(plain_runs)) * 1e6
        both = float(np.median(both_runs)) * 1e6
        res["us_per_step_without_append"] = round(plain, 2)
        res["us_per_step_with_append"] = round(both, 2)
        res["append_encode_us"] = round(both - plain, 2)
    res["device_errors"] = int(err.item())
    return res


OTHER_WORKLOADS = {"long_llama_b4": 4, "long_llama_b1": 8, "ragged_1p96": 2, "window_split_qwen3_8b": 2,
                   "mean_qwen3_8b": 2}   # name: cache copies (their total above the 256 MB MALL)


def other_workloads(dq, torch, workloads, only=None) -> dict:
    return {name: config_measurement(dq, torch, workloads, name, copies=c)
            for name, c in OTHER_WORKLOADS.items() if only is None or name == only}


def token_attention_time(dq, torch, workloads, tables, name: str, copies: int, reps: int):
    """Mean HIP-event time of one per-token decode attention call on workload
    `name`, rotating through `copies` caches (each above the MALL), with the
    workload's bf16 window and key block means when it has them. Returns
    (seconds, compressed tokens, bytes read per call, device error word)."""
    w = workloads.WORKLOADS[name]
    caches = [workloads.build_token_cache(dq, tables, w, layer=l) for l in range(copies)]
    qs = [workloads.query_rows(w, l) for l in range(copies)]
    B, hq, P = w.batch, w.num_q_heads, w.page_size
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_token_workspace_size(B, hq, w.context), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(l):
        c = caches[l]
        kw = {}
        if w.window:
            kw.update(window_k=c.win_k, window_v=c.win_v, window_lens=c.win_lens)
        if w.means:
            kw.update(k_mean=c.k_mean, k_mean_scale=c.k_mean_scale)
        dq.dq_token_decode_attention(tables, qs[l], c.k_cache, c.v_cache, c.k_norm, c.v_norm, c.block_table,
                                     c.context_lens, P, w.context, out, ws, err_word=err, stream=stream, **kw)

    # runs of reps x copies back-to-back calls, each between one pair of events; the median run
    def run() -> float:
        n = reps * copies
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            call(i % copies)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n

    warm_up(torch, call, copies)
    t = float(np.median([run() for _ in range(3)]))
    ntok = int(np.sum(caches[0].lens))
    nbytes = ntok * (w.container + 4 + w.cv + 4)
    if w.means:
        nbytes += int(np.sum(-(-caches[0].lens // 128))) * w.num_kv_heads * (128 + 2)
    if w.window:
        nbytes += int(caches[0].win_lens.sum().item()) * w.num_kv_heads * 128 * 2 * 2
    del caches
    return t, ntok, nbytes, int(err.item())


def token_measurement(dq, torch, workloads, name: str = "token_qwen3_8b", full_name: str = "token_full_qwen3_8b",
                      copies: int = 2, reps: int = 5, enc_seqs: int = 16) -> dict:
    """The per-token format on the Qwen3-8B layer (one 1024-value stream per
    token over the 8 KV heads, 331 / 231-byte containers, 8 / 6 levels):
    decode attention rotating through `copies` caches (each above the MALL),
    the same with the paper's full configuration (key block means and a bf16
    window of the newest 128 tokens), and the cache write of `enc_seqs`
    sequences in one call."""
    from decode_attention_dq_amd import synth
    w = workloads.WORKLOADS[name]
    tables = dq.dq_token_tables_init(dq.make_params(w.k_levels, w.container), dq.make_params(w.v_levels, w.cv))
    B, hq, P = w.batch, w.num_q_heads, w.page_size
    t, ntok, nbytes, derr = token_attention_time(dq, torch, workloads, tables, name, copies, reps)
    full = workloads.WORKLOADS[full_name]
    tf, ntok_f, nbytes_f, derr_f = token_attention_time(dq, torch, workloads, tables, full_name, copies, reps)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    # cache write of enc_seqs sequences in one call
    n = enc_seqs * w.context
    k = torch.cat([workloads.kv_rows(w, 0, synth.T_K, b, w.context) for b in range(enc_seqs)])
    v = torch.cat([workloads.kv_rows(w, 0, synth.T_V, b, w.context) for b in range(enc_seqs)])
    slots = torch.arange(n, dtype=torch.int32, device="cuda")
    kc = torch.zeros(dq.token_cache_shape(n // P, P, w.container), dtype=torch.uint8, device="cuda")
    vc = torch.zeros(dq.token_cache_shape(n // P, P, w.cv), dtype=torch.uint8, device="cuda")
    km = torch.zeros((n // P, P, 2), dtype=torch.int16, device="cuda")
    vm = torch.zeros_like(km)
    st = torch.zeros((n, 2), dtype=torch.int32, device="cuda")
    dq.dq_encode_tokens(tables, k, v, slots, kc, vc, km, vm, P, drift_stats=st, err_word=err, stream=stream)
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    dq.dq_encode_tokens(tables, k, v, slots, kc, vc, km, vm, P, drift_stats=st, err_word=err, stream=stream)
    a1.record(stream)
    torch.cuda.synchronize()
    te = a0.elapsed_time(a1) / 1e3
    s = st.cpu().numpy().view(np.uint32)
    changed, rounds = s & 0xFFFF, s >> 16
    return {"workload": name, "batch": B, "context": w.context, "container_bytes": [w.container, w.cv],
            "levels": [w.k_levels, w.v_levels], "kv_heads_per_stream": 8, "cache_copies": copies,
            "us_per_call": round(t * 1e6, 2), "GBps": round(nbytes / t / 1e9, 2),
            "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4), "bytes_per_call": nbytes,
            "symbols_per_s": round(ntok * 2048 / t, 1), "device_errors": derr | derr_f | int(err.item()),
            "full_config": {"workload": full_name, "window": full.window, "key_means": True,
                            "us_per_call": round(tf * 1e6, 2), "compressed_tokens": ntok_f,
                            "bytes_per_call": nbytes_f, "GBps": round(nbytes_f / tf / 1e9, 2)},
            "encode": {"streams": 2 * n, "ms": round(te * 1e3, 3), "streams_per_s": round(2 * n / te, 1),
                       "drift_rate_symbols": {"K": round(float(changed[:, 0].sum()) / (n * 1024), 5),
                                              "V": round(float(changed[:, 1].sum()) / (n * 1024), 5)},
                       "fallback_streams": int((rounds > 1).sum())}}


def bf16_measurement(dq, torch, workloads, name: str, copies: int, dq_us: float, reps: int = 5) -> dict:
    """The uncompressed bf16 reference kernel on the same shape, rotating
    through `copies` bf16 caches (each far above the 256 MB MALL)."""
    w = workloads.WORKLOADS[name]
    caches = [workloads.build_bf16_cache(w, layer=l) for l in range(copies)]
    qs = [workloads.query_rows(w, l) for l in range(copies)]
    B, hq, hkv = w.batch, w.num_q_heads, w.num_kv_heads
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_workspace_size(B, hq, hkv, w.context), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def call(l):
        kc, vc, bt, cl = caches[l]
        dq.dq_bf16_decode_attention(qs[l], kc, vc, bt, cl, hkv, w.page_size, w.context, out, ws, stream=stream)

    warm_up(torch, call, copies)
    ev = []
    for _ in range(reps):
        for l in range(copies):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            call(l)
            e1.record(stream)
            ev.append((e0, e1))
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) for a, b in ev])) / 1e3
    nbytes = int(np.sum(workloads.context_lengths(w))) * hkv * 2 * 256
    del caches
    torch.cuda.empty_cache()
    return {"workload": name, "kv_bytes_per_call": nbytes, "cache_copies": copies, "us_per_call": round(t * 1e6, 2),
            "GBps": round(nbytes / t / 1e9, 2), "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
            "kv_bytes_vs_compressed": round(nbytes / algorithmic_bytes(w, workloads.context_lengths(w)), 3),
            "compressed_time_ratio": round(dq_us / (t * 1e6), 3)}


# the sources attn_kernel is built from: counters taken on other sources are stale
ATTN_SOURCES = ("dq_attn.hip", "dq_device.h", "dq_wave.h", "dq_sched.h", "dq_internal.h")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def copy_measurement(torch, nbytes: int = 1 << 30, reps: int = 7) -> dict:
    """The box's achievable HBM rate for a plain device-to-device copy of
    `nbytes` (read + write bytes over the median copy time), the reference the
    compressed-byte rate is also quoted against."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / 1e3)
    del src, dst
    t = float(np.median(times))
    return {"bytes": nbytes, "read_plus_write_GBps": round(2 * nbytes / t / 1e9, 1),
            "frac_of_peak": round(2 * nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}


def attn_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        h.update(open(os.path.join(ROOT, "decode_attention_dq_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def recorded_issue(kernel: str, workload: str):
    """The decode kernel's measured VALU-issue and LDS-active fractions of its
    busy CU cycles (SQ counters of one rocprofv3 pass), or None when the kernel
    sources changed since those counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_JSON))[kernel]
        sq = rec["sq"]
    except (OSError, KeyError, ValueError):
        return None
    if sq.get("source_sha256") != attn_source_hash() or sq.get("workload") != workload:
        return None
    return {"valu_issue_frac": sq["valu_issue_frac"], "lds_active_frac": sq["lds_active_frac"]}


def record_issue(sq_csv: str, workload: str = "decode_qwen3_8b", cus: int = 256, simds: int = 1024) -> dict:
    """Host only: from a rocprofv3 --pmc CSV holding SQ_INSTS_VALU,
    SQ_BUSY_CU_CYCLES and SQ_LDS_IDX_ACTIVE for the headline kernel, the VALU
    issue cycles per SIMD (4 per wave instruction) and the LDS-active cycles as
    fractions of the busy cycles per CU, written to profiles/traffic.json with
    the hash of the current kernel sources. The VALU figure counts every wave
    instruction at 4 cycles; simple VOP2 instructions issue in fewer, so it can
    pass 1 when the VALU is saturated."""
    import csv
    sums = {}
    for r in csv.DictReader(open(sq_csv)):
        if "attn_kernel<false, false, false>" in r["Kernel_Name"]:
            sums.setdefault(r["Counter_Name"], {}).setdefault(r["Dispatch_Id"], 0.0)
            sums[r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
    mean = {c: sum(v.values()) / len(v) for c, v in sums.items()}
    busy_per_cu = mean["SQ_BUSY_CU_CYCLES"] / cus
    sq = {"workload": workload, "source_sha256": attn_source_hash(),
          "valu_issue_frac": round(mean["SQ_INSTS_VALU"] * 4 / simds / busy_per_cu, 4),
          "lds_active_frac": round(mean["SQ_LDS_IDX_ACTIVE"] / mean["SQ_BUSY_CU_CYCLES"], 4),
          "dispatches": len(sums["SQ_INSTS_VALU"])}
    allrec = json.load(open(TRAFFIC_JSON))
    allrec["attn_kernel"]["sq"] = sq
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(allrec, f, indent=1)
        f.write("\n")
    return sq


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernel sources changed since those counters were taken."""
    try:
        rec = json.load(open(TRAFFIC_JSON))[kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != attn_source_hash() or rec.get("workload") != workload:
        return None
    return int(rec["traffic_bytes_per_launch"])


def record_traffic(fetch_csv: str, write_csv: str, workload: str = "decode_qwen3_8b") -> dict:
    """Host only: HBM bytes per attn_kernel launch from two rocprofv3 --pmc
    counter CSVs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch, mean over the
    headline kernel's dispatches), scaled by what the same counters read for
    a plain device copy of known size (kept in the record), written to
    profiles/traffic.json with the hash of the current kernel sources."""
    import csv

    def mean_kib(path, counter):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if r["Counter_Name"] == counter and "attn_kernel<false, false, false>" in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"no {counter} rows for attn_kernel<false, false, false> in {path}")
        return sum(vals) / len(vals), len(vals)

    allrec = json.load(open(TRAFFIC_JSON))
    rec = allrec["attn_kernel"]
    fk, nf = mean_kib(fetch_csv, "FETCH_SIZE")
    wk, nw = mean_kib(write_csv, "WRITE_SIZE")
    copy = rec["copy_bytes"]
    fs, ws_ = copy / (rec["copy_fetch_kib"] * 1024), copy / (rec["copy_write_kib"] * 1024)
    rec.update({"workload": workload, "source_sha256": attn_source_hash(), "fetch_size_kib": fk,
                "write_size_kib": wk, "fetch_scale": fs, "write_scale": ws_, "dispatches": [nf, nw],
                "traffic_bytes_per_launch": fk * 1024 * fs + wk * 1024 * ws_})
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(allrec, f, indent=1)
        f.write("\n")
    return rec


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_qwen3_8b")
    ap.add_argument("--splits", type=int, default=0, help="token splits per (sequence, KV head); 0 = library rule")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="CPU-baseline pool size (0: min(16, os.cpu_count()), this GPU's share of the host)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layers", type=int, default=0,
                    help="counter collection only: build and run this many layer caches (marked in the output)")
    ap.add_argument("--section", choices=["encode", "bf16", "token", "workloads"], default=None,
                    help="profiling only: run just this measurement and print its JSON")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                    help="only run one device-to-device copy of BYTES (reference for HBM byte counters)")
    ap.add_argument("--record-issue", metavar="SQ_CSV", default=None,
                    help="host only: write the VALU-issue and LDS-active fractions to profiles/traffic.json")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: write profiles/traffic.json from two rocprofv3 --pmc counter CSVs")
    args = ap.parse_args()
    if args.record_traffic:
        print(json.dumps(record_traffic(*args.record_traffic)), flush=True)
        return 0
    if args.record_issue:
        print(json.dumps(record_issue(args.record_issue)), flush=True)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the decode-attention path runs on "
              f"one GPU and has no multi-GPU mode.", file=sys.stderr)
        return 2

    cpu = None
    if not args.no_cpu_baseline and not (args.calibrate_copy or args.section or args.layers):
        # before anything touches the GPU: the pool's workers are forked from this process
        workers = args.cpu_workers or max(1, min(16, os.cpu_count() or 1))
        cpu = cpu_baseline(workers)
        print(f"[bench] CPU oracle baseline done in {cpu['wall_s']} s", file=sys.stderr, flush=True)

    import torch
    from decode_attention_dq_amd import dq, workloads

    if args.calibrate_copy:
        n = int(args.calibrate_copy)
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n}), flush=True)
        return 0

    if args.section == "encode":
        print(json.dumps({"encode": encode_measurement(dq, torch, workloads)}), flush=True)
        return 0
    if args.section == "token":
        print(json.dumps({"token_format": token_measurement(dq, torch, workloads)}), flush=True)
        return 0
    if args.section == "workloads":
        # --workload names one of them alone (the default runs all)
        only = args.workload if args.workload in OTHER_WORKLOADS else None
        print(json.dumps({"other_workloads": other_workloads(dq, torch, workloads, only)}), flush=True)
        return 0
    if args.section == "bf16":
        print(json.dumps({"bf16_reference": bf16_measurement(dq, torch, workloads, args.workload, copies=2,
                                                             dq_us=float("nan"))}), flush=True)
        return 0

    w = workloads.WORKLOADS[args.workload]
    if args.layers:
        import dataclasses
        w = dataclasses.replace(w, layers=int(args.layers))
    torch.cuda.set_device(0)
    tables = dq.dq_tables_init(dq.make_params(w.k_levels, w.container), dq.make_params(w.v_levels, w.container))
    t_build = time.perf_counter()
    caches = [workloads.build_cache(dq, tables, w, layer=l) for l in range(w.layers)]
    qs = [workloads.query_rows(w, l) for l in range(w.layers)]
    torch.cuda.synchronize()
    t_build = time.perf_counter() - t_build
    print(f"[bench] built {w.layers} layer caches of {w.name} in {t_build:.1f} s", file=sys.stderr, flush=True)

    B, hq, hkv = w.batch, w.num_q_heads, w.num_kv_heads
    lens = caches[0].lens
    out = torch.empty((B, hq, 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(dq.dq_workspace_size(B, hq, hkv, w.context, args.splits), dtype=torch.uint8, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def call(l):
        c = caches[l]
        dq.dq_decode_attention(tables, qs[l], c.k_cache, c.v_cache, c.k_norm, c.v_norm, c.block_table,
                               c.context_lens, hkv, w.page_size, w.context, out, ws, num_splits=args.splits,
                               err_word=err, stream=stream)

    for _ in range(args.warmup):
        for l in range(w.layers):
            call(l)
    torch.cuda.synchronize()

    # the timed region: exactly K steps of one call per layer, back to back
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record(stream)
    for _ in range(args.steps):
        for l in range(w.layers):
            call(l)
    t_all1.record(stream)
    torch.cuda.synchronize()
    if int(err.item()) != 0:
        print("[bench] device integrity error", file=sys.stderr)
        return 1
    ms_total = t_all0.elapsed_time(t_all1)
    ms_per_step = ms_total / args.steps
    per_call_s = ms_per_step / 1e3 / w.layers
    # the spread of single calls, from one more step with an event pair around each
    # call (after the timed region; the markers add their own gaps)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(w.layers)]
    for l in range(w.layers):
        ev[l][0].record(stream)
        call(l)
        ev[l][1].record(stream)
    torch.cuda.synchronize()
    call_ms = np.array([a.elapsed_time(b) for a, b in ev])

    nbytes = algorithmic_bytes(w, lens)
    symbols = int(np.sum(lens)) * hkv * 128 * 2
    gbs = nbytes / per_call_s / 1e9
    tops = symbols * OPS_PER_SYMBOL / per_call_s / 1e12
    issue = recorded_issue("attn_kernel", w.name)
    # the workspace holds one partial slot per split plus one for a bf16 window
    splits = args.splits or dq._lib.dq_workspace_size(B, hq, hkv, w.context, 0) // (B * hq * 132 * 4) - 1
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32 rANS decode; f16 MFMA products, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "context": w.context, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": 128, "layers": w.layers, "container_bytes": w.container,
                   "levels": [w.k_levels, w.v_levels], "page_size": w.page_size, "splits": int(splits),
                   "q_dtype": "bf16" if w.q_bf16 else "f32",
                   **({"layers_override": True} if args.layers else {})},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(B / (ms_per_step / 1e3), 1),
        "us_per_layer_call": round(per_call_s * 1e6, 2),
        "us_per_layer_call_p10_p50_p90": [round(float(np.percentile(call_ms, q)) * 1e3, 2) for q in (10, 50, 90)],
        "symbols_per_s": round(symbols / per_call_s, 1),
        # achieved: algorithmic bytes (K and V containers + fp16 norms of every token and KV head) per
        # call over the mean HIP-event time of the call (attn_kernel + its split merge, ~1.3% of it)
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic("attn_kernel", w.name),
                     "kernel": "attn_kernel (timed with its merge_kernel)", "algorithmic_bytes_per_call": nbytes},
        # what actually binds the kernel: instruction issue and LDS, not HBM
        "compute_bound": {
            "measured": issue,
            "alu_floor": {"ops_per_symbol": OPS_PER_SYMBOL, "achieved": round(tops, 3),
                          "peak": round(VALU_PEAK_TOPS, 3), "unit": "T lane-ops/s",
                          "frac": round(tops / VALU_PEAK_TOPS, 4),
                          "note": "the least integer work of a rANS decode step, not a count of issued "
                                  "instructions"},
            "symbols_per_call": symbols},
        "published": {"source": "D-Quant paper, section 5.3 Efficiency (Figure 3)",
                      "hardware": "1x NVIDIA H20 96GB",
                      "workload": "Qwen3-8B end-to-end decoding, 8K prompt, each at its largest feasible batch",
                      "decode_tokens_per_s": {"d_quant_2.26_bit": 563.6, "bf16": 159.5},
                      "peak_memory_GiB_d_quant_batch_128": 49.4,
                      "note": "end-to-end serving on other hardware; context, not comparable to the "
                              "attention-only figures here"},
        "cpu_baseline": cpu,
    }
    if not args.layers:
        del caches, qs
        torch.cuda.empty_cache()
        cp = copy_measurement(torch)
        cp["compressed_frac_of_copy"] = round(gbs / cp["read_plus_write_GBps"], 4)
        result["copy_reference"] = cp
        result["encode"] = encode_measurement(dq, torch, workloads)
        result["other_workloads"] = other_workloads(dq, torch, workloads)
        result["bf16_reference"] = bf16_measurement(dq, torch, workloads, w.name, copies=2,
                                                    dq_us=per_call_s * 1e6)
        torch.cuda.empty_cache()
        result["token_format"] = token_measurement(dq, torch, workloads)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
