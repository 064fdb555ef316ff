"""The benchmark workloads, their seeded inputs and their paged caches.

Shapes follow the model layers D-Quant evaluates (section 5.1: Qwen3-8B and
Llama-3.1-8B, 32 query heads, 8 KV heads, head_dim 128) at the 2.26-bit
budget (8 key levels, 6 value levels, 37-byte containers) and a 1.96-bit
budget (32-byte containers). Inputs are seeded synthetic Gaussian rows
(optionally with x10 outlier channels), standing in for captured KV; caches
are filled by the library's own encoder (``dq_encode_kv``).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import synth


@dataclass
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    context: int                 # uniform context, or the upper bound of a ragged batch
    k_levels: int = 8
    v_levels: int = 6
    container: int = 37
    page_size: int = 256
    layers: int = 1
    q_bf16: bool = True
    kv_bf16: bool = False
    outliers: int = 0
    ragged: tuple | None = None  # (lo, hi) inclusive range of context lengths
    config_id: int = 0
    extra: dict = field(default_factory=dict)
    container_v: int = 0         # value container bytes (0: same as `container`)
    window: int = 0              # most recent tokens kept uncompressed in bf16
    key_offset: float = 0.0      # std of a per-(layer, KV head, channel) offset added to the keys
    means: bool = False          # keys written in 128-token blocks with their channel means
    token: bool = False          # the per-token format: one 1024-value stream per token over the 8 KV heads

    @property
    def cv(self) -> int:
        return self.container_v or self.container


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 256, page_size=16, q_bf16=False, config_id=1),
    "encode_llama": Workload("encode_llama", 16, 32, 8, 8192, kv_bf16=True, outliers=4, config_id=2),
    "decode_qwen3_8b": Workload("decode_qwen3_8b", 128, 32, 8, 8192, layers=36, config_id=3),
    "long_llama_b4": Workload("long_llama_b4", 4, 32, 8, 65536, config_id=4),
    "long_llama_b1": Workload("long_llama_b1", 1, 32, 8, 131072, config_id=4, extra={"part": 1}),
    "ragged_1p96": Workload("ragged_1p96", 64, 32, 8, 16384, container=32, page_size=16,
                            ragged=(1024, 16384), config_id=5),
    # the paper's serving layout: last 128 tokens in bf16, keys given more bytes than values
    "window_split_qwen3_8b": Workload("window_split_qwen3_8b", 128, 32, 8, 8192, container=41, container_v=27,
                                      window=128, config_id=6),
    # keys with a strong channel mean, removed per 128-token block (the paper's key preprocessing)
    "mean_qwen3_8b": Workload("mean_qwen3_8b", 128, 32, 8, 8192, key_offset=2.0, means=True, config_id=7),
    # the paper's default format: 331 / 231-byte per-token containers, 8 / 6 levels
    "token_qwen3_8b": Workload("token_qwen3_8b", 128, 32, 8, 8192, container=331, container_v=231, token=True,
                               config_id=8),
    # the paper's full per-token configuration: 331 / 231-byte containers, key block means,
    # the last 128 tokens in bf16
    "token_full_qwen3_8b": Workload("token_full_qwen3_8b", 128, 32, 8, 8192, container=331, container_v=231,
                                    token=True, window=128, key_offset=2.0, means=True, config_id=9),
}


def context_lengths(w: Workload) -> np.ndarray:
    if w.ragged is None:
        return np.full(w.batch, w.context, dtype=np.int32)
    return synth.ragged_lengths(w.config_id, w.batch, *w.ragged)


def page_plan(w: Workload, lens: np.ndarray):
    """Physical pages per sequence: a seeded permutation for ragged batches,
    in order otherwise. Returns (block_table [B][max_pages] int32, num_pages)."""
    P = w.page_size
    npages = [-(-int(t) // P) for t in lens]
    total = int(sum(npages))
    perm = synth.page_permutation(w.config_id, total) if w.ragged is not None else np.arange(total, dtype=np.int32)
    maxp = max(1, -(-w.context // P))
    bt = np.zeros((w.batch, maxp), dtype=np.int32)
    nxt = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[nxt:nxt + n]
        nxt += n
    return bt, total


def slot_mapping(block_table: np.ndarray, lens: np.ndarray, page_size: int) -> np.ndarray:
    """Physical slot of every token of every sequence, sequences concatenated."""
    out = []
    for b, T in enumerate(lens):
        t = np.arange(int(T))
        out.append(block_table[b, t // page_size] * page_size + (t % page_size))
    return np.concatenate(out).astype(np.int32)


def kv_rows(w: Workload, layer: int, tensor: int, b: int, T: int, device="cuda"):
    """K (tensor = synth.T_K) or V rows of sequence b: [T][Hkv][128] on the device."""
    import torch
    seed = int(np.random.SeedSequence([0, w.config_id, tensor, layer, b]).generate_state(1)[0])
    ch = None
    if w.outliers:
        ch = synth.outlier_channels(w.config_id, synth.T_OUTLIER_K if tensor == synth.T_K else synth.T_OUTLIER_V,
                                    w.num_kv_heads, w.outliers)
    x = synth.device_gaussian((T, w.num_kv_heads, 128), seed, device=device,
                              dtype=torch.bfloat16 if w.kv_bf16 else torch.float32,
                              outlier_channels=ch)
    if w.key_offset and tensor == synth.T_K:
        oseed = int(np.random.SeedSequence([0, w.config_id, synth.T_K, layer, 999]).generate_state(1)[0])
        off = synth.device_gaussian((w.num_kv_heads, 128), oseed, device=device, dtype=torch.float32) * w.key_offset
        x = (x.float() + off[None]).to(x.dtype)
    return x


def query_rows(w: Workload, layer: int = 0, device="cuda"):
    import torch
    seed = int(np.random.SeedSequence([0, w.config_id, synth.T_Q, layer]).generate_state(1)[0])
    return synth.device_gaussian((w.batch, w.num_q_heads, 128), seed, device=device,
                                 dtype=torch.bfloat16 if w.q_bf16 else torch.float32)


@dataclass
class Cache:
    k_cache: object
    v_cache: object
    k_norm: object
    v_norm: object
    block_table: object
    context_lens: object
    lens: np.ndarray
    drift_stats: object | None = None
    k_mean: object | None = None       # int8 [pages][Hkv][R][128] with the block means
    k_mean_scale: object | None = None
    win_k: object | None = None        # bf16 [B][Hkv][window][128]
    win_v: object | None = None
    win_lens: object | None = None


def build_cache(dq, tables, w: Workload, layer: int = 0, keep_stats: bool = False, device="cuda") -> Cache:
    """Encode every sequence of one layer into a fresh paged cache. With a
    window, the last `w.window` tokens of each sequence stay uncompressed (bf16)
    and only the earlier ones are encoded."""
    import torch
    full = context_lengths(w)
    lens = np.maximum(full - w.window, 0).astype(np.int32)
    bt, total = page_plan(w, lens)
    P, H = w.page_size, w.num_kv_heads
    kc = torch.zeros((total, H, P, w.container), dtype=torch.uint8, device=device)
    vc = torch.zeros((total, H, P, w.cv), dtype=torch.uint8, device=device)
    kn = torch.zeros((total, H, P), dtype=torch.int16, device=device)
    vn = torch.zeros((total, H, P), dtype=torch.int16, device=device)
    if w.window:
        wk = torch.zeros((w.batch, H, w.window, 128), dtype=torch.bfloat16, device=device)
        wv = torch.zeros_like(wk)
    if w.means:
        R = dq.mean_rows_per_page(P)
        km = torch.zeros((total, H, R, 128), dtype=torch.int8, device=device)
        ks = torch.zeros((total, H, R), dtype=torch.int16, device=device)
    stats = []
    for b in range(w.batch):
        T = int(lens[b])
        slots = torch.as_tensor(slot_mapping(bt[b:b + 1], lens[b:b + 1], P), device=device)
        k = kv_rows(w, layer, synth.T_K, b, int(full[b]), device)
        v = kv_rows(w, layer, synth.T_V, b, int(full[b]), device)
        if w.window:
            nw = int(full[b]) - T
            wk[b, :, :nw] = k[T:].transpose(0, 1).to(torch.bfloat16)
            wv[b, :, :nw] = v[T:].transpose(0, 1).to(torch.bfloat16)
            k, v = k[:T].contiguous(), v[:T].contiguous()
        st = torch.zeros((T, H, 2), dtype=torch.int16, device=device) if keep_stats else None
        if T and w.means:
            if T % 128:
                raise ValueError("block writes need whole 128-token blocks")
            dq.dq_encode_kv_blocks(tables, k, v, slots, kc, vc, kn, vn, km, ks, P, drift_stats=st)
        elif T:
            dq.dq_encode_kv(tables, k, v, slots, kc, vc, kn, vn, P, drift_stats=st)
        if keep_stats:
            stats.append(st)
        del k, v
    c = Cache(kc, vc, kn, vn, torch.as_tensor(bt, device=device),
              torch.as_tensor(lens, device=device), lens,
              torch.cat(stats) if keep_stats else None)
    if w.means:
        c.k_mean, c.k_mean_scale = km, ks
    if w.window:
        c.win_k, c.win_v = wk, wv
        c.win_lens = torch.as_tensor((full - lens).astype(np.int32), device=device)
    return c


def build_token_cache(dq, tables, w: Workload, layer: int = 0, keep_stats: bool = False, device="cuda") -> Cache:
    """Encode every sequence of one layer into a per-token cache: containers
    [pages][ceil(C/4)][P][4] (dword-interleaved across a page's slots), and
    (o16, s16) metadata [pages][P][2] in the norm fields. With a window, the
    last `w.window` tokens of each sequence stay in bf16 ([B][8][window][128]);
    with means, the keys are written in 128-token blocks with their block means
    ([pages][8][R][128] int8 and [pages][8][R] fp16 scales)."""
    import torch
    full = context_lengths(w)
    lens = np.maximum(full - w.window, 0).astype(np.int32)
    bt, total = page_plan(w, lens)
    P, H = w.page_size, w.num_kv_heads
    kc = torch.zeros(dq.token_cache_shape(total, P, w.container), dtype=torch.uint8, device=device)
    vc = torch.zeros(dq.token_cache_shape(total, P, w.cv), dtype=torch.uint8, device=device)
    km = torch.zeros((total, P, 2), dtype=torch.int16, device=device)
    vm = torch.zeros((total, P, 2), dtype=torch.int16, device=device)
    if w.window:
        wk = torch.zeros((w.batch, H, w.window, 128), dtype=torch.bfloat16, device=device)
        wv = torch.zeros_like(wk)
    if w.means:
        R = dq.mean_rows_per_page(P)
        kmu = torch.zeros((total, H, R, 128), dtype=torch.int8, device=device)
        ksc = torch.zeros((total, H, R), dtype=torch.int16, device=device)
    stats = []
    for b in range(w.batch):
        T = int(lens[b])
        slots = torch.as_tensor(slot_mapping(bt[b:b + 1], lens[b:b + 1], P), device=device)
        k = kv_rows(w, layer, synth.T_K, b, int(full[b]), device)
        v = kv_rows(w, layer, synth.T_V, b, int(full[b]), device)
        if w.window:
            nw = int(full[b]) - T
            wk[b, :, :nw] = k[T:].transpose(0, 1).to(torch.bfloat16)
            wv[b, :, :nw] = v[T:].transpose(0, 1).to(torch.bfloat16)
            k, v = k[:T].contiguous(), v[:T].contiguous()
        st = torch.zeros((T, 2), dtype=torch.int32, device=device) if keep_stats else None
        if T and w.means:
            if T % 128:
                raise ValueError("block writes need whole 128-token blocks")
            dq.dq_encode_tokens_blocks(tables, k, v, slots, kc, vc, km, vm, kmu, ksc, P, drift_stats=st)
        elif T:
            dq.dq_encode_tokens(tables, k, v, slots, kc, vc, km, vm, P, drift_stats=st)
        if keep_stats:
            stats.append(st)
        del k, v
    c = Cache(kc, vc, km, vm, torch.as_tensor(bt, device=device), torch.as_tensor(lens, device=device), lens,
              torch.cat(stats) if keep_stats else None)
    if w.means:
        c.k_mean, c.k_mean_scale = kmu, ksc
    if w.window:
        c.win_k, c.win_v = wk, wv
        c.win_lens = torch.as_tensor((full - lens).astype(np.int32), device=device)
    return c


def build_bf16_cache(w: Workload, layer: int = 0, device="cuda"):
    """The same sequences as build_cache, stored uncompressed: bf16 K and V
    caches [pages][Hkv][P][128] with the same page plan. Rows past a
    sequence's end are left unset. Returns (k_cache, v_cache, block_table,
    context_lens) as device tensors."""
    import torch
    lens = context_lengths(w)
    bt, total = page_plan(w, lens)
    P, H = w.page_size, w.num_kv_heads
    kc = torch.empty((total, H, P, 128), dtype=torch.bfloat16, device=device)
    vc = torch.empty_like(kc)
    for b in range(w.batch):
        T = int(lens[b])
        slots = torch.as_tensor(slot_mapping(bt[b:b + 1], lens[b:b + 1], P), device=device, dtype=torch.long)
        pg, off = slots // P, slots % P
        kc[pg, :, off] = kv_rows(w, layer, synth.T_K, b, T, device).to(torch.bfloat16)
        vc[pg, :, off] = kv_rows(w, layer, synth.T_V, b, T, device).to(torch.bfloat16)
    return kc, vc, torch.as_tensor(bt, device=device), torch.as_tensor(lens, device=device)
