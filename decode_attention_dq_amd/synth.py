"""Seeded synthetic inputs shared by the tests, the bench and the CPU baseline.

This module holds random-number generation and dtype rounding only: none of
the codec's arithmetic lives here, so both the HIP path and the CPU oracle can
take their inputs from it without sharing any of the method.

Workload shapes follow the model layers the D-Quant paper evaluates on
(Qwen3-8B and Llama-3.1-8B: 32 query heads, 8 KV heads, head_dim 128; paper
section 5.1 "Models and benchmarks"). The paper measures on captured KV of
those models; here seeded Gaussian data of the same shape stands in for it:

* i.i.d. N(0, 1) keys/values (the distribution the paper's preprocessing
  aims at, section 3.2 "Observations");
* optionally a few outlier channels per (tensor, KV head) scaled x10, the
  structure Hadamard rotation is meant to spread (section 3.2, Table 1).

Seeding: the tiny check draws K, then V, then q from ``default_rng(0)`` as
float64 and casts to float32. Every other tensor draws from its own
``SeedSequence([0, config, tensor, layer, part])`` stream, so any slice
(for instance one sequence of a batch) can be regenerated on its own.
"""
from __future__ import annotations

import numpy as np

HEAD_DIM = 128

# tensor ids used in the SeedSequence key
T_K, T_V, T_Q, T_LENS, T_PAGES, T_OUTLIER_K, T_OUTLIER_V = range(7)


def rng_for(config: int, tensor: int, layer: int = 0, part: int = 0) -> np.random.Generator:
    """Independent generator for one (config, tensor, layer, part) slice."""
    return np.random.default_rng(np.random.SeedSequence([0, config, tensor, layer, part]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def tiny_check_inputs(seed: int = 0, tokens: int = 256):
    """1 sequence, 1 KV head, 1 query head, head_dim 128.

    K and V are i.i.d. N(0,1) drawn as float64 from ``default_rng(seed)`` (K
    first, then V, then the query) and cast to float32.
    Returns (k [tokens][1][128] f32, v [tokens][1][128] f32, q [1][1][128] f32).
    """
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((tokens, 1, HEAD_DIM)).astype(np.float32)
    v = rng.standard_normal((tokens, 1, HEAD_DIM)).astype(np.float32)
    q = rng.standard_normal((1, 1, HEAD_DIM)).astype(np.float32)
    return k, v, q


def outlier_channels(config: int, tensor_outlier: int, n_kv_heads: int, count: int = 4) -> np.ndarray:
    """Per KV head, `count` distinct channel indices (seeded) that get scaled."""
    rng = rng_for(config, tensor_outlier)
    return np.stack([rng.choice(HEAD_DIM, count, replace=False) for _ in range(n_kv_heads)])


def gaussian_kv(config: int, tensor: int, n_tokens: int, n_kv_heads: int, *, layer: int = 0,
                part: int = 0, outliers: int = 0, outlier_scale: float = 10.0,
                bf16: bool = False) -> np.ndarray:
    """Rows [n_tokens][n_kv_heads][128] of N(0,1) float32 data.

    With ``outliers > 0`` that many channels per KV head (the same for every
    token and every part of the tensor) are multiplied by ``outlier_scale``.
    With ``bf16`` the values are rounded to bfloat16 (still returned as float32;
    use :func:`f32_to_bf16_bits` for the bit patterns).
    """
    rng = rng_for(config, tensor, layer, part)
    x = rng.standard_normal((n_tokens, n_kv_heads, HEAD_DIM)).astype(np.float32)
    if outliers:
        ch = outlier_channels(config, T_OUTLIER_K if tensor == T_K else T_OUTLIER_V,
                              n_kv_heads, outliers)
        for g in range(n_kv_heads):
            x[:, g, ch[g]] *= np.float32(outlier_scale)
    if bf16:
        x = round_to_bf16(x)
    return x


def queries(config: int, batch: int, n_q_heads: int, *, layer: int = 0, bf16: bool = True) -> np.ndarray:
    """Query rows [batch][n_q_heads][128], N(0,1), optionally rounded to bfloat16."""
    q = rng_for(config, T_Q, layer).standard_normal((batch, n_q_heads, HEAD_DIM)).astype(np.float32)
    return round_to_bf16(q) if bf16 else q


def ragged_lengths(config: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """Context lengths drawn uniformly from [lo, hi] (inclusive), int32."""
    return rng_for(config, T_LENS).integers(lo, hi + 1, batch).astype(np.int32)


def page_permutation(config: int, n_pages: int) -> np.ndarray:
    """A seeded permutation of physical page ids, int32."""
    return rng_for(config, T_PAGES).permutation(n_pages).astype(np.int32)


def device_gaussian(shape, seed: int, *, device="cuda", dtype=None, outlier_channels=None,
                    outlier_scale: float = 10.0):
    """N(0,1) float32 rows drawn on the device by torch's seeded generator.

    For workloads too large to draw on the host. ``outlier_channels`` is an
    int array [n_kv_heads][count] (axis -2 of ``shape`` is the KV head): those
    channels are multiplied by ``outlier_scale``. With ``dtype`` the result is
    cast (rounded to nearest even for bfloat16). Tests that check a slice
    against the CPU oracle copy that slice of this very tensor to the host.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32)
    if outlier_channels is not None:
        ch = np.asarray(outlier_channels)
        for g in range(ch.shape[0]):
            idx = torch.as_tensor(ch[g], device=device, dtype=torch.long)
            x[..., g, idx] = x[..., g, idx] * float(outlier_scale)
    if dtype is not None:
        x = x.to(dtype)
    return x
