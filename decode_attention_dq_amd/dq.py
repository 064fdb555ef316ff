"""Python binding of libdq (the C ABI in include/dq.h).

Argument marshalling only: every function here checks shapes and dtypes,
passes raw device pointers and the current HIP stream to the library, and
raises DQError on a non-zero status. All compute runs in the HIP kernels of
libdq.so; importing this module fails loudly when the library is missing.
Function names are those of the C ABI.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# DQ_LIBRARY may name another build of the same library (for example a debug build)
LIB_PATH = os.environ.get("DQ_LIBRARY") or os.path.join(_HERE, "libdq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libdq.so not found at {LIB_PATH}; build it with "
                      f"`python -m decode_attention_dq_amd.build_lib`")
_lib = ctypes.CDLL(LIB_PATH)

DQ_OK, DQ_ERR_INVALID_ARG, DQ_ERR_UNSUPPORTED, DQ_ERR_INFEASIBLE, DQ_ERR_WORKSPACE, DQ_ERR_HIP = range(6)
DQ_DTYPE_F32, DQ_DTYPE_BF16 = 0, 1
DQ_KEYS, DQ_VALUES = 0, 1
DQ_DEVERR_DECODE, DQ_DEVERR_ENCODE, DQ_DEVERR_MEAN_SLOT, DQ_DEVERR_CONTEXT = 1, 2, 4, 8
HEAD_DIM = 128


class DQError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = _lib.dq_strerror(code).decode()
        if code == DQ_ERR_HIP:
            msg += ": " + _lib.dq_last_hip_error().decode()
        super().__init__(f"{where}: {msg} (code {code})")
        self.code = code


class dq_table_params(ctypes.Structure):
    _fields_ = [("levels", ctypes.c_int), ("container", ctypes.c_int), ("step", ctypes.c_double),
                ("alpha", ctypes.c_double), ("prob_bits", ctypes.c_int)]


class dq_table_info(ctypes.Structure):
    _fields_ = [("levels", ctypes.c_int), ("container", ctypes.c_int), ("prob_bits", ctypes.c_int),
                ("feasible", ctypes.c_int), ("step", ctypes.c_double), ("alpha", ctypes.c_double),
                ("recon", ctypes.c_double * 16), ("bounds", ctypes.c_double * 16),
                ("mass", ctypes.c_double * 16), ("freq", ctypes.c_uint32 * 16),
                ("cum", ctypes.c_uint32 * 17), ("cost", ctypes.c_int64 * 16),
                ("inner", ctypes.c_int32 * 16), ("budget_fx", ctypes.c_int64)]

    def as_dict(self) -> dict:
        M = self.levels
        return {
            "levels": M, "container": self.container, "prob_bits": self.prob_bits,
            "feasible": bool(self.feasible), "step": self.step, "alpha": self.alpha,
            "recon": list(self.recon[:M]), "bounds": list(self.bounds[:M - 1]),
            "mass": list(self.mass[:M]), "freq": list(self.freq[:M]), "cum": list(self.cum[:M + 1]),
            "cost": list(self.cost[:M]), "inner": list(self.inner[:M]), "budget_fx": self.budget_fx,
        }


_p = ctypes.c_void_p
_i = ctypes.c_int


class dq_attention_extras(ctypes.Structure):
    _fields_ = [("window_k", ctypes.c_void_p), ("window_v", ctypes.c_void_p), ("window_lens", ctypes.c_void_p),
                ("window_cap", ctypes.c_int), ("k_mean", ctypes.c_void_p), ("k_mean_scale", ctypes.c_void_p)]
_sig = {
    "dq_table_describe": (_i, [ctypes.POINTER(dq_table_params), ctypes.POINTER(dq_table_info)]),
    "dq_tables_init": (_i, [ctypes.POINTER(_p), ctypes.POINTER(dq_table_params),
                            ctypes.POINTER(dq_table_params)]),
    "dq_tables_destroy": (_i, [_p]),
    "dq_tables_info": (_i, [_p, _i, ctypes.POINTER(dq_table_info)]),
    "dq_encode_kv": (_i, [_p, _p, _p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p]),
    "dq_encode_kv_blocks": (_i, [_p, _p, _p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "dq_workspace_size": (ctypes.c_size_t, [_i, _i, _i, _i, _i]),
    "dq_decode_attention": (_i, [_p, _p, _i, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                 ctypes.c_float, _i, _p, _p, ctypes.c_size_t, _p, _p]),
    "dq_decode_attention_noalloc": (_i, [_p, _p, _i, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                         ctypes.c_float, _i, _p, _p, _p]),
    "dq_decode_attention_window": (_i, [_p, _p, _i, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                        ctypes.c_float, _i, _p, _p, _p, _i, _p, _p, ctypes.c_size_t, _p, _p]),
    "dq_decode_attention_ext": (_i, [_p, _p, _i, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                     ctypes.c_float, _i, ctypes.POINTER(dq_attention_extras), _p, _p,
                                     ctypes.c_size_t, _p, _p]),
    "dq_bf16_decode_attention": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, ctypes.c_float, _i, _p, _p,
                                      ctypes.c_size_t, _p]),
    "dq_decode_symbols": (_i, [_p, _i, _p, _i, _p, _p, _p]),
    "dq_selftest_fp64": (_i, [_p, _p, _i, _p, _p, _p, _p]),
    "dq_token_tables_init": (_i, [ctypes.POINTER(_p), ctypes.POINTER(dq_table_params),
                                  ctypes.POINTER(dq_table_params)]),
    "dq_token_table_describe": (_i, [ctypes.POINTER(dq_table_params), ctypes.POINTER(dq_table_info)]),
    "dq_encode_tokens": (_i, [_p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p]),
    "dq_encode_tokens_blocks": (_i, [_p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "dq_token_workspace_size": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "dq_token_decode_attention": (_i, [_p, _p, _i, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, ctypes.c_float, _i,
                                       _p, _p, ctypes.c_size_t, _p, _p]),
    "dq_token_decode_symbols": (_i, [_p, _i, _p, _i, _p, _p, _p]),
    "dq_token_decode_attention_ext": (_i, [_p, _p, _i, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, ctypes.c_float,
                                           _i, ctypes.POINTER(dq_attention_extras), _p, _p, ctypes.c_size_t, _p, _p]),
    "dq_strerror": (ctypes.c_char_p, [_i]),
    "dq_last_hip_error": (ctypes.c_char_p, []),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_sig)


def _check(code: int, where: str) -> None:
    if code != DQ_OK:
        raise DQError(code, where)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _need(t, name, dtype=None, shape=None, device=True):
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def make_params(levels: int, container: int, step: float = 0.0, alpha: float = 0.0,
                prob_bits: int = 0) -> dq_table_params:
    return dq_table_params(int(levels), int(container), float(step), float(alpha), int(prob_bits))


def dq_strerror(code: int) -> str:
    return _lib.dq_strerror(int(code)).decode()


def dq_table_describe(params: dq_table_params) -> dict:
    """Host-side table derivation (no device work)."""
    info = dq_table_info()
    _check(_lib.dq_table_describe(ctypes.byref(params), ctypes.byref(info)), "dq_table_describe")
    return info.as_dict()


class Tables:
    """Owns a dq_tables handle (keys and values) on the current device;
    ``token``: tables of the per-token format."""

    def __init__(self, keys: dq_table_params, values: dq_table_params, token: bool = False):
        h = _p()
        init = _lib.dq_token_tables_init if token else _lib.dq_tables_init
        _check(init(ctypes.byref(h), ctypes.byref(keys), ctypes.byref(values)),
               "dq_token_tables_init" if token else "dq_tables_init")
        self.handle = h
        self.token = token

    def info(self, which: int) -> dict:
        info = dq_table_info()
        _check(_lib.dq_tables_info(self.handle, int(which), ctypes.byref(info)), "dq_tables_info")
        return info.as_dict()

    def destroy(self) -> None:
        if self.handle:
            _check(_lib.dq_tables_destroy(self.handle), "dq_tables_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def dq_tables_init(keys: dq_table_params, values: dq_table_params) -> Tables:
    return Tables(keys, values)


def dq_tables_destroy(tables: Tables) -> None:
    tables.destroy()


def dq_encode_kv(tables: Tables, k, v, slot_mapping, k_cache, v_cache, k_norm, v_norm, page_size: int,
                 drift_stats=None, err_word=None, stream=None) -> None:
    """k, v: [num_tokens][Hkv][128] float32 or bfloat16 device tensors."""
    import torch
    if k.dtype != v.dtype or k.shape != v.shape or k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError("k and v must both be [num_tokens][Hkv][128] of one dtype")
    dtype = {torch.float32: DQ_DTYPE_F32, torch.bfloat16: DQ_DTYPE_BF16}.get(k.dtype)
    if dtype is None:
        raise ValueError("k/v dtype must be float32 or bfloat16")
    n, hkv = int(k.shape[0]), int(k.shape[1])
    _need(k, "k"); _need(v, "v")
    _need(slot_mapping, "slot_mapping", torch.int32, (n,))
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, torch.uint8)
    for t, nm in ((k_norm, "k_norm"), (v_norm, "v_norm")):
        _need(t, nm)
        if t.element_size() != 2:
            raise ValueError(f"{nm} must hold 16-bit elements")
    if drift_stats is not None:
        _need(drift_stats, "drift_stats", shape=(n, hkv, 2))
        if drift_stats.element_size() != 2:
            raise ValueError("drift_stats must hold 16-bit elements")
    if err_word is not None:
        _need(err_word, "err_word")
    _check(_lib.dq_encode_kv(tables.handle, _ptr(k), _ptr(v), dtype, n, hkv, int(page_size),
                             _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), _ptr(k_norm), _ptr(v_norm),
                             _ptr(drift_stats), _ptr(err_word), _stream(stream)), "dq_encode_kv")


MEAN_BLOCK = 128


def mean_rows_per_page(page_size: int) -> int:
    """Key-mean rows each page owns: one per 128-token block it holds, or one."""
    return page_size // MEAN_BLOCK if page_size >= MEAN_BLOCK else 1


def dq_encode_kv_blocks(tables: Tables, k, v, slot_mapping, k_cache, v_cache, k_norm, v_norm, k_mean, k_mean_scale,
                        page_size: int, drift_stats=None, err_word=None, stream=None) -> None:
    """Cache write with key channel-mean removal: k, v [128 * blocks][Hkv][128]
    (block j = rows 128j .. 128j+127), k_mean int8 [pages][Hkv][R][128],
    k_mean_scale 16-bit [pages][Hkv][R] with R = mean_rows_per_page(page_size)."""
    import torch
    if k.dtype != v.dtype or k.shape != v.shape or k.dim() != 3 or k.shape[2] != HEAD_DIM:
        raise ValueError("k and v must both be [num_tokens][Hkv][128] of one dtype")
    if k.shape[0] % MEAN_BLOCK:
        raise ValueError("the token count must be a multiple of 128")
    dtype = {torch.float32: DQ_DTYPE_F32, torch.bfloat16: DQ_DTYPE_BF16}.get(k.dtype)
    if dtype is None:
        raise ValueError("k/v dtype must be float32 or bfloat16")
    n, hkv = int(k.shape[0]), int(k.shape[1])
    _need(k, "k"); _need(v, "v")
    _need(slot_mapping, "slot_mapping", torch.int32, (n,))
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, torch.uint8)
    for t, nm in ((k_norm, "k_norm"), (v_norm, "v_norm"), (k_mean_scale, "k_mean_scale")):
        _need(t, nm)
        if t.element_size() != 2:
            raise ValueError(f"{nm} must hold 16-bit elements")
    _need(k_mean, "k_mean", torch.int8)
    if drift_stats is not None:
        _need(drift_stats, "drift_stats", shape=(n, hkv, 2))
    if err_word is not None:
        _need(err_word, "err_word")
    _check(_lib.dq_encode_kv_blocks(tables.handle, _ptr(k), _ptr(v), dtype, n // MEAN_BLOCK, hkv, int(page_size),
                                    _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), _ptr(k_norm), _ptr(v_norm),
                                    _ptr(k_mean), _ptr(k_mean_scale), _ptr(drift_stats), _ptr(err_word),
                                    _stream(stream)), "dq_encode_kv_blocks")


def dq_decode_attention_ext(tables: Tables, q, k_cache, v_cache, k_norm, v_norm, block_table, context_lens,
                            num_kv_heads: int, page_size: int, max_context: int, out, workspace,
                            window_k=None, window_v=None, window_lens=None, k_mean=None, k_mean_scale=None,
                            softmax_scale: float = 0.0, num_splits: int = 0, err_word=None, stream=None) -> None:
    """dq_decode_attention with the optional bf16 window and key block means."""
    import torch
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [B][Hq][128]")
    qd = {torch.float32: DQ_DTYPE_F32, torch.bfloat16: DQ_DTYPE_BF16}.get(q.dtype)
    if qd is None:
        raise ValueError("q dtype must be float32 or bfloat16")
    B, hq = int(q.shape[0]), int(q.shape[1])
    _need(q, "q")
    _need(out, "out", torch.float32, (B, hq, HEAD_DIM))
    _need(block_table, "block_table", torch.int32)
    _need(context_lens, "context_lens", torch.int32, (B,))
    _need(workspace, "workspace")
    ex = dq_attention_extras()
    if window_k is not None:
        for t, nm in ((window_k, "window_k"), (window_v, "window_v")):
            _need(t, nm, torch.bfloat16)
            if t.dim() != 4 or t.shape[0] != B or t.shape[1] != num_kv_heads or t.shape[3] != HEAD_DIM:
                raise ValueError(f"{nm} must be [B][Hkv][cap][128]")
        _need(window_lens, "window_lens", torch.int32, (B,))
        ex.window_k, ex.window_v, ex.window_lens = _ptr(window_k), _ptr(window_v), _ptr(window_lens)
        ex.window_cap = int(window_k.shape[2])
    if k_mean is not None:
        _need(k_mean, "k_mean", torch.int8)
        _need(k_mean_scale, "k_mean_scale")
        ex.k_mean, ex.k_mean_scale = _ptr(k_mean), _ptr(k_mean_scale)
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.dq_decode_attention_ext(tables.handle, _ptr(q), qd, _ptr(k_cache), _ptr(v_cache), _ptr(k_norm),
                                        _ptr(v_norm), _ptr(block_table), _ptr(context_lens), B, hq,
                                        int(num_kv_heads), int(block_table.shape[1]), int(page_size),
                                        int(max_context), float(softmax_scale), int(num_splits),
                                        ctypes.byref(ex), _ptr(out), _ptr(workspace), nbytes, _ptr(err_word),
                                        _stream(stream)), "dq_decode_attention_ext")


DQ_NOALLOC_SCRATCH = 32 << 20


def dq_decode_attention_noalloc(tables: Tables, q, k_cache, v_cache, k_norm, v_norm, block_table, context_lens,
                                num_kv_heads: int, page_size: int, max_context: int, out, softmax_scale: float = 0.0,
                                num_splits: int = 0, err_word=None, stream=None) -> None:
    """dq_decode_attention without a workspace argument: the library's fixed
    per-device scratch holds the split partials (calls overlapping on one
    device race)."""
    import torch
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [B][Hq][128]")
    qd = {torch.float32: DQ_DTYPE_F32, torch.bfloat16: DQ_DTYPE_BF16}.get(q.dtype)
    if qd is None:
        raise ValueError("q dtype must be float32 or bfloat16")
    B, hq = int(q.shape[0]), int(q.shape[1])
    _need(q, "q")
    _need(out, "out", torch.float32, (B, hq, HEAD_DIM))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages_per_seq]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    _need(k_cache, "k_cache", torch.uint8); _need(v_cache, "v_cache", torch.uint8)
    _need(k_norm, "k_norm"); _need(v_norm, "v_norm")
    if err_word is not None:
        _need(err_word, "err_word")
    _check(_lib.dq_decode_attention_noalloc(tables.handle, _ptr(q), qd, _ptr(k_cache), _ptr(v_cache),
                                            _ptr(k_norm), _ptr(v_norm), _ptr(block_table), _ptr(context_lens), B,
                                            hq, int(num_kv_heads), int(block_table.shape[1]), int(page_size),
                                            int(max_context), float(softmax_scale), int(num_splits), _ptr(out),
                                            _ptr(err_word), _stream(stream)), "dq_decode_attention_noalloc")


def dq_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, max_context: int,
                      num_splits: int = 0) -> int:
    return int(_lib.dq_workspace_size(int(batch), int(num_q_heads), int(num_kv_heads), int(max_context),
                                      int(num_splits)))


def dq_decode_attention(tables: Tables, q, k_cache, v_cache, k_norm, v_norm, block_table, context_lens,
                        num_kv_heads: int, page_size: int, max_context: int, out, workspace,
                        softmax_scale: float = 0.0, num_splits: int = 0, err_word=None, stream=None) -> None:
    """q: [B][Hq][128] float32 or bfloat16; out: [B][Hq][128] float32."""
    import torch
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [B][Hq][128]")
    qd = {torch.float32: DQ_DTYPE_F32, torch.bfloat16: DQ_DTYPE_BF16}.get(q.dtype)
    if qd is None:
        raise ValueError("q dtype must be float32 or bfloat16")
    B, hq = int(q.shape[0]), int(q.shape[1])
    _need(q, "q")
    _need(out, "out", torch.float32, (B, hq, HEAD_DIM))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages_per_seq]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    _need(k_cache, "k_cache", torch.uint8); _need(v_cache, "v_cache", torch.uint8)
    _need(k_norm, "k_norm"); _need(v_norm, "v_norm")
    _need(workspace, "workspace")
    if err_word is not None:
        _need(err_word, "err_word")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.dq_decode_attention(tables.handle, _ptr(q), qd, _ptr(k_cache), _ptr(v_cache), _ptr(k_norm),
                                    _ptr(v_norm), _ptr(block_table), _ptr(context_lens), B, hq,
                                    int(num_kv_heads), int(block_table.shape[1]), int(page_size),
                                    int(max_context), float(softmax_scale), int(num_splits), _ptr(out),
                                    _ptr(workspace), nbytes, _ptr(err_word), _stream(stream)),
           "dq_decode_attention")


def dq_bf16_decode_attention(q, k_cache, v_cache, block_table, context_lens, num_kv_heads: int, page_size: int,
                             max_context: int, out, workspace, softmax_scale: float = 0.0, num_splits: int = 0,
                             stream=None) -> None:
    """Uncompressed reference: q [B][Hq][128] bf16, k_cache / v_cache
    [pages][Hkv][page_size][128] bf16, out [B][Hq][128] float32."""
    import torch
    if q.dim() != 3 or q.shape[2] != HEAD_DIM or q.dtype != torch.bfloat16:
        raise ValueError("q must be bfloat16 [B][Hq][128]")
    B, hq = int(q.shape[0]), int(q.shape[1])
    _need(q, "q")
    _need(out, "out", torch.float32, (B, hq, HEAD_DIM))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages_per_seq]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, torch.bfloat16)
        if t.dim() != 4 or t.shape[1] != num_kv_heads or t.shape[2] != page_size or t.shape[3] != HEAD_DIM:
            raise ValueError(f"{nm} must be [pages][Hkv][page_size][128]")
    _need(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.dq_bf16_decode_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                         _ptr(context_lens), B, hq, int(num_kv_heads), int(block_table.shape[1]),
                                         int(page_size), int(max_context), float(softmax_scale), int(num_splits),
                                         _ptr(out), _ptr(workspace), nbytes, _stream(stream)),
           "dq_bf16_decode_attention")


def dq_decode_attention_window(tables: Tables, q, k_cache, v_cache, k_norm, v_norm, block_table, context_lens,
                               window_k, window_v, window_lens, num_kv_heads: int, page_size: int,
                               max_context: int, out, workspace, softmax_scale: float = 0.0, num_splits: int = 0,
                               err_word=None, stream=None) -> None:
    """As dq_decode_attention, plus a bf16 window of recent tokens:
    window_k / window_v [B][Hkv][cap][128] bfloat16, window_lens [B] int32."""
    import torch
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [B][Hq][128]")
    qd = {torch.float32: DQ_DTYPE_F32, torch.bfloat16: DQ_DTYPE_BF16}.get(q.dtype)
    if qd is None:
        raise ValueError("q dtype must be float32 or bfloat16")
    B, hq = int(q.shape[0]), int(q.shape[1])
    _need(q, "q")
    _need(out, "out", torch.float32, (B, hq, HEAD_DIM))
    _need(block_table, "block_table", torch.int32)
    _need(context_lens, "context_lens", torch.int32, (B,))
    _need(window_lens, "window_lens", torch.int32, (B,))
    for t, nm in ((window_k, "window_k"), (window_v, "window_v")):
        _need(t, nm, torch.bfloat16)
        if t.dim() != 4 or t.shape[0] != B or t.shape[1] != num_kv_heads or t.shape[3] != HEAD_DIM:
            raise ValueError(f"{nm} must be [B][Hkv][cap][128]")
    cap = int(window_k.shape[2])
    _need(workspace, "workspace")
    nbytes = workspace.numel() * workspace.element_size()
    _check(_lib.dq_decode_attention_window(
        tables.handle, _ptr(q), qd, _ptr(k_cache), _ptr(v_cache), _ptr(k_norm), _ptr(v_norm), _ptr(block_table),
        _ptr(context_lens), B, hq, int(num_kv_heads), int(block_table.shape[1]), int(page_size), int(max_context),
        float(softmax_scale), int(num_splits), _ptr(window_k), _ptr(window_v), _ptr(window_lens), cap, _ptr(out),
        _ptr(workspace), nbytes, _ptr(err_word), _stream(stream)), "dq_decode_attention_window")


def dq_decode_symbols(tables: Tables, which: int, containers, symbols_out, err_word=None, stream=None) -> None:
    """containers: uint8 [n][C]; symbols_out: uint8 [n][128]."""
    import torch
    _need(containers, "containers", torch.uint8)
    n = int(containers.shape[0])
    _need(symbols_out, "symbols_out", torch.uint8, (n, HEAD_DIM))
    if err_word is not None:
        _need(err_word, "err_word")
    _check(_lib.dq_decode_symbols(tables.handle, int(which), _ptr(containers), n, _ptr(symbols_out),
                                  _ptr(err_word), _stream(stream)), "dq_decode_symbols")


# ---- per-token format: one 1024-value stream per token over the 8 KV heads

TOKEN_HEADS, TOKEN_VALUES = 8, 1024


def token_cache_shape(pages: int, page_size: int, container: int) -> tuple:
    """Shape of a per-token cache: [pages][ceil(C/4)][page_size][4] bytes."""
    return (int(pages), (int(container) + 3) // 4, int(page_size), 4)


def dq_token_table_describe(params: dq_table_params) -> dict:
    info = dq_table_info()
    _check(_lib.dq_token_table_describe(ctypes.byref(params), ctypes.byref(info)), "dq_token_table_describe")
    return info.as_dict()


def dq_token_tables_init(keys: dq_table_params, values: dq_table_params) -> Tables:
    return Tables(keys, values, token=True)


def dq_encode_tokens(tables: Tables, k, v, slot_mapping, k_cache, v_cache, k_meta, v_meta, page_size: int,
                     drift_stats=None, err_word=None, stream=None) -> None:
    """k, v: [num_tokens][8][128] float32 or bfloat16; caches uint8
    [pages][ceil(C/4)][page_size][4] (containers dword-interleaved across a
    page's slots); metadata 16-bit [pages][page_size][2] (o16, s16);
    drift_stats optional int32/uint32 [num_tokens][2]."""
    import torch
    if k.dtype != v.dtype or k.shape != v.shape or k.dim() != 3 or tuple(k.shape[1:]) != (TOKEN_HEADS, HEAD_DIM):
        raise ValueError("k and v must both be [num_tokens][8][128] of one dtype")
    dtype = {torch.float32: DQ_DTYPE_F32, torch.bfloat16: DQ_DTYPE_BF16}.get(k.dtype)
    if dtype is None:
        raise ValueError("k/v dtype must be float32 or bfloat16")
    n = int(k.shape[0])
    _need(k, "k"); _need(v, "v")
    _need(slot_mapping, "slot_mapping", torch.int32, (n,))
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, torch.uint8)
    for t, nm in ((k_meta, "k_meta"), (v_meta, "v_meta")):
        _need(t, nm)
        if t.element_size() != 2:
            raise ValueError(f"{nm} must hold 16-bit elements")
    if drift_stats is not None:
        _need(drift_stats, "drift_stats", shape=(n, 2))
        if drift_stats.element_size() != 4:
            raise ValueError("drift_stats must hold 32-bit elements")
    if err_word is not None:
        _need(err_word, "err_word")
    _check(_lib.dq_encode_tokens(tables.handle, _ptr(k), _ptr(v), dtype, n, int(page_size), _ptr(slot_mapping),
                                 _ptr(k_cache), _ptr(v_cache), _ptr(k_meta), _ptr(v_meta), _ptr(drift_stats),
                                 _ptr(err_word), _stream(stream)), "dq_encode_tokens")


def dq_encode_tokens_blocks(tables: Tables, k, v, slot_mapping, k_cache, v_cache, k_meta, v_meta, k_mean,
                            k_mean_scale, page_size: int, drift_stats=None, err_word=None, stream=None) -> None:
    """Per-token cache write with key block means: k, v [128 * blocks][8][128]
    (block j = rows 128j .. 128j+127), k_mean int8 [pages][8][R][128],
    k_mean_scale 16-bit [pages][8][R] with R = mean_rows_per_page(page_size);
    the rest as dq_encode_tokens."""
    import torch
    if k.dtype != v.dtype or k.shape != v.shape or k.dim() != 3 or tuple(k.shape[1:]) != (TOKEN_HEADS, HEAD_DIM):
        raise ValueError("k and v must both be [num_tokens][8][128] of one dtype")
    if k.shape[0] % MEAN_BLOCK:
        raise ValueError("the token count must be a multiple of 128")
    dtype = {torch.float32: DQ_DTYPE_F32, torch.bfloat16: DQ_DTYPE_BF16}.get(k.dtype)
    if dtype is None:
        raise ValueError("k/v dtype must be float32 or bfloat16")
    n = int(k.shape[0])
    _need(k, "k"); _need(v, "v")
    _need(slot_mapping, "slot_mapping", torch.int32, (n,))
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, nm, torch.uint8)
    for t, nm in ((k_meta, "k_meta"), (v_meta, "v_meta"), (k_mean_scale, "k_mean_scale")):
        _need(t, nm)
        if t.element_size() != 2:
            raise ValueError(f"{nm} must hold 16-bit elements")
    _need(k_mean, "k_mean", torch.int8)
    if drift_stats is not None:
        _need(drift_stats, "drift_stats", shape=(n, 2))
        if drift_stats.element_size() != 4:
            raise ValueError("drift_stats must hold 32-bit elements")
    if err_word is not None:
        _need(err_word, "err_word")
    _check(_lib.dq_encode_tokens_blocks(tables.handle, _ptr(k), _ptr(v), dtype, n // MEAN_BLOCK, int(page_size),
                                        _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), _ptr(k_meta), _ptr(v_meta),
                                        _ptr(k_mean), _ptr(k_mean_scale), _ptr(drift_stats), _ptr(err_word),
                                        _stream(stream)), "dq_encode_tokens_blocks")


def dq_token_workspace_size(batch: int, num_q_heads: int, max_context: int, num_splits: int = 0) -> int:
    return int(_lib.dq_token_workspace_size(int(batch), int(num_q_heads), int(max_context), int(num_splits)))


def dq_token_decode_attention(tables: Tables, q, k_cache, v_cache, k_meta, v_meta, block_table, context_lens,
                              page_size: int, max_context: int, out, workspace, softmax_scale: float = 0.0,
                              num_splits: int = 0, err_word=None, stream=None, window_k=None, window_v=None,
                              window_lens=None, k_mean=None, k_mean_scale=None) -> None:
    """q: [B][Hq][128] float32 or bfloat16 with Hq = 8 G, G <= 4; out: [B][Hq][128] float32.
    Optional bf16 window of the newest tokens: window_k / window_v [B][8][cap][128],
    window_lens int32 [B]; optional key block means k_mean / k_mean_scale as written by
    dq_encode_tokens_blocks (both through dq_token_decode_attention_ext)."""
    import torch
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [B][Hq][128]")
    q_dtype = {torch.float32: DQ_DTYPE_F32, torch.bfloat16: DQ_DTYPE_BF16}.get(q.dtype)
    if q_dtype is None:
        raise ValueError("q dtype must be float32 or bfloat16")
    B, hq = int(q.shape[0]), int(q.shape[1])
    _need(q, "q")
    _need(out, "out", torch.float32, (B, hq, HEAD_DIM))
    _need(block_table, "block_table", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B][max_pages_per_seq]")
    _need(context_lens, "context_lens", torch.int32, (B,))
    for t, nm in ((k_cache, "k_cache"), (v_cache, "v_cache"), (workspace, "workspace")):
        _need(t, nm, torch.uint8)
    for t, nm in ((k_meta, "k_meta"), (v_meta, "v_meta")):
        _need(t, nm)
        if t.element_size() != 2:
            raise ValueError(f"{nm} must hold 16-bit elements")
    if err_word is not None:
        _need(err_word, "err_word")
    if window_k is None and k_mean is None:
        _check(_lib.dq_token_decode_attention(tables.handle, _ptr(q), q_dtype, _ptr(k_cache), _ptr(v_cache),
                                              _ptr(k_meta), _ptr(v_meta), _ptr(block_table), _ptr(context_lens), B, hq,
                                              int(block_table.shape[1]), int(page_size), int(max_context),
                                              float(softmax_scale), int(num_splits), _ptr(out), _ptr(workspace),
                                              int(workspace.numel()), _ptr(err_word), _stream(stream)),
               "dq_token_decode_attention")
        return
    cap = 0
    if window_k is not None:
        if window_v is None or window_lens is None:
            raise ValueError("a window needs window_k, window_v and window_lens")
        if window_k.dtype != torch.bfloat16 or window_v.dtype != torch.bfloat16 or window_k.shape != window_v.shape:
            raise ValueError("window_k / window_v must be bfloat16 of one shape")
        if (window_k.dim() != 4 or window_k.shape[0] != B or window_k.shape[1] != TOKEN_HEADS
                or window_k.shape[3] != HEAD_DIM):
            raise ValueError("window_k must be [B][8][cap][128]")
        _need(window_k, "window_k"); _need(window_v, "window_v")
        _need(window_lens, "window_lens", torch.int32, (B,))
        cap = int(window_k.shape[2])
    if k_mean is not None:
        if k_mean_scale is None:
            raise ValueError("key means need k_mean and k_mean_scale")
        _need(k_mean, "k_mean", torch.int8)
        _need(k_mean_scale, "k_mean_scale")
        if k_mean_scale.element_size() != 2:
            raise ValueError("k_mean_scale must hold 16-bit elements")
    ex = dq_attention_extras(_ptr(window_k), _ptr(window_v), _ptr(window_lens), cap, _ptr(k_mean),
                             _ptr(k_mean_scale))
    _check(_lib.dq_token_decode_attention_ext(tables.handle, _ptr(q), q_dtype, _ptr(k_cache), _ptr(v_cache),
                                              _ptr(k_meta), _ptr(v_meta), _ptr(block_table), _ptr(context_lens), B, hq,
                                              int(block_table.shape[1]), int(page_size), int(max_context),
                                              float(softmax_scale), int(num_splits), ctypes.byref(ex), _ptr(out),
                                              _ptr(workspace), int(workspace.numel()), _ptr(err_word),
                                              _stream(stream)),
           "dq_token_decode_attention_ext")


def dq_token_decode_symbols(tables: Tables, which: int, containers, symbols_out, err_word=None,
                            stream=None) -> None:
    """containers: uint8 [n][C]; symbols_out: uint8 [n][1024]."""
    import torch
    _need(containers, "containers", torch.uint8)
    n = int(containers.shape[0])
    _need(symbols_out, "symbols_out", torch.uint8, (n, TOKEN_VALUES))
    if err_word is not None:
        _need(err_word, "err_word")
    _check(_lib.dq_token_decode_symbols(tables.handle, int(which), _ptr(containers), n, _ptr(symbols_out),
                                        _ptr(err_word), _stream(stream)), "dq_token_decode_symbols")


def dq_selftest_fp64(a, b, sqrt_out, div_out, f16_out, stream=None) -> None:
    """Device fp64 primitives of the encoder, elementwise over float64 vectors a, b."""
    import torch
    n = int(a.numel())
    for t, nm, dt in ((a, "a", torch.float64), (b, "b", torch.float64), (sqrt_out, "sqrt_out", torch.float64),
                      (div_out, "div_out", torch.float64)):
        _need(t, nm, dt, (n,))
    _need(f16_out, "f16_out", shape=(n,))
    _check(_lib.dq_selftest_fp64(_ptr(a), _ptr(b), n, _ptr(sqrt_out), _ptr(div_out), _ptr(f16_out),
                                 _stream(stream)), "dq_selftest_fp64")
