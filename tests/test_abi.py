"""Host-side checks of the C ABI (no GPU work): the library loads and exports
every function include/dq.h declares, error codes for invalid arguments are
returned before any device call, and the host table derivation equals the
oracle's table for a grid of parameters."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def dq(built_library):
    from decode_attention_dq_amd import dq as mod
    return mod


def declared_functions():
    text = open(os.path.join(ROOT, "include", "dq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\**\s*(dq_\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(dq):
    names = declared_functions()
    assert len(names) >= 10
    lib = ctypes.CDLL(dq.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(dq.EXPORTED)


def test_strerror(dq):
    assert dq.dq_strerror(0) == "ok"
    assert "workspace" in dq.dq_strerror(dq.DQ_ERR_WORKSPACE)
    assert dq.dq_strerror(99) == "unknown error"


@pytest.mark.parametrize("M", [2, 4, 5, 6, 8, 9])
@pytest.mark.parametrize("C", [24, 32, 37, 64])
@pytest.mark.parametrize("p", [9, 10])
def test_host_tables_equal_oracle(dq, M, C, p):
    for step in (0.5, 0.9, 1.3):
        t = oracle.make_table(M, C, step, 1.4, p)
        try:
            d = dq.dq_table_describe(dq.make_params(M, C, step, 0.0, p))
        except dq.DQError as e:
            assert e.code == dq.DQ_ERR_INFEASIBLE and not t.feasible
            continue
        assert t.feasible
        assert d["freq"] == t.freq.tolist()
        assert d["cum"] == t.cum.tolist()
        assert d["cost"] == t.cost.tolist()
        assert d["inner"] == t.inner.tolist()
        assert d["recon"] == t.recon.tolist()
        assert d["bounds"] == t.bounds.tolist()
        assert d["mass"] == t.mass.tolist()
        assert d["budget_fx"] == t.budget_fx


def test_default_steps_and_unsupported(dq):
    for (M, C) in [(8, 37), (6, 37), (8, 32), (6, 32), (8, 41), (6, 27)]:
        assert dq.dq_table_describe(dq.make_params(M, C))["step"] == oracle.default_step(M, C)
    for bad in (dq.make_params(10, 37, 1.0), dq.make_params(1, 37, 1.0), dq.make_params(8, 200, 1.0),
                dq.make_params(8, 37, 1.0, 0.0, 8), dq.make_params(8, 37, 1.0, 0.0, 11)):
        with pytest.raises(dq.DQError) as ei:
            dq.dq_table_describe(bad)
        assert ei.value.code == dq.DQ_ERR_UNSUPPORTED
    with pytest.raises(dq.DQError) as ei:
        dq.dq_table_describe(dq.make_params(7, 37))          # no default step for (7, 37)
    assert ei.value.code == dq.DQ_ERR_INVALID_ARG


def test_invalid_arguments_rejected_on_host(dq):
    lib = dq._lib
    fake = ctypes.c_void_p(16)
    # null tables / pointers, bad dtype, page size not a multiple of 16
    assert lib.dq_encode_kv(None, fake, fake, 0, 4, 8, 16, fake, fake, fake, fake, fake, None, None, None) == \
        dq.DQ_ERR_INVALID_ARG
    assert lib.dq_decode_attention(None, fake, 1, fake, fake, fake, fake, fake, fake, 1, 4, 1, 1, 16, 16, 0.0, 0,
                                   fake, fake, 1 << 20, None, None) == dq.DQ_ERR_INVALID_ARG
    assert lib.dq_decode_attention_window(None, fake, 1, fake, fake, fake, fake, fake, fake, 1, 4, 1, 1, 16, 16, 0.0,
                                          0, None, None, None, 0, fake, fake, 1 << 20, None, None) == \
        dq.DQ_ERR_INVALID_ARG
    assert lib.dq_decode_symbols(None, 0, fake, 1, fake, None, None) == dq.DQ_ERR_INVALID_ARG
    # per-token block write: null tables, missing means, non-power-of-two pages
    assert lib.dq_encode_tokens_blocks(None, fake, fake, 0, 1, 64, fake, fake, fake, fake, fake, fake, fake, None,
                                       None, None) == dq.DQ_ERR_INVALID_ARG
    assert lib.dq_encode_tokens_blocks(fake, fake, fake, 0, 1, 64, fake, fake, fake, fake, fake, None, fake, None,
                                       None, None) == dq.DQ_ERR_INVALID_ARG
    assert lib.dq_encode_tokens_blocks(fake, fake, fake, 0, 1, 48, fake, fake, fake, fake, fake, fake, fake, None,
                                       None, None) == dq.DQ_ERR_UNSUPPORTED
    assert lib.dq_selftest_fp64(None, None, -1, None, None, None, None) == dq.DQ_ERR_INVALID_ARG
    assert lib.dq_tables_destroy(None) == dq.DQ_OK


def test_workspace_size(dq):
    assert dq.dq_workspace_size(0, 32, 8, 100) == 0
    # one slot per split plus one for an optional bf16 window
    assert dq.dq_workspace_size(2, 8, 2, 1000, 3) == 2 * 8 * 4 * 132 * 4
    # the automatic split count never splits below one 256-token tile
    assert dq.dq_workspace_size(1, 4, 1, 100) == 1 * 4 * 2 * 132 * 4
    assert dq.dq_workspace_size(128, 32, 8, 8192) >= 128 * 32 * 132 * 4


@pytest.mark.parametrize("B,hkv,ctx,splits", [
    (128, 8, 8192, 6),      # >= 4 work-groups per slot: 1536-token splits
    (64, 8, 16384, 11),
    (4, 8, 65536, 64),      # 2048-token splits would make one round: 1024-token splits, two rounds
    (16, 8, 16384, 16),     # the same at 16 x 16K
    (8, 8, 65536, 32),      # two rounds of 2048-token splits
    (1, 8, 131072, 128),    # fewer: shorter splits up to 1024 work-groups
    (1, 1, 300, 2),         # never below one 256-token tile
])
def test_split_rule(dq, B, hkv, ctx, splits):
    """The automatic split count, read back from the workspace size (one
    partial slot per split plus one for a window)."""
    assert dq.dq_workspace_size(B, 4 * hkv, hkv, ctx) == B * 4 * hkv * (splits + 1) * 132 * 4


@pytest.mark.parametrize("M,C", [(8, 331), (6, 231), (4, 160), (9, 400), (2, 140)])
def test_host_token_tables_equal_oracle(dq, M, C):
    """Per-token tables (1024 symbols per stream, default min-max step) on the
    host equal the oracle's, including the step from the expected maximum."""
    t = oracle.make_token_table(M, C)
    try:
        d = dq.dq_token_table_describe(dq.make_params(M, C))
    except dq.DQError as e:
        assert e.code == dq.DQ_ERR_INFEASIBLE and not t.feasible
        return
    assert t.feasible
    assert d["step"] == pytest.approx(t.step, rel=1e-14)
    assert d["freq"] == t.freq.tolist() and d["cum"] == t.cum.tolist()
    assert d["cost"] == t.cost.tolist() and d["inner"] == t.inner.tolist()
    assert d["budget_fx"] == t.budget_fx


def test_token_tables_unsupported_sizes(dq):
    for bad in (dq.make_params(8, 15), dq.make_params(8, 1025), dq.make_params(10, 331)):
        with pytest.raises(dq.DQError) as ei:
            dq.dq_token_table_describe(bad)
        assert ei.value.code == dq.DQ_ERR_UNSUPPORTED
    # a budget too small for 1024 central symbols is refused
    with pytest.raises(dq.DQError) as ei:
        dq.dq_token_table_describe(dq.make_params(8, 100))
    assert ei.value.code == dq.DQ_ERR_INFEASIBLE
