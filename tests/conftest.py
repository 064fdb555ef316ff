import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def built_library():
    """Path of libdq.so, building it in place first if it is missing."""
    path = os.path.join(ROOT, "decode_attention_dq_amd", "libdq.so")
    if not os.path.exists(path):
        from decode_attention_dq_amd import build_lib
        build_lib.build()
    return path


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding, on cuda:0 (gpu tests only)."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test collected on a machine without a GPU")
    from decode_attention_dq_amd import dq
    return dq
