"""Device fp64 primitives the bit-exact encoder rests on, against numpy:
correctly rounded sqrt and division, and a single round-to-nearest-even
fp64 -> fp16 conversion (numpy's float64 -> float16 cast rounds once)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


def _fp16_midpoints(rng, n):
    h = rng.integers(0, 0x7BFF, n, dtype=np.uint16)          # finite positive halves (and subnormals)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2.0                                       # exact in fp64
    return np.concatenate([mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)])


def test_fp64_primitives(gpu_lib):
    dq = gpu_lib
    rng = np.random.default_rng(7)
    n1 = 200_000
    a = np.concatenate([
        rng.standard_normal(n1) * 10.0 ** rng.uniform(-9, 6, n1),
        np.abs(rng.standard_normal(n1)) * 2.0 ** rng.integers(-40, 40, n1).astype(np.float64),
        _fp16_midpoints(rng, 50_000),
        -_fp16_midpoints(rng, 10_000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26,
                  2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 6.1e-5, 1e-300, 5e-324, 128.0, 8192.0 * 128]),
        rng.uniform(0, 2 ** 30, n1).round() * 2.0 ** -rng.integers(0, 60, n1),   # sums of squares-like values
    ])
    b = np.where(rng.random(a.size) < 0.5, rng.standard_normal(a.size), rng.integers(1, 2000, a.size).astype(float))
    b[b == 0] = 1.0
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).cuda()
    da, db = dev(a), dev(b)
    sq = torch.empty_like(da)
    dv = torch.empty_like(da)
    f16 = torch.empty(a.size, dtype=torch.int16, device="cuda")
    dq.dq_selftest_fp64(da, db, sq, dv, f16)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", over="ignore"):
        exp_sq = np.sqrt(np.where(a >= 0, a, 0.0))     # IEEE: sqrt(-0) = -0
        exp_dv = a / b
        exp_f16 = a.astype(np.float16).view(np.uint16)
    got_sq = sq.cpu().numpy()
    got_dv = dv.cpu().numpy()
    got_f16 = f16.cpu().numpy().view(np.uint16)
    assert np.array_equal(got_sq.view(np.uint64), exp_sq.view(np.uint64)), \
        f"sqrt differs at {np.flatnonzero(got_sq.view(np.uint64) != exp_sq.view(np.uint64))[:5]}"
    assert np.array_equal(got_dv.view(np.uint64), exp_dv.view(np.uint64)), \
        f"division differs at {np.flatnonzero(got_dv.view(np.uint64) != exp_dv.view(np.uint64))[:5]}"
    bad = np.flatnonzero(got_f16 != exp_f16)
    assert bad.size == 0, f"fp16 rounding differs for {a[bad[:5]]}: {got_f16[bad[:5]]} vs {exp_f16[bad[:5]]}"
