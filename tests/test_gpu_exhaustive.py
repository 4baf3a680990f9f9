"""Exhaustive GPU checks of the arithmetic primitives the kernels are built
from, compiled exactly as inside them (lema_probe_fp32,
lema_probe_q8_reciprocal of include/lema_measure.h).

The method's reading fixes IEEE binary32 arithmetic with correctly rounded
square roots and bf16 rounding to nearest even (include/lema.h).  Division
has two operands and cannot be enumerated; the square root and the bf16
conversion are checked on all 2^32 fp32 bit patterns, against numpy's
float32 sqrt (an IEEE operation on the host) and the oracle's rne16 (itself
pinned exhaustively against torch).  The int8 kernels' division-free
quantization is exact when their reciprocal of a row scale s satisfies
|r*s - 1| <= 2^-23; that bound is checked for every scale a row can have.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity import to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"
CHUNK = 1 << 28


@pytest.fixture(scope="module")
def L():
    import optimizer_step_lema_amd as lema
    lema.load()
    return lema


def test_sqrt_and_bf16_of_every_fp32_pattern(L):
    ones = torch.ones(CHUNK, device=DEV)
    for start in range(0, 1 << 32, CHUNK):
        bits = np.arange(start, start + CHUNK, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        _, root, half = L.probe_fp32(torch.from_numpy(x).to(DEV), ones)
        got = to_np(root)
        with np.errstate(invalid="ignore"):
            ref = np.sqrt(x)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), f"sqrt NaN set, chunk {start:#x}"
        bad = np.nonzero(got.view(np.uint32)[~nan] != ref.view(np.uint32)[~nan])[0]
        assert bad.size == 0, f"sqrt of {bits[~nan][bad[:4]]}: {got[~nan][bad[:4]]}"
        h = to_np(half)
        r16 = oracle.rne16(x)
        xnan = np.isnan(x)
        assert np.array_equal((h & 0x7FFF) > 0x7F80, xnan), f"bf16 NaN set, chunk {start:#x}"
        bad = np.nonzero(h[~xnan] != r16[~xnan])[0]
        assert bad.size == 0, f"bf16 of {bits[~xnan][bad[:4]]}: {h[~xnan][bad[:4]]}"
        del root, half


def test_q8_reciprocal_bound_over_every_row_scale(L):
    """Every scale a row can get, s = RN(absmax / 127) from a finite absmax of
    at least 127 * 2^-126 (smaller scales are subnormal and take the IEEE
    division): from 2^-126 to RN(FLT_MAX / 127)."""
    lo = 0x00800000
    hi = int(np.array(np.float32(np.finfo(np.float32).max) / np.float32(127)).view(np.uint32))
    worst = 0.0
    for start in range(lo, hi + 1, CHUNK // 2):
        stop = min(start + CHUNK // 2, hi + 1)
        s = np.arange(start, stop, dtype=np.uint64).astype(np.uint32).view(np.float32)
        r = to_np(L.probe_q8_reciprocal(torch.from_numpy(s).to(DEV)))
        assert np.all(np.isfinite(r)) and np.all(r > 0)
        err = np.abs(r.astype(np.float64) * s.astype(np.float64) - 1.0)   # exact product
        worst = max(worst, float(err.max()))
        assert err.max() <= 2.0 ** -23, f"chunk {start:#x}: {err.max()}"
    print(f"largest |r*s - 1| over {hi - lo + 1} scales: {worst:.3e} "
          f"({worst / 2.0 ** -24:.3f} x 2^-24)")
