"""Host check of the int8 kernels' division-free quantization.

The kernels (lema_q8.hip, quant_row/quant) form the code of x / s from
y = x * (1/s) and fall back to the IEEE division only within 2^-15 of a
half-integer or for subnormal scales.  Their comment argues that this gives
round-half-even(RN(x / s)) exactly; this test replays those steps in numpy
float32 (every operation an IEEE binary32 one) against the IEEE quotient on
values built to sit on and next to half-integers, across the exponent range
of scales.
"""
from __future__ import annotations

import numpy as np

F = np.float32


def kernel_codes(x: np.ndarray, s: np.float32) -> np.ndarray:
    """The kernels' steps for one row with a normal scale s."""
    with np.errstate(all="ignore"):
        r = F(1.0) / s
        y = x * r
        k = np.rint(y)
        off_half = np.abs(np.abs(y - k) - F(0.5))
        slow = off_half < F(2.0 ** -15)
        k = np.where(slow, np.rint(x / s), k)
    return np.clip(k, -127, 127).astype(np.int32), slow


def ieee_codes(x: np.ndarray, s: np.float32) -> np.ndarray:
    with np.errstate(all="ignore"):
        return np.clip(np.rint(x / s), -127, 127).astype(np.int32)


def near_half_integers(s: np.float32, rng) -> np.ndarray:
    """Values whose quotient by s is a half-integer or a few ulps off one."""
    k = rng.integers(-127, 127, 600).astype(np.float64) + 0.5
    out = []
    for j in range(-6, 7):
        out.append((k + j * 2.0 ** -19) * float(s))
    x = np.concatenate(out).astype(np.float32)
    # also the float32 neighbours of each value
    up = np.nextafter(x, np.float32(np.inf))
    dn = np.nextafter(x, np.float32(-np.inf))
    return np.concatenate([x, up, dn])


def test_shortcut_equals_ieee_division_near_ties():
    rng = np.random.default_rng(5)
    slow_total = 0
    for e in list(range(-125, 120, 7)) + [-126, 126]:
        for a_mant in (1.0, 1.37, 1.9999, 1.5):
            a = F(a_mant * 2.0 ** e)
            s = F(a / F(127.0))
            if not (np.isfinite(s) and s >= F(2.0 ** -126)):
                continue
            x = near_half_integers(s, rng)
            x = x[np.abs(x) <= a]
            got, slow = kernel_codes(x, s)
            assert np.array_equal(got, ieee_codes(x, s)), (e, a_mant)
            slow_total += int(slow.sum())
    assert slow_total > 0          # the fallback really is exercised


def test_shortcut_equals_ieee_division_random_rows():
    """Ordinary rows: codes agree everywhere and the fallback is rare."""
    rng = np.random.default_rng(6)
    n_slow = n_all = 0
    for _ in range(200):
        x = (rng.standard_normal(4096) * np.exp(rng.uniform(-40, 40))).astype(np.float32)
        a = np.abs(x).max()
        s = F(a / F(127.0))
        if not (np.isfinite(s) and s >= F(2.0 ** -126)):
            continue
        got, slow = kernel_codes(x, s)
        assert np.array_equal(got, ieee_codes(x, s))
        n_slow += int(slow.sum())
        n_all += x.size
    assert n_slow / n_all < 1e-3
