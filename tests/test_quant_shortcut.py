"""Host check of the int8 kernels' division-free quantization.

The kernels (lema_q8.hip, quant_row and quant4_fast) form the code of x / s
from y = x * r, where r is one Newton step from the hardware reciprocal r0
of s: r = fma(fma(-s, r0, 1), r0, r0).  They fall back to the IEEE division
when some |y - round(y)| exceeds 1/2 - 2^-15, and for subnormal scales.
Their comment argues that |r*s - 1| <= 2^-23 for any r0 within 2^-21 of 1/s
and that the codes are then round-half-even(RN(x / s)) exactly; this test
replays those steps (numpy float32 for the element operations, exact
rationals for the fused multiply-adds) with r0 set anywhere from 8 ulps below
to 8 ulps above the correctly rounded 1/s, against the IEEE quotient, on
values built to sit on and next to half-integers, across the exponent range
of scales.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

F = np.float32


def round32(q: Fraction) -> np.float32:
    """The float32 nearest to the rational q, ties to even (normal range)."""
    c = F(float(q))
    best = None
    for cand in (np.nextafter(c, F(-np.inf)), c, np.nextafter(c, F(np.inf))):
        d = abs(Fraction(float(cand)) - q)
        key = (d, int(cand.view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def fma32(a, b, c) -> np.float32:
    return round32(Fraction(float(a)) * Fraction(float(b)) + Fraction(float(c)))


def newton_reciprocal(s: np.float32, r0: np.float32) -> np.float32:
    e = fma32(-s, r0, F(1.0))
    return fma32(e, r0, r0)


def kernel_codes(x: np.ndarray, s: np.float32, r: np.float32):
    """The kernels' steps for one row with a normal scale s."""
    with np.errstate(all="ignore"):
        y = x * r
        k = (y + F(12582912.0)) - F(12582912.0)      # 1.5 * 2^23: nearest, ties to even
        slow = np.abs(y - k) > F(0.5) - F(2.0 ** -15)
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


def step_ulps(v: np.float32, k: int) -> np.float32:
    for _ in range(abs(k)):
        v = np.nextafter(v, F(np.inf) if k > 0 else F(-np.inf))
    return v


def test_newton_reciprocal_bound():
    """|r*s - 1| <= 2^-23 from any r0 within 8 ulps of 1/s."""
    rng = np.random.default_rng(4)
    for e in list(range(-126, 122, 5)) + [121]:
        for mant in (1.0, 1.0000001, 1.37, 1.5, 1.9999999) + tuple(rng.uniform(1, 2, 3)):
            s = F(mant * 2.0 ** e)
            r_exact = F(1.0) / s
            for k in range(-8, 9):
                r = newton_reciprocal(s, step_ulps(r_exact, k))
                err = abs(Fraction(float(r)) * Fraction(float(s)) - 1)
                assert err <= Fraction(1, 2 ** 23), (e, mant, k, float(err))


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
            for k in (-8, -1, 0, 1, 8):
                r = newton_reciprocal(s, step_ulps(F(1.0) / s, k))
                got, slow = kernel_codes(x, s, r)
                assert np.array_equal(got, ieee_codes(x, s)), (e, a_mant, k)
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
        r = newton_reciprocal(s, step_ulps(F(1.0) / s, int(rng.integers(-2, 3))))
        got, slow = kernel_codes(x, s, r)
        assert np.array_equal(got, ieee_codes(x, s))
        n_slow += int(slow.sum())
        n_all += x.size
    assert n_slow / n_all < 1e-3
