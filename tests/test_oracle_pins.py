"""Pins of the CPU oracle against facts it does not compute itself.

Each test names the passage it follows and the mistake it would catch.
Pages cited: the LEMA README ("Quick Start": torch.optim.AdamW with lr 1e-4;
"Selective Full Fine-Tuning": per-layer AdamW, fp32 states and fp32
gradient accumulation, fp32 delta checkpoint) and the LLMScale fine-tuning
VRAM page (16 B per trained parameter: bf16 weight/grad, fp32 master/m/v).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import bruteforce
import synth

H = synth.HPARAMS
U32 = 2.0 ** -24          # unit roundoff of binary32


def ulp32(x):
    """Spacing of binary32 numbers at |x| (float64 array)."""
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(x).astype(np.float64)


def consts(step, **over):
    hp = dict(H, **over)
    return oracle.adamw_constants(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                  hp["weight_decay"], step)


def rng_state(n, seed, fresh=False, grad_sigma=1e-3):
    g = np.random.default_rng(seed)
    master = (g.standard_normal(n) * 0.02).astype(np.float32)
    if fresh:
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
    else:
        m = (g.standard_normal(n) * 1e-4).astype(np.float32)
        v = np.square((g.standard_normal(n) * 1e-3).astype(np.float32))
    grad = oracle.rne16((g.standard_normal(n) * grad_sigma).astype(np.float32))
    return master, m, v, grad


# ----------------------------------------------------------------- constants

def _exact_fp32_of(real: Fraction) -> np.float32:
    """Correctly rounded binary32 of an exact rational, by bracketing."""
    f = np.float32(float(real))            # within 1 ulp of the exact value
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f,
                 np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - real)
        if best is None or d < best[0]:
            best = (d, cand)
    return best[1]


@pytest.mark.parametrize("t", [1, 2, 3, 10, 50, 100, 1000, 12345])
def test_constants_against_exact_arithmetic(t):
    """Step size and bias-correction root versus exact real arithmetic.

    The AdamW bias corrections (LEMA README "Quick Start" names
    torch.optim.AdamW) are 1 - beta^t.  The oracle's fp32 constant must be the
    correctly rounded value of the real quantity, or 1 ulp away (double
    rounding).  A wrong exponent (t-1), a missing correction or a swapped beta
    moves these by far more than an ulp.
    """
    c = consts(t)
    b1, b2, lr = Fraction(H["beta1"]), Fraction(H["beta2"]), Fraction(H["lr"])
    step_exact = lr / (1 - b1 ** t)
    ref = _exact_fp32_of(step_exact)
    assert abs(float(c[6]) - float(ref)) <= float(np.spacing(ref))

    bc2 = 1 - b2 ** t
    bits = 100                                  # 1/sqrt(bc2) to within 2^-100
    inv_root = Fraction(math.isqrt((bc2.denominator << (2 * bits)) // bc2.numerator), 1 << bits)
    ref2 = _exact_fp32_of(inv_root)
    assert abs(float(c[7]) - float(ref2)) <= float(np.spacing(ref2))

    assert c[0] == np.float32(0.9) and c[2] == np.float32(0.999)
    assert c[1] == _exact_fp32_of(1 - Fraction(H["beta1"]))
    assert c[3] == _exact_fp32_of(1 - Fraction(H["beta2"]))
    assert c[4] == np.float32(1e-8)
    assert c[5] == _exact_fp32_of(1 - Fraction(H["lr"]) * Fraction(H["weight_decay"]))


def test_constants_two_implementations_agree():
    for t in [1, 2, 7, 10, 50, 100, 999, 2 ** 20 + 3]:
        for hp in [H, dict(H, beta1=0.0, beta2=0.0), dict(H, lr=3e-3, weight_decay=0.1),
                   dict(H, beta1=0.5, beta2=0.25, eps=1e-6)]:
            c = oracle.adamw_constants(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                       hp["weight_decay"], t)
            b = bruteforce.constants(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                     hp["weight_decay"], t)
            got = [b["b1"], b["one_minus_b1"], b["b2"], b["one_minus_b2"], b["eps"],
                   b["decay"], b["step_size"], b["inv_bc2_root"]]
            assert c.view(np.uint32).tolist() == np.array(got, np.float32).view(np.uint32).tolist()


def test_constants_known_values():
    """lr/(1-0.9^t) and 1/sqrt(1-0.999^t) at the workloads' steps."""
    expect = {1: (1.0e-3, 31.622776), 10: (1.53534e-4, 10.022516),
              50: (1.00518e-4, 4.5270486), 100: (1.00003e-4, 3.240885)}
    for t, (s, r) in expect.items():
        c = consts(t)
        assert math.isclose(float(c[6]), s, rel_tol=1e-5)
        assert math.isclose(float(c[7]), r, rel_tol=1e-6)
        assert math.isclose(float(c[6]), H["lr"] / (1 - H["beta1"] ** t), rel_tol=1e-7)


# ------------------------------------------------------------------- bf16

def test_rne16_exhaustive_against_torch():
    """Every one of the 2^32 fp32 patterns against torch's bf16 conversion.

    torch.Tensor.to(torch.bfloat16) rounds to nearest even (its documented
    behaviour); NaN is compared as a class because torch returns a canonical
    NaN.  Catches truncation, ties away from zero, overflow mistakes.
    """
    chunk = 1 << 26
    for start in range(0, 1 << 32, chunk):
        bits = np.arange(start, start + chunk, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        ours = oracle.rne16(x)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan_in = np.isnan(x)
        ours_nan = ((ours & 0x7FFF) > 0x7F80)
        assert np.array_equal(ours_nan, nan_in), hex(start)
        keep = ~nan_in
        if not np.array_equal(ours[keep], ref[keep]):
            bad = np.nonzero(ours[keep] != ref[keep])[0][:5]
            raise AssertionError(f"chunk {start:#x}: {bits[keep][bad]} "
                                 f"{ours[keep][bad]} {ref[keep][bad]}")


def test_rne16_textbook_on_boundaries():
    """Nearest bf16 by exact rational distance, ties to the even pattern.

    Covers every rounding situation (exact, just below/at/above the half-way
    point, largest dropped field) for a spread of upper halves, plus the
    overflow threshold next to the largest finite bf16.  Independent of torch.
    """
    rng = np.random.default_rng(5)
    his = np.concatenate([np.arange(0, 1 << 16, 257), [0x7F7F, 0xFF7F, 0x0000, 0x0080]])
    los = [0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF] + list(rng.integers(0, 1 << 16, 4))
    bits = np.array([(int(h) << 16) | int(lo) for h in his for lo in los],
                    dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    got = oracle.rne16(x)
    max_f = Fraction(float(np.array(0x7F7F0000, np.uint32).view(np.float32)))
    overflow_at = max_f + Fraction(2) ** 119          # half a bf16 ulp above max
    for xi, gi in zip(x, got):
        u = int(np.array(xi).view(np.uint32))
        xf = Fraction(float(xi))
        lo = u >> 16                                  # toward zero
        up = lo + 1                                   # away from zero
        if (up & 0x7FFF) == 0x7F80:
            expect = up if abs(xf) >= overflow_at else lo
        else:
            val = lambda p: Fraction(float(np.array(p << 16, np.uint32).view(np.float32)))
            da, db = abs(xf - val(lo)), abs(xf - val(up))
            expect = lo if da < db else up if db < da else (lo if lo % 2 == 0 else up)
        assert int(gi) == expect, (hex(u), hex(int(gi)), hex(expect))


def test_rne16_special_values():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0], np.float32)
    assert oracle.rne16(vals).tolist() == [0x0000, 0x8000, 0x7F80, 0xFF80, 0x3F80, 0xBF80]
    nan = np.array([np.nan, -np.nan], np.float32)
    out = oracle.rne16(nan)
    assert all((o & 0x7FFF) > 0x7F80 for o in out)
    assert out[1] & 0x8000 == (nan.view(np.uint32)[1] >> 16) & 0x8000


# --------------------------------------------------------- AdamW closed forms

def test_step1_closed_form_every_element():
    """P1: t=1 from m=v=0 gives the step lr*g/(|g|+eps) (sign-like step).

    With m = v = 0 the bias-corrected moments are g and g^2, so the update is
    lr * g / (|g| + eps): lr times the sign of g, up to eps.  Checked on every
    element of the GPT-2 c_attn workload's shape.  A wrong sign, a missing
    bias correction or eps inside the root fails.
    """
    w = synth.WORKLOADS["gpt2_cattn_first2"]
    n = w.params
    master, m, v, grad = rng_state(n, 11, fresh=True)
    c = consts(1)
    w_in = master.copy()
    oracle.adamw_step(master, m, v, grad, c)
    g = oracle.bf16_to_f32(grad).astype(np.float64)
    w1 = (w_in * np.float32(1.0 - H["lr"] * H["weight_decay"])).astype(np.float64)
    step = w1 - master.astype(np.float64)
    expect = H["lr"] * g / (np.abs(g) + H["eps"])
    bound = ulp32(w1) + 16 * U32 * H["lr"]
    assert np.all(np.abs(step - expect) <= bound)
    big = np.abs(expect) > bound                  # steps above rounding noise
    assert big.mean() > 0.99
    assert np.all(np.sign(step[big]) == np.sign(g[big]))


@pytest.mark.parametrize("scale", [1e-9, 1e-8, 3e-8])
def test_step1_eps_placement(scale):
    """P1 with |g| near eps: eps is added outside the square root.

    With eps inside the root the step would be lr*g/sqrt(g^2+eps), orders of
    magnitude smaller at these gradient sizes.
    """
    n = 4096
    master, m, v, _ = rng_state(n, 3, fresh=True)
    grad = oracle.rne16((np.random.default_rng(4).standard_normal(n) * scale).astype(np.float32))
    w_in = master.copy()
    oracle.adamw_step(master, m, v, grad, consts(1))
    g = oracle.bf16_to_f32(grad).astype(np.float64)
    w1 = (w_in * np.float32(1.0 - H["lr"] * H["weight_decay"])).astype(np.float64)
    step = w1 - master.astype(np.float64)
    expect = H["lr"] * g / (np.abs(g) + H["eps"])
    assert np.all(np.abs(step - expect) <= ulp32(w1) + 16 * U32 * H["lr"])


@pytest.mark.parametrize("t", [1, 2, 10, 100, 12345])
def test_zero_gradient_fresh_state(t):
    """P2: g = 0, m = v = 0 gives w * (1 - lr*wd), one rounding, and m=v=+0."""
    n = 10000
    master, m, v, _ = rng_state(n, 7, fresh=True)
    grad = np.zeros(n, np.uint16)
    w_in = master.copy()
    wb, _ = oracle.adamw_step(master, m, v, grad, consts(t))
    decay = np.float32(1.0 - H["lr"] * H["weight_decay"])
    assert np.array_equal(master.view(np.uint32), (w_in * decay).view(np.uint32))
    assert not m.view(np.uint32).any() and not v.view(np.uint32).any()
    assert np.array_equal(wb, oracle.rne16(master))


def test_zero_lr_keeps_weights():
    """P3: lr = 0 leaves w bit-exact (a -0 weight with m' < 0 becomes +0)."""
    n = 20000
    master, m, v, grad = rng_state(n, 9)
    master[:16] = -0.0
    w_in = master.copy()
    m_in, v_in = m.copy(), v.copy()
    c = consts(10, lr=0.0)
    oracle.adamw_step(master, m, v, grad, c)
    g = oracle.bf16_to_f32(grad)
    m_expect = np.float32(H["beta1"]) * m_in + np.float32(1 - H["beta1"]) * g
    assert np.array_equal(m.view(np.uint32), m_expect.view(np.uint32))
    v_expect = np.float32(H["beta2"]) * v_in + np.float32(1 - H["beta2"]) * (g * g)
    assert np.array_equal(v.view(np.uint32), v_expect.view(np.uint32))
    flip = (w_in.view(np.uint32) == 0x80000000) & (m < 0)
    assert np.array_equal(master.view(np.uint32)[~flip], w_in.view(np.uint32)[~flip])
    assert np.all(master.view(np.uint32)[flip] == 0)


@pytest.mark.parametrize("t", [1, 7, 100])
def test_zero_betas_sign_sgd(t):
    """P4: beta1 = beta2 = 0 is sign-SGD with decoupled decay, for any t, m, v.

    The old moments must drop out completely and the step must be
    lr*g/(|g|+eps).  Catches beta and 1-beta swapped, or a moment term read
    from the wrong array.
    """
    n = 50000
    master, m, v, grad = rng_state(n, 21)
    w_in = master.copy()
    c = consts(t, beta1=0.0, beta2=0.0)
    assert c[6] == np.float32(H["lr"]) and c[7] == np.float32(1.0)
    oracle.adamw_step(master, m, v, grad, c)
    g = oracle.bf16_to_f32(grad)
    assert np.array_equal(m, g)
    assert np.array_equal(v, g * g)
    w1 = (w_in * np.float32(1.0 - H["lr"] * H["weight_decay"])).astype(np.float64)
    g64 = g.astype(np.float64)
    expect = H["lr"] * g64 / (np.abs(g64) + H["eps"])
    assert np.all(np.abs((w1 - master) - expect) <= ulp32(w1) + 8 * U32 * H["lr"])


# --------------------------------------------------------------- brute force

@pytest.mark.parametrize("n", [1, 7, 64, 257])
def test_bruteforce_recurrence_200_steps(n):
    """P5: numpy scalar recurrence == C oracle bit for bit, T = 1..200.

    Alongside, the fp32 master stays within a derived bound of the float64
    textbook AdamW recurrence on the same gradients.
    """
    rng = np.random.default_rng(100 + n)
    master, m, v, _ = rng_state(n, 200 + n)
    bm, bmm, bv = master.copy(), m.copy(), v.copy()
    w64, m64, v64 = master.astype(np.float64), m.astype(np.float64), v.astype(np.float64)
    err_bound = np.zeros(n)
    for t in range(1, 201):
        grad = oracle.rne16((rng.standard_normal(n) * 1e-3).astype(np.float32))
        c = consts(t)
        wb, _ = oracle.adamw_step(master, m, v, grad, c)
        bc = bruteforce.constants(H["lr"], H["beta1"], H["beta2"], H["eps"],
                                  H["weight_decay"], t)
        bm, bmm, bv, bwb, _ = bruteforce.adamw_step(bm, bmm, bv, grad, bc)
        assert np.array_equal(master.view(np.uint32), bm.view(np.uint32)), t
        assert np.array_equal(m.view(np.uint32), bmm.view(np.uint32)), t
        assert np.array_equal(v.view(np.uint32), bv.view(np.uint32)), t
        assert np.array_equal(wb, bwb), t
        # float64 textbook AdamW
        g = oracle.bf16_to_f32(grad).astype(np.float64)
        b1, b2, lr, eps, wd = H["beta1"], H["beta2"], H["lr"], H["eps"], H["weight_decay"]
        m64 = b1 * m64 + (1 - b1) * g
        v64 = b2 * v64 + (1 - b2) * g * g
        upd = lr * (m64 / (1 - b1 ** t)) / (np.sqrt(v64 / (1 - b2 ** t)) + eps)
        w64 = w64 * (1 - lr * wd) - upd
        # per step: the decay factor's own fp32 rounding acting on |w|, one
        # rounding of w', and the worst-case drift of the fp32 moments, which
        # grows at most linearly in t
        decay_err = abs(float(np.float32(1 - lr * wd)) - (1 - lr * wd))
        err_bound = (err_bound * (1 - lr * wd) + decay_err * np.abs(w64)
                     + ulp32(master) + (8 + 4 * t) * U32 * np.abs(upd))
        assert np.all(np.abs(master - w64) <= err_bound), t


def test_bruteforce_4096_with_delta_and_fp32_grad():
    n = 4096
    master, m, v, grad = rng_state(n, 77)
    orig = oracle.rne16(master)
    acc = (np.random.default_rng(3).standard_normal(n) * 3e-3).astype(np.float32)
    for g in (grad, acc):
        a = [x.copy() for x in (master, m, v)]
        c = consts(50)
        wb, d = oracle.adamw_step(a[0], a[1], a[2], g, c, orig=orig)
        bc = bruteforce.constants(H["lr"], H["beta1"], H["beta2"], H["eps"], H["weight_decay"], 50)
        r = bruteforce.adamw_step(master, m, v, g, bc, orig=orig)
        for x, y in zip((a[0], a[1], a[2], d), (r[0], r[1], r[2], r[4])):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))
        assert np.array_equal(wb, r[3])


# -------------------------------------------------------- library routine

@pytest.mark.parametrize("t", [1, 10, 50, 100])
def test_against_torch_adamw(t):
    """P6: torch.optim.AdamW (the routine the README's Quick Start calls).

    torch orders some operations differently (lerp for m, divide by
    sqrt(bc2) instead of multiplying by its inverse), so agreement is to a
    few ulps of each term, not bit for bit; the master must also be within
    2e-6 relative of torch wherever the update does not cancel it.
    """
    n = 1 << 16
    master, m, v, grad = rng_state(n, 300 + t, fresh=(t == 1))
    p = torch.nn.Parameter(torch.from_numpy(master.copy()))
    p.grad = torch.from_numpy(oracle.bf16_to_f32(grad).copy())
    opt = torch.optim.AdamW([p], lr=H["lr"], betas=(H["beta1"], H["beta2"]), eps=H["eps"],
                            weight_decay=H["weight_decay"], foreach=False, fused=False)
    opt.state[p] = {"step": torch.tensor(float(t - 1)),
                    "exp_avg": torch.from_numpy(m.copy()),
                    "exp_avg_sq": torch.from_numpy(v.copy())}
    opt.step()
    tw = p.detach().numpy().astype(np.float64)
    tm = opt.state[p]["exp_avg"].numpy().astype(np.float64)
    tv = opt.state[p]["exp_avg_sq"].numpy().astype(np.float64)

    g = oracle.bf16_to_f32(grad).astype(np.float64)
    m_terms = H["beta1"] * np.abs(m) + (1 - H["beta1"]) * np.abs(g)
    v_terms = H["beta2"] * np.abs(v) + (1 - H["beta2"]) * g * g
    w0 = master.astype(np.float64)
    oracle.adamw_step(master, m, v, grad, consts(t))
    upd = np.abs(w0 * (1 - H["lr"] * H["weight_decay"]) - master)
    assert np.all(np.abs(m - tm) <= 4 * U32 * m_terms)
    assert np.all(np.abs(v - tv) <= 4 * U32 * v_terms)
    # the update inherits m's absolute error (m' may cancel) through c_step/d
    c = consts(t)
    d = np.sqrt(v.astype(np.float64)) * float(c[7]) + H["eps"]
    m_err_in_upd = float(c[6]) * 4 * U32 * m_terms / d
    assert np.all(np.abs(master - tw) <= ulp32(master) + 16 * U32 * upd + m_err_in_upd)
    # relative agreement where w' is not the result of heavy cancellation
    keep = np.abs(tw) > 1e-3
    rel = np.abs(master[keep] - tw[keep]) / np.abs(tw[keep])
    assert keep.mean() > 0.9 and rel.max() <= 2e-6


# ------------------------------------------------------------- accumulation

def test_accumulate_exact_sums():
    """P7: gradients that are multiples of 2^-16 sum exactly in fp32."""
    rng = np.random.default_rng(1)
    n, k = 100000, 8
    ints = rng.integers(-255, 256, size=(k, n))
    grads = [oracle.rne16((ints[j] * 2.0 ** -16).astype(np.float32)) for j in range(k)]
    for j in range(k):       # representable: rne16 changed nothing
        assert np.array_equal(oracle.bf16_to_f32(grads[j]), (ints[j] * 2.0 ** -16).astype(np.float32))
    acc = np.full(n, 123.0, np.float32)
    oracle.grad_accum(acc, grads[0], overwrite=True)
    for j in range(1, k):
        oracle.grad_accum(acc, grads[j], overwrite=False)
    assert np.array_equal(acc.astype(np.float64), ints.sum(axis=0) * 2.0 ** -16)


def test_accumulate_random_bound_and_bruteforce():
    rng = np.random.default_rng(2)
    n, k = 3000, 8
    grads = [oracle.rne16((rng.standard_normal(n) * 10.0 ** rng.integers(-6, 1)).astype(np.float32))
             for _ in range(k)]
    acc = np.empty(n, np.float32)
    oracle.grad_accum(acc, grads[0], overwrite=True)
    for j in range(1, k):
        oracle.grad_accum(acc, grads[j], overwrite=False)
    ref = bruteforce.accumulate(grads)
    assert np.array_equal(acc.view(np.uint32), ref.view(np.uint32))
    gs = np.stack([oracle.bf16_to_f32(x).astype(np.float64) for x in grads])
    assert np.all(np.abs(acc - gs.sum(0)) <= (k - 1) * U32 * np.abs(gs).sum(0))


def test_accumulate_overwrite_keeps_negative_zero_and_specials():
    g = np.array([0x8000, 0x0000, 0x7F80, 0xFF80, 0x7FC1, 0x0001], np.uint16)
    acc = np.full(6, 5.0, np.float32)
    oracle.grad_accum(acc, g, overwrite=True)
    assert acc.view(np.uint32)[0] == 0x80000000 and acc.view(np.uint32)[1] == 0
    assert acc[2] == np.inf and acc[3] == -np.inf and np.isnan(acc[4])
    assert acc.view(np.uint32)[5] == 0x00010000          # bf16 subnormal kept
    acc2 = np.full(6, -0.0, np.float32)
    oracle.grad_accum(acc2, np.full(6, 0x8000, np.uint16), overwrite=False)
    assert np.all(acc2.view(np.uint32) == 0x80000000)    # -0 + -0 = -0


# ------------------------------------------------------------------- delta

def test_delta_reconstructs_master():
    """P9: delta = w' - base; base + delta gives w' back (README checkpoint).

    With the base equal to the bf16 copy of the starting weight, w' and the
    base are within a factor of two, so the fp32 subtraction is exact and
    base + delta == w' exactly.  A reversed sign or a delta taken from the
    previous step fails.
    """
    n = 100000
    master, m, v, grad = rng_state(n, 31, fresh=True)
    orig = oracle.rne16(master)
    _, delta = oracle.adamw_step(master, m, v, grad, consts(1), orig=orig)
    base = oracle.bf16_to_f32(orig).astype(np.float64)
    w = master.astype(np.float64)
    same = (np.sign(w) == np.sign(base)) & (np.abs(w) <= 2 * np.abs(base)) & (np.abs(base) <= 2 * np.abs(w))
    assert same.mean() > 0.99
    assert np.array_equal(delta[same].astype(np.float64) + base[same], w[same])
    assert np.all(np.abs(delta.astype(np.float64) + base - w) <= ulp32(master))


def test_delta_zero_when_master_equals_base():
    n = 5000
    master, m, v, grad = rng_state(n, 32)
    orig = oracle.rne16(master)
    master = oracle.bf16_to_f32(orig).copy()
    master[:3] = [0.0, -0.0, 1.0]
    orig[:3] = [0x0000, 0x8000, 0x3F80]
    _, delta = oracle.adamw_step(master, m, v, grad, consts(5, lr=0.0), orig=orig)
    assert not delta.view(np.uint32).any()


# ------------------------------------------------------------- specials

def test_nan_and_inf_propagate():
    n = 8
    master = np.array([np.nan, 1.0, 1.0, 1.0, np.inf, 1.0, 0.5, 0.0], np.float32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    grad = np.array([0x3A83, 0x7FC0, 0x7F80, 0xFF80, 0x3A83, 0x0001, 0x3A83, 0x3A83], np.uint16)
    v[6] = np.inf
    wb, _ = oracle.adamw_step(master, m, v, grad, consts(3))
    assert np.isnan(master[0]) and np.isnan(master[1]) and np.isnan(master[2])
    assert np.isnan(master[3]) and master[4] == np.inf
    assert np.isfinite(master[5]) and master[6] == np.float32(0.5) * np.float32(1 - 1e-6)
    assert ((wb[:4] & 0x7FFF) > 0x7F80).all()


# ---------------------------------------------------------------- merge delta

def test_merge_delta_reproduces_step_weight():
    """README merge_delta: base + saved delta gives the servable weight back.

    The delta a step writes is w' - f32(base), exact wherever w' and the base
    are within a factor of two (Sterbenz), so merging it reproduces
    rne16(w'), the bf16 weight of the same step, bit for bit there.
    """
    n = 200000
    master, m, v, grad = rng_state(n, 41)
    base = oracle.rne16(master)
    wb, delta = oracle.adamw_step(master, m, v, grad, consts(100), orig=base)
    merged = oracle.merge_delta(base, delta)
    b = oracle.bf16_to_f32(base).astype(np.float64)
    w = master.astype(np.float64)
    same = (np.sign(w) == np.sign(b)) & (np.abs(w) <= 2 * np.abs(b)) & (np.abs(b) <= 2 * np.abs(w))
    assert same.mean() > 0.99
    assert np.array_equal(merged[same], wb[same])


def test_merge_delta_zero_delta_and_bruteforce():
    rng = np.random.default_rng(8)
    base = oracle.rne16((rng.standard_normal(5000) * 0.02).astype(np.float32))
    base[:4] = [0x0000, 0x8000, 0x7F80, 0x7FC0]
    zero = np.zeros(5000, np.float32)
    merged = oracle.merge_delta(base, zero)
    assert np.array_equal(merged[4:], base[4:])                     # exact
    assert merged[0] == 0 and merged[1] == 0 and merged[2] == 0x7F80  # -0 + 0 = +0
    assert (merged[3] & 0x7FFF) > 0x7F80
    delta = (rng.standard_normal(5000) * 1e-4).astype(np.float32)
    got = oracle.merge_delta(base, delta)
    ref = bruteforce.merge_delta(base, delta)
    nan = (ref & 0x7FFF) > 0x7F80
    assert np.array_equal(got[~nan], ref[~nan])
    # against float64 arithmetic: the merged value is the bf16 nearest to base+delta
    exact = oracle.bf16_to_f32(base[4:]).astype(np.float64) + delta[4:].astype(np.float64)
    mval = oracle.bf16_to_f32(got[4:]).astype(np.float64)
    ulp16 = np.spacing(np.abs(mval).astype(np.float32)).astype(np.float64) * 65536
    assert np.all(np.abs(mval - exact) <= 0.5 * ulp16 + np.spacing(np.abs(exact).astype(np.float32)))


def test_thread_count_does_not_change_results():
    """The oracle's loops run element by element, so one thread and all
    threads must give identical bytes."""
    n = 200_003
    cores = oracle.num_threads()
    outs = []
    try:
        for t in (1, max(2, cores)):
            oracle.set_num_threads(t)
            assert oracle.num_threads() == t
            master, m, v, grad = rng_state(n, 77)
            wb, delta = oracle.adamw_step(master, m, v, grad, consts(10), orig=oracle.rne16(master))
            outs.append([a.view(np.uint32) if a.dtype == np.float32 else a
                         for a in (master, m, v, wb, delta)])
    finally:
        oracle.set_num_threads(cores)
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
