"""Second, independent oracle: a per-element loop over numpy float32 scalars.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).  It is written apart from
``lema_oracle.c`` and is only fast enough for tiny tensors; the tests use it
to check the C oracle element by element.

Each numpy float32 scalar operation is one IEEE binary32 operation rounded to
nearest even, so the loop below is the AdamW step of the LEMA README ("Quick
Start": torch.optim.AdamW; "Selective Full Fine-Tuning": fp32 states and
accumulation, fp32 delta) with the same fixed rounding points as the C
oracle, restated from the definition rather than from that file.
"""
from __future__ import annotations

import math

import numpy as np

F = np.float32


def beta_power(beta: float, t: int) -> float:
    """beta**t in double precision by square-and-multiply (low bit first)."""
    acc, base = 1.0, float(beta)
    while t:
        if t % 2 == 1:
            acc *= base
        base *= base
        t //= 2
    return acc


def constants(lr, beta1, beta2, eps, weight_decay, step):
    """dict of the eight fp32 constants, each one double->fp32 rounding."""
    return {
        "b1": F(beta1),
        "one_minus_b1": F(1.0 - beta1),
        "b2": F(beta2),
        "one_minus_b2": F(1.0 - beta2),
        "eps": F(eps),
        "decay": F(1.0 - lr * weight_decay),
        "step_size": F(lr / (1.0 - beta_power(beta1, step))),
        "inv_bc2_root": F(1.0 / math.sqrt(1.0 - beta_power(beta2, step))),
    }


def to_bf16_bits(x) -> int:
    """fp32 -> bf16 pattern, nearest with ties to even, by integer arithmetic."""
    u = int(np.array(x, dtype=np.float32).view(np.uint32))
    if (u & 0x7FFFFFFF) > 0x7F800000:
        return ((u >> 16) | 0x40) & 0xFFFF
    hi, lo = divmod(u, 1 << 16)
    if lo > 0x8000 or (lo == 0x8000 and hi % 2 == 1):
        hi += 1
    return hi & 0xFFFF


def from_bf16_bits(b) -> np.float32:
    return np.array(int(b) << 16, dtype=np.uint32).view(np.float32)[()]


def adamw_element(w, m, v, g, c):
    """One element of one step; returns (w', m', v', bf16(w'))."""
    w, m, v, g = F(w), F(m), F(v), F(g)
    w1 = w * c["decay"]
    m2 = c["b1"] * m + c["one_minus_b1"] * g
    v2 = c["b2"] * v + c["one_minus_b2"] * (g * g)
    d = np.sqrt(v2) * c["inv_bc2_root"] + c["eps"]
    w2 = w1 - c["step_size"] * (m2 / d)
    return F(w2), F(m2), F(v2), to_bf16_bits(w2)


def adamw_step(master, m, v, grad, c, orig=None):
    """Loop version over 1-D arrays; returns new copies (nothing in place).

    ``grad`` is uint16 (bf16 patterns) or float32.
    Returns (master', m', v', weight_bf16, delta or None).
    """
    n = len(master)
    out_w = np.empty(n, np.float32)
    out_m = np.empty(n, np.float32)
    out_v = np.empty(n, np.float32)
    out_b = np.empty(n, np.uint16)
    out_d = None if orig is None else np.empty(n, np.float32)
    with np.errstate(all="ignore"):
        for i in range(n):
            g = from_bf16_bits(grad[i]) if grad.dtype == np.uint16 else F(grad[i])
            w2, m2, v2, b = adamw_element(master[i], m[i], v[i], g, c)
            out_w[i], out_m[i], out_v[i], out_b[i] = w2, m2, v2, b
            if orig is not None:
                out_d[i] = w2 - from_bf16_bits(orig[i])
    return out_w, out_m, out_v, out_b, out_d


def accumulate(grads_bf16):
    """Left fold of bf16 micro-batch gradients into fp32, in order."""
    n = len(grads_bf16[0])
    acc = np.empty(n, np.float32)
    with np.errstate(all="ignore"):
        for i in range(n):
            s = from_bf16_bits(grads_bf16[0][i])
            for k in range(1, len(grads_bf16)):
                s = F(s + from_bf16_bits(grads_bf16[k][i]))
            acc[i] = s
    return acc


def merge_delta(base_bf16, delta):
    """Loop version of the bf16 merge: rne16(f32(base) + delta) per element."""
    out = np.empty(len(base_bf16), np.uint16)
    with np.errstate(all="ignore"):
        for i in range(len(base_bf16)):
            out[i] = to_bf16_bits(F(from_bf16_bits(base_bf16[i]) + F(delta[i])))
    return out


# ------------------------------------------------- int8 rows with scales
#
# Symmetric absmax int8 with one fp32 scale per row (README "Quantization",
# the int8 + per-row-scale storage of moments and accumulators), restated
# with Python integers and numpy float32 scalars: the absmax by comparing
# magnitudes one at a time, the half-to-even rounding by Python's round() on
# the exactly widened quotient.

def quantize_row(xs):
    """list of fp32 values -> (list of int codes, fp32 scale)."""
    a = F(0.0)
    nan = False
    for x in xs:
        mag = abs(F(x))
        if mag != mag:
            nan = True
        elif mag > a:
            a = mag
    with np.errstate(all="ignore"):
        s = F(np.nan) if nan else F(a / F(127.0))
        usable = bool(np.isfinite(s)) and s > 0
        codes = []
        for x in xs:
            if not usable:
                codes.append(0)
                continue
            k = round(float(F(F(x) / s)))      # round() on a float: ties to even
            codes.append(max(-127, min(127, k)))
    return codes, s


def quantize(x, row_len):
    """1-D fp32 array -> (int8 array, fp32 scales), rows of row_len (last short)."""
    n = len(x)
    q = np.zeros(n, np.int8)
    scales = []
    for lo in range(0, n, row_len):
        codes, s = quantize_row([x[i] for i in range(lo, min(n, lo + row_len))])
        q[lo:lo + len(codes)] = codes
        scales.append(s)
    return q, np.array(scales, np.float32)


def dequantize(q, scales, row_len):
    out = np.empty(len(q), np.float32)
    with np.errstate(all="ignore"):
        for i in range(len(q)):
            out[i] = F(F(int(q[i])) * scales[i // row_len])
    return out


def adamw_step_q8(master, m_q, m_s, v_q, v_s, grad, c, row_len, orig=None):
    """Dequantize the moments, loop the fp32 step, quantize the new moments.

    ``grad`` is uint16 (bf16), float32, or a tuple (int8 codes, scales).
    Returns (master', (m_q', m_s'), (v_q', v_s'), weight_bf16, delta or None).
    """
    if isinstance(grad, tuple):
        grad = dequantize(grad[0], grad[1], row_len)
    m = dequantize(m_q, m_s, row_len)
    v = dequantize(v_q, v_s, row_len)
    w2, m2, v2, wb, d = adamw_step(master, m, v, grad, c, orig)
    return w2, quantize(m2, row_len), quantize(v2, row_len), wb, d


def accumulate_q8(grads_bf16, row_len):
    """int8 accumulator after each bf16 micro-batch: the first is quantized on
    its own, every later one is added to the dequantized accumulator."""
    acc_q, acc_s = None, None
    for k, g in enumerate(grads_bf16):
        with np.errstate(all="ignore"):
            if k == 0:
                vals = np.array([from_bf16_bits(b) for b in g], np.float32)
            else:
                prev = dequantize(acc_q, acc_s, row_len)
                vals = np.array([F(prev[i] + from_bf16_bits(g[i])) for i in range(len(g))],
                                np.float32)
        acc_q, acc_s = quantize(vals, row_len)
    return acc_q, acc_s
