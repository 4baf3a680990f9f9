"""Validation of the int8 entry points without a GPU.

Every argument is checked before any HIP call, so descriptors with made-up,
disjoint device addresses reach every error path here.
"""
from __future__ import annotations

import ctypes

import pytest
import torch

from optimizer_step_lema_amd import _native as N

BASE = 1 << 32
STRIDE = 1 << 26


@pytest.fixture(scope="module")
def lib():
    return N.load()


def args(**kw):
    base = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=10,
                grad_dtype=N.LEMA_GRAD_BF16, reserved=0)
    base.update(kw)
    return N.AdamwArgs(**base)


def qseg(n=4096, row_len=256, base=BASE, delta=False):
    p = [base + k * STRIDE for k in range(10)]
    return N.AdamwQ8Seg(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7],
                        p[8] if delta else 0, p[9] if delta else 0, n, row_len)


def step(lib, segs, a=None, moments=N.LEMA_STATE_Q8):
    arr = (N.AdamwQ8Seg * max(1, len(segs)))(*segs)
    return lib.lema_adamw_step_q8(arr, len(segs), ctypes.byref(a or args()), moments, None)


def test_dtype_errors(lib):
    assert step(lib, [qseg()], moments=2) == N.LEMA_ERR_DTYPE
    assert step(lib, [qseg()], moments=-1) == N.LEMA_ERR_DTYPE
    assert step(lib, [qseg()], args(grad_dtype=3)) == N.LEMA_ERR_DTYPE
    # the plain step does not take an int8 gradient
    plain = N.AdamwSeg(BASE, BASE + STRIDE, BASE + 2 * STRIDE, BASE + 3 * STRIDE,
                       BASE + 4 * STRIDE, 0, 0, 64)
    assert lib.lema_adamw_step(ctypes.byref(plain), 1, ctypes.byref(args(grad_dtype=N.LEMA_GRAD_Q8)),
                               None) == N.LEMA_ERR_DTYPE


@pytest.mark.parametrize("row_len", [0, -4, N.LEMA_Q8_MAX_ROW + 1, 1 << 40])
def test_row_length_limits(lib, row_len):
    assert step(lib, [qseg(row_len=row_len)]) == N.LEMA_ERR_SIZE
    acc = N.AccumQ8Seg(BASE, BASE + STRIDE, BASE + 2 * STRIDE, 100, row_len)
    assert lib.lema_grad_accum_q8(ctypes.byref(acc), 1, 0, None) == N.LEMA_ERR_SIZE
    t = N.Q8Tensor(BASE, BASE + STRIDE, BASE + 2 * STRIDE, 100, row_len)
    assert lib.lema_quantize_rows(ctypes.byref(t), 1, None) == N.LEMA_ERR_SIZE
    assert lib.lema_dequantize_rows(ctypes.byref(t), 1, None) == N.LEMA_ERR_SIZE


def test_null_pointers(lib):
    for field in ("master", "exp_avg", "exp_avg_scale", "exp_avg_sq", "exp_avg_sq_scale",
                  "grad", "weight_bf16"):
        s = qseg()
        setattr(s, field, 0)
        assert step(lib, [s]) == N.LEMA_ERR_NULL, field
    s = qseg()
    s.grad_scale = 0
    assert step(lib, [s], args(grad_dtype=N.LEMA_GRAD_Q8)) == N.LEMA_ERR_NULL
    # fp32 moments need no scales
    s = qseg()
    s.exp_avg_scale = s.exp_avg_sq_scale = 0
    assert step(lib, [s], args(grad_dtype=N.LEMA_GRAD_Q8), N.LEMA_STATE_FP32) != N.LEMA_ERR_NULL
    s = qseg(delta=True)
    s.delta = 0
    assert step(lib, [s]) == N.LEMA_ERR_NULL
    assert lib.lema_adamw_step_q8(None, 1, ctypes.byref(args()), 1, None) == N.LEMA_ERR_NULL
    assert lib.lema_adamw_step_q8(None, -1, ctypes.byref(args()), 1, None) == N.LEMA_ERR_SIZE
    assert lib.lema_grad_accum_q8(None, 1, 0, None) == N.LEMA_ERR_NULL
    acc = N.AccumQ8Seg(BASE, 0, BASE + 2 * STRIDE, 100, 10)
    assert lib.lema_grad_accum_q8(ctypes.byref(acc), 1, 0, None) == N.LEMA_ERR_NULL
    t = N.Q8Tensor(BASE, 0, BASE + 2 * STRIDE, 100, 10)
    assert lib.lema_quantize_rows(ctypes.byref(t), 1, None) == N.LEMA_ERR_NULL


def test_alignment(lib):
    s = qseg()
    s.exp_avg += 1                       # int8 codes need no alignment
    assert step(lib, [s]) != N.LEMA_ERR_ALIGN
    s = qseg()
    s.exp_avg_scale += 2                 # scales are fp32
    assert step(lib, [s]) == N.LEMA_ERR_ALIGN
    s = qseg()
    s.exp_avg += 2                       # fp32 moments must be 4-byte aligned
    assert step(lib, [s], args(grad_dtype=N.LEMA_GRAD_Q8), N.LEMA_STATE_FP32) == N.LEMA_ERR_ALIGN
    s = qseg()
    s.grad += 1
    assert step(lib, [s], args(grad_dtype=N.LEMA_GRAD_Q8)) != N.LEMA_ERR_ALIGN
    assert step(lib, [s]) == N.LEMA_ERR_ALIGN                    # as bf16 it is misaligned
    acc = N.AccumQ8Seg(BASE + 1, BASE + STRIDE + 2, BASE + 2 * STRIDE, 100, 10)
    assert lib.lema_grad_accum_q8(ctypes.byref(acc), 1, 0, None) == N.LEMA_ERR_ALIGN


def test_overlaps_include_scale_arrays(lib):
    s = qseg(n=4096, row_len=256)        # 16 rows: scales span 64 bytes
    s.exp_avg_sq_scale = s.exp_avg_scale + 32
    assert step(lib, [s]) == N.LEMA_ERR_OVERLAP
    s = qseg(n=4096, row_len=256)
    s.exp_avg_sq_scale = s.exp_avg_scale + 64     # adjacent, not overlapping
    assert step(lib, [s]) != N.LEMA_ERR_OVERLAP
    s = qseg(n=4096, row_len=256)
    s.exp_avg = s.master + 4 * 4096 - 8           # codes start inside master's tail
    assert step(lib, [s]) == N.LEMA_ERR_OVERLAP
    t = N.Q8Tensor(BASE, BASE + 100, BASE + STRIDE, 100, 10)
    assert lib.lema_quantize_rows(ctypes.byref(t), 1, None) == N.LEMA_ERR_OVERLAP
    # two dequantizations writing one x overlap; two quantizations reading it do not
    t2 = (N.Q8Tensor * 2)(N.Q8Tensor(BASE, BASE + STRIDE, BASE + 2 * STRIDE, 100, 10),
                          N.Q8Tensor(BASE, BASE + 3 * STRIDE, BASE + 4 * STRIDE, 100, 10))
    assert lib.lema_dequantize_rows(t2, 2, None) == N.LEMA_ERR_OVERLAP
    assert lib.lema_quantize_rows(t2, 2, None) != N.LEMA_ERR_OVERLAP  # x only read there


def test_empty_calls_are_noops_without_gpu(lib):
    assert lib.lema_adamw_step_q8(None, 0, ctypes.byref(args()), 1, None) == N.LEMA_OK
    z = qseg(n=0, row_len=0)
    z.master = 0
    assert step(lib, [z]) == N.LEMA_OK
    assert lib.lema_grad_accum_q8(None, 0, 1, None) == N.LEMA_OK
    assert lib.lema_quantize_rows(None, 0, None) == N.LEMA_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
def test_valid_calls_without_gpu_report_hip_error(lib):
    assert step(lib, [qseg()]) == N.LEMA_ERR_HIP
    acc = N.AccumQ8Seg(BASE, BASE + STRIDE, BASE + 2 * STRIDE, 100, 10)
    assert lib.lema_grad_accum_q8(ctypes.byref(acc), 1, 0, None) == N.LEMA_ERR_HIP
