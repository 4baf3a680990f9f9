"""C-ABI checks that need no GPU: exports, constant derivation, validation.

Validation happens before any HIP call, so descriptors with made-up device
addresses exercise every error path here without touching a GPU.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest
import torch

import oracle
from optimizer_step_lema_amd import _native as N

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("lema.h", "lema_measure.h")]


@pytest.fixture(scope="module")
def lib():
    return N.load()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[\w\s\*]+?\b(lema_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert names == {s[0] for s in N.SIGNATURES}


def test_status_strings(lib):
    for code in range(-11, 1):
        assert lib.lema_status_string(code).startswith(b"LEMA_")
    assert b"unknown" in lib.lema_status_string(-99)
    assert lib.lema_version() >= 200


def args(**kw):
    base = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=10,
                grad_dtype=N.LEMA_GRAD_BF16, reserved=0)
    base.update(kw)
    return N.AdamwArgs(**base)


@pytest.mark.parametrize("hp", [
    dict(), dict(lr=3e-3, weight_decay=0.1), dict(beta1=0.0, beta2=0.0),
    dict(beta1=0.5, beta2=0.25, eps=1e-6), dict(lr=0.0), dict(weight_decay=0.0)])
@pytest.mark.parametrize("t", [1, 2, 10, 50, 100, 12345, 2 ** 40 + 1])
def test_constants_match_oracle(lib, hp, t):
    """The host derivation (C++) and the oracle's (C) give identical fp32 bits."""
    a = args(step=t, **hp)
    out = N.AdamwConsts()
    assert lib.lema_adamw_constants(ctypes.byref(a), ctypes.byref(out)) == N.LEMA_OK
    got = np.array([getattr(out, f) for f, _ in N.AdamwConsts._fields_], np.float32)
    ref = oracle.adamw_constants(a.lr, a.beta1, a.beta2, a.eps, a.weight_decay, t)
    assert got.view(np.uint32).tolist() == ref.view(np.uint32).tolist()


@pytest.mark.parametrize("bad,code", [
    (dict(step=0), N.LEMA_ERR_HPARAM), (dict(step=-3), N.LEMA_ERR_HPARAM),
    (dict(beta1=1.0), N.LEMA_ERR_HPARAM), (dict(beta2=-0.1), N.LEMA_ERR_HPARAM),
    (dict(eps=0.0), N.LEMA_ERR_HPARAM), (dict(lr=-1e-4), N.LEMA_ERR_HPARAM),
    (dict(weight_decay=-1.0), N.LEMA_ERR_HPARAM), (dict(lr=float("nan")), N.LEMA_ERR_HPARAM),
    (dict(eps=float("inf")), N.LEMA_ERR_HPARAM), (dict(reserved=1), N.LEMA_ERR_HPARAM),
    (dict(grad_dtype=2), N.LEMA_ERR_DTYPE), (dict(grad_dtype=-1), N.LEMA_ERR_DTYPE)])
def test_hparam_errors(lib, bad, code):
    a = args(**bad)
    out = N.AdamwConsts()
    assert lib.lema_adamw_constants(ctypes.byref(a), ctypes.byref(out)) == code
    seg = fake_seg(0x10000, 64)
    assert lib.lema_adamw_step(ctypes.byref(seg), 1, ctypes.byref(a), None) == code


def fake_seg(base, n, delta=False, gsize=2):
    """Descriptor with made-up, disjoint, well-aligned device addresses."""
    stride = 1 << 24
    p = [base + k * stride for k in range(7)]
    return N.AdamwSeg(p[0], p[1], p[2], p[3], p[4], p[5] if delta else 0,
                      p[6] if delta else 0, n)


def call(lib, segs, a=None):
    arr = (N.AdamwSeg * max(1, len(segs)))(*segs)
    return lib.lema_adamw_step(arr, len(segs), ctypes.byref(a or args()), None)


def test_null_and_size_errors(lib):
    a = args()
    assert lib.lema_adamw_step(None, 1, ctypes.byref(a), None) == N.LEMA_ERR_NULL
    assert lib.lema_adamw_step(None, -1, ctypes.byref(a), None) == N.LEMA_ERR_SIZE
    seg = fake_seg(1 << 32, 10)
    assert lib.lema_adamw_step(ctypes.byref(seg), 1, None, None) == N.LEMA_ERR_NULL
    s = fake_seg(1 << 32, -1)
    assert call(lib, [s]) == N.LEMA_ERR_SIZE
    for field in ("master", "exp_avg", "exp_avg_sq", "grad", "weight_bf16"):
        s = fake_seg(1 << 32, 10)
        setattr(s, field, 0)
        assert call(lib, [s]) == N.LEMA_ERR_NULL, field
    s = fake_seg(1 << 32, 10, delta=True)
    s.delta = 0
    assert call(lib, [s]) == N.LEMA_ERR_NULL            # orig without delta
    s = fake_seg(1 << 32, 10, delta=True)
    s.orig_bf16 = 0
    assert call(lib, [s]) == N.LEMA_ERR_NULL            # delta without orig
    # the error in the second segment is still found before anything runs
    assert call(lib, [fake_seg(1 << 32, 10), fake_seg(1 << 40, -5)]) == N.LEMA_ERR_SIZE


def test_alignment_errors(lib):
    s = fake_seg(1 << 32, 10)
    s.master += 2
    assert call(lib, [s]) == N.LEMA_ERR_ALIGN
    s = fake_seg(1 << 32, 10)
    s.weight_bf16 += 1
    assert call(lib, [s]) == N.LEMA_ERR_ALIGN
    s = fake_seg(1 << 32, 10)
    s.grad += 2                                          # bf16 grad: 2-byte aligned is fine
    assert call(lib, [s]) != N.LEMA_ERR_ALIGN
    s = fake_seg(1 << 32, 10)
    s.grad += 2
    assert call(lib, [s], args(grad_dtype=N.LEMA_GRAD_FP32)) == N.LEMA_ERR_ALIGN


def test_overlap_errors(lib):
    s = fake_seg(1 << 32, 1000)
    s.exp_avg = s.master + 400                           # m inside master
    assert call(lib, [s]) == N.LEMA_ERR_OVERLAP
    s = fake_seg(1 << 32, 1000)
    s.weight_bf16 = s.grad + 100                         # written over a read array
    assert call(lib, [s]) == N.LEMA_ERR_OVERLAP
    a, b = fake_seg(1 << 32, 1000), fake_seg(1 << 32, 1000)
    b2 = fake_seg((1 << 32) + 8 * 1000, 1000)            # shifted copy: disjoint? no, same stride
    assert call(lib, [a, b]) == N.LEMA_ERR_OVERLAP       # two segments on the same arrays
    # two segments may read one gradient buffer (read-only overlap is allowed)
    c, d = fake_seg(1 << 32, 1000), fake_seg(1 << 40, 1000)
    d.grad = c.grad
    assert call(lib, [c, d]) != N.LEMA_ERR_OVERLAP
    del b2


def test_overlap_check_of_repeated_long_lists(lib):
    """Long span lists (here 40 segments, 280 spans) are checked once per
    thread and then recognized when repeated: a repeat of a clean list passes,
    any change is checked again, and a list with a conflict is rejected every
    time, also right after its clean twin."""
    clean = [fake_seg((1 << 32) + i * (1 << 28), 1000, delta=True) for i in range(40)]
    for _ in range(3):
        assert call(lib, clean) != N.LEMA_ERR_OVERLAP
    bad = [fake_seg((1 << 32) + i * (1 << 28), 1000, delta=True) for i in range(40)]
    bad[17].exp_avg = bad[3].master + 4 * 500          # m of one tensor inside another's master
    for _ in range(2):
        assert call(lib, bad) == N.LEMA_ERR_OVERLAP
    assert call(lib, clean) != N.LEMA_ERR_OVERLAP
    assert call(lib, bad) == N.LEMA_ERR_OVERLAP
    # same addresses, one length longer: the tensor now runs into the next array
    longer = [fake_seg((1 << 32) + i * (1 << 28), 1000, delta=True) for i in range(40)]
    longer[5].numel = (1 << 24) // 4 + 1
    assert call(lib, longer) == N.LEMA_ERR_OVERLAP
    assert call(lib, clean) != N.LEMA_ERR_OVERLAP


def test_empty_calls_are_noops_without_gpu(lib):
    assert lib.lema_adamw_step(None, 0, ctypes.byref(args()), None) == N.LEMA_OK
    z = fake_seg(1 << 32, 0)
    z.master = 0                                         # numel 0: pointers may be NULL
    assert call(lib, [z]) == N.LEMA_OK
    acc0 = N.AccumSeg(0, 0, 0)
    assert lib.lema_grad_accum(ctypes.byref(acc0), 1, 0, None) == N.LEMA_OK


def test_accum_validation(lib):
    assert lib.lema_grad_accum(None, 2, 1, None) == N.LEMA_ERR_NULL
    assert lib.lema_grad_accum(None, -2, 1, None) == N.LEMA_ERR_SIZE
    s = N.AccumSeg(0, 1 << 33, 10)
    assert lib.lema_grad_accum(ctypes.byref(s), 1, 1, None) == N.LEMA_ERR_NULL
    s = N.AccumSeg((1 << 32) + 2, 1 << 33, 10)
    assert lib.lema_grad_accum(ctypes.byref(s), 1, 1, None) == N.LEMA_ERR_ALIGN
    s = N.AccumSeg(1 << 32, (1 << 32) + 8, 10)
    assert lib.lema_grad_accum(ctypes.byref(s), 1, 1, None) == N.LEMA_ERR_OVERLAP
    s = N.AccumSeg(1 << 32, 1 << 33, -1)
    assert lib.lema_grad_accum(ctypes.byref(s), 1, 1, None) == N.LEMA_ERR_SIZE


def test_slot_and_measure_validation(lib):
    h = ctypes.c_void_p()
    assert lib.lema_slot_pool_create(None, 1 << 20, 2, 1, 2, ctypes.byref(h)) == N.LEMA_ERR_NULL
    assert lib.lema_slot_pool_create(1 << 32, 1 << 20, 1, 1, 2, ctypes.byref(h)) == N.LEMA_ERR_SIZE
    assert lib.lema_slot_pool_create(1 << 32, 1000, 2, 1, 2, ctypes.byref(h)) == N.LEMA_ERR_SIZE
    assert lib.lema_slot_pool_create(1 << 32, 1 << 20, 2, 1, 1, ctypes.byref(h)) == N.LEMA_ERR_NULL
    assert lib.lema_slot_pool_destroy(None) == N.LEMA_OK
    assert lib.lema_slot_stream(None, None, 0, ctypes.byref(args()), None) == N.LEMA_ERR_NULL
    assert lib.lema_measure_copy(None, 1 << 32, 16, None) == N.LEMA_ERR_NULL
    assert lib.lema_measure_copy(1 << 32, 1 << 33, 15, None) == N.LEMA_ERR_SIZE
    assert lib.lema_measure_copy((1 << 32) + 4, 1 << 33, 16, None) == N.LEMA_ERR_ALIGN
    assert lib.lema_measure_copy(1 << 32, (1 << 32) + 16, 64, None) == N.LEMA_ERR_OVERLAP
    assert lib.lema_probe_fp32(0, 0, 0, 0, 0, -1, None) == N.LEMA_ERR_SIZE
    assert lib.lema_probe_fp32(0, 0, 0, 0, 0, 5, None) == N.LEMA_ERR_NULL
    assert lib.lema_host_alloc(None, 16) == N.LEMA_ERR_NULL
    assert lib.lema_host_free(None) == N.LEMA_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-GPU error path")
def test_valid_call_without_gpu_reports_hip_error(lib):
    s = fake_seg(1 << 32, 10)
    assert call(lib, [s]) == N.LEMA_ERR_HIP
    assert lib.lema_last_hip_error() != 0


def test_step_accum_validation(lib):
    a16 = args(grad_dtype=N.LEMA_GRAD_BF16)
    a32 = args(grad_dtype=N.LEMA_GRAD_FP32)
    s = fake_seg(1 << 32, 100)
    arr = (N.AdamwSeg * 1)(s)
    last = (ctypes.c_void_p * 1)(1 << 40)
    assert lib.lema_adamw_step_accum(arr, last, 1, ctypes.byref(a16), None) == N.LEMA_ERR_DTYPE
    assert lib.lema_adamw_step_accum(arr, None, 1, ctypes.byref(a32), None) == N.LEMA_ERR_NULL
    nul = (ctypes.c_void_p * 1)(0)
    assert lib.lema_adamw_step_accum(arr, nul, 1, ctypes.byref(a32), None) == N.LEMA_ERR_NULL
    odd = (ctypes.c_void_p * 1)((1 << 40) + 1)
    assert lib.lema_adamw_step_accum(arr, odd, 1, ctypes.byref(a32), None) == N.LEMA_ERR_ALIGN
    over = (ctypes.c_void_p * 1)(s.weight_bf16 + 10)     # last overlaps a written array
    assert lib.lema_adamw_step_accum(arr, over, 1, ctypes.byref(a32), None) == N.LEMA_ERR_OVERLAP
    shared = (ctypes.c_void_p * 1)(s.grad)               # reading the accumulator twice is fine
    assert lib.lema_adamw_step_accum(arr, shared, 1, ctypes.byref(a32), None) != N.LEMA_ERR_OVERLAP
    assert lib.lema_adamw_step_accum(None, None, 0, ctypes.byref(a32), None) == N.LEMA_OK


def test_merge_validation(lib):
    assert lib.lema_merge_delta(None, 1, None) == N.LEMA_ERR_NULL
    assert lib.lema_merge_delta(None, -1, None) == N.LEMA_ERR_SIZE
    assert lib.lema_merge_delta(None, 0, None) == N.LEMA_OK
    s = N.MergeSeg(1 << 32, 1 << 33, 0, 10)
    assert lib.lema_merge_delta(ctypes.byref(s), 1, None) == N.LEMA_ERR_NULL
    s = N.MergeSeg((1 << 32) + 1, 1 << 33, 1 << 34, 10)
    assert lib.lema_merge_delta(ctypes.byref(s), 1, None) == N.LEMA_ERR_ALIGN
    s = N.MergeSeg(1 << 32, (1 << 33) + 2, 1 << 34, 10)
    assert lib.lema_merge_delta(ctypes.byref(s), 1, None) == N.LEMA_ERR_ALIGN
    s = N.MergeSeg(1 << 32, 1 << 33, (1 << 32) + 4, 10)        # output over the base
    assert lib.lema_merge_delta(ctypes.byref(s), 1, None) == N.LEMA_ERR_OVERLAP
    s = N.MergeSeg(1 << 32, 1 << 33, 1 << 34, -3)
    assert lib.lema_merge_delta(ctypes.byref(s), 1, None) == N.LEMA_ERR_SIZE


def microbatch_call(lib, segs, grads, nmb, a=None):
    arr = (N.AdamwSeg * max(1, len(segs)))(*segs)
    ptrs = (ctypes.c_void_p * max(1, len(grads)))(*grads)
    return lib.lema_adamw_step_microbatches(arr, ptrs, len(segs), nmb, ctypes.byref(a or args()),
                                            None)


def test_microbatch_step_validation(lib):
    """lema_adamw_step_microbatches: K range, grad field NULL, every micro-batch
    pointer present, aligned and not overlapping a written array."""
    def seg():
        s = fake_seg(1 << 32, 1000)
        s.grad = 0
        return s
    grads = [(1 << 40) + k * (1 << 24) for k in range(3)]
    assert microbatch_call(lib, [seg()], grads, 0) == N.LEMA_ERR_SIZE
    assert microbatch_call(lib, [seg()], grads * 6, 17) == N.LEMA_ERR_SIZE
    s = fake_seg(1 << 32, 1000)                           # grad must be NULL
    assert microbatch_call(lib, [s], grads, 3) == N.LEMA_ERR_NULL
    assert microbatch_call(lib, [seg()], grads, 3, args(grad_dtype=N.LEMA_GRAD_FP32)) == \
        N.LEMA_ERR_DTYPE
    assert microbatch_call(lib, [seg()], [grads[0], 0, grads[2]], 3) == N.LEMA_ERR_NULL
    assert microbatch_call(lib, [seg()], [grads[0], grads[1] + 1, grads[2]], 3) == N.LEMA_ERR_ALIGN
    s = seg()
    assert microbatch_call(lib, [s], [grads[0], s.master + 8, grads[2]], 3) == N.LEMA_ERR_OVERLAP
    arr = (N.AdamwSeg * 1)(seg())
    assert lib.lema_adamw_step_microbatches(arr, None, 1, 3, ctypes.byref(args()), None) == \
        N.LEMA_ERR_NULL
    assert lib.lema_adamw_step_microbatches(None, None, 0, 3, ctypes.byref(args()), None) == \
        N.LEMA_OK
    z = seg()
    z.numel = 0
    assert microbatch_call(lib, [z], [0, 0, 0], 3) == N.LEMA_OK   # empty segment: no pointers needed


def test_noalloc_validation(lib):
    """lema_adamw_step_noalloc validates as lema_adamw_step does, and refuses
    more than LEMA_NOALLOC_MAX_SEGMENTS segments, all before any HIP call."""
    a = args()

    def na(segs, a=a):
        arr = (N.AdamwSeg * max(1, len(segs)))(*segs)
        return lib.lema_adamw_step_noalloc(arr, len(segs), ctypes.byref(a), None)

    assert lib.lema_adamw_step_noalloc(None, 0, ctypes.byref(a), None) == N.LEMA_OK
    assert lib.lema_adamw_step_noalloc(None, -1, ctypes.byref(a), None) == N.LEMA_ERR_SIZE
    assert lib.lema_adamw_step_noalloc(None, 1, ctypes.byref(a), None) == N.LEMA_ERR_NULL
    assert na([fake_seg(1 << 32, 10)], args(step=0)) == N.LEMA_ERR_HPARAM
    lim = N.LEMA_NOALLOC_MAX_SEGMENTS
    many = [fake_seg((1 << 36) + (k << 28), 8) for k in range(lim + 1)]
    assert na(many) == N.LEMA_ERR_SIZE
    s = fake_seg(1 << 32, 1000)
    s.exp_avg = s.master + 400
    assert na([s]) == N.LEMA_ERR_OVERLAP
    s = fake_seg(1 << 32, 10)
    s.master += 2
    assert na([s]) == N.LEMA_ERR_ALIGN
    z = fake_seg(1 << 32, 0)
    z.master = 0
    assert na([z] * 3) == N.LEMA_OK                      # only empty segments: a no-op
    # a valid call at the limit gets past validation (no GPU here: HIP error)
    assert na(many[:lim]) == N.LEMA_ERR_HIP


def test_residency_probe_validation(lib):
    rec = 1 << 32
    assert lib.lema_probe_residency(None, 10, 64, 0, 20, None) == N.LEMA_ERR_NULL
    for wg, lanes, lds, spin in ((0, 64, 0, 20), (10, 32, 0, 20), (10, 96, 0, 20),
                                 (10, 2048, 0, 20), (10, 64, -1, 20), (10, 64, 65537, 20),
                                 (10, 64, 0, 0), (10, 64, 0, 1001)):
        assert lib.lema_probe_residency(rec, wg, lanes, lds, spin, None) == N.LEMA_ERR_SIZE
    assert lib.lema_probe_residency(rec + 4, 10, 64, 0, 20, None) == N.LEMA_ERR_ALIGN
    out = (ctypes.c_int32 * 6)()
    assert lib.lema_step_occupancy(0, None) == N.LEMA_ERR_NULL
    assert lib.lema_step_occupancy(4, out) == N.LEMA_ERR_SIZE
    assert lib.lema_step_occupancy(-1, out) == N.LEMA_ERR_SIZE
