"""Thin torch-facing binding over liblema.so.

Argument marshalling only: tensors are checked for dtype, device, length and
contiguity, turned into raw pointers and passed to the C ABI of
include/lema.h together with the current HIP stream.  Every step of the
optimizer path runs in the library's HIP kernels.

Method (LEMA README "Quick Start" and "Selective Full Fine-Tuning"; LLMScale
fine-tuning VRAM page): one per-layer AdamW step over fp32 master/m/v with a
bf16 gradient (or an fp32 accumulator), bf16 weight write-back and an
optional fp32 delta; fp32 accumulation of bf16 micro-batch gradients;
streaming of host-resident state through a pool of HBM slots.  README
"Quantization": the same step with int8 moments and int8 accumulators kept
as codes with per-row scales.  README "Features" and "Selective Full
Fine-Tuning": checkpoints of the delta and the optimizer state as
safetensors files.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Mapping, Optional, Sequence

import numpy as np
import torch

from . import _native as N


def _stream_handle(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(t: Optional[torch.Tensor], dtype, n: int, name: str, where: str = "cuda") -> int:
    if t is None:
        return 0
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.numel() != n:
        raise ValueError(f"{name}: expected {n} elements, got {t.numel()}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if where == "cuda":
        if not t.is_cuda:
            raise ValueError(f"{name}: must be a GPU tensor")
        if t.device.index != torch.cuda.current_device():
            raise ValueError(f"{name}: on {t.device}, but the current device is "
                             f"cuda:{torch.cuda.current_device()} (the library launches there)")
    if where == "cpu" and t.is_cuda:
        raise ValueError(f"{name}: must be a host tensor")
    return t.data_ptr() if n > 0 else 0


@dataclass
class AdamwSegment:
    """One trainable tensor: fp32 master/m/v, bf16 or fp32 grad, bf16 weight out.
    `grad` is None when the step takes resident micro-batch gradients."""
    master: torch.Tensor
    exp_avg: torch.Tensor
    exp_avg_sq: torch.Tensor
    grad: Optional[torch.Tensor]
    weight: torch.Tensor
    orig: Optional[torch.Tensor] = None
    delta: Optional[torch.Tensor] = None

    def to_c(self, where: str = "cuda") -> N.AdamwSeg:
        n = self.master.numel()
        gdt = torch.bfloat16 if self.grad is None else self.grad.dtype
        if gdt not in (torch.bfloat16, torch.float32):
            raise TypeError(f"grad: expected bfloat16 or float32, got {gdt}")
        return N.AdamwSeg(
            _check(self.master, torch.float32, n, "master", where),
            _check(self.exp_avg, torch.float32, n, "exp_avg", where),
            _check(self.exp_avg_sq, torch.float32, n, "exp_avg_sq", where),
            _check(self.grad, gdt, n, "grad", where),
            _check(self.weight, torch.bfloat16, n, "weight", where),
            _check(self.orig, torch.bfloat16, n, "orig", where),
            _check(self.delta, torch.float32, n, "delta", where),
            n)


def _args(lr, beta1, beta2, eps, weight_decay, step, grad_dtype) -> N.AdamwArgs:
    return N.AdamwArgs(float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                       int(step), int(grad_dtype), 0)


def _grad_dtype(segments: Sequence[AdamwSegment]) -> int:
    kinds = {torch.bfloat16 if s.grad is None else s.grad.dtype for s in segments}
    if len(kinds) > 1:
        raise TypeError("all segments of one call must share the gradient dtype")
    return N.LEMA_GRAD_FP32 if kinds == {torch.float32} else N.LEMA_GRAD_BF16


def adamw_constants(*, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step,
                    grad_dtype=N.LEMA_GRAD_BF16) -> dict:
    """The fp32 constants the kernel uses for this step (host only)."""
    lib = N.load()
    out = N.AdamwConsts()
    N.check(lib.lema_adamw_constants(ctypes.byref(_args(lr, beta1, beta2, eps, weight_decay, step,
                                                        grad_dtype)), ctypes.byref(out)),
            "lema_adamw_constants")
    return {name: np.float32(getattr(out, name)) for name, _ in N.AdamwConsts._fields_}


def _microbatch_pointers(segments, microbatch_grads):
    """Flat nseg * K pointer array of resident micro-batch gradients."""
    if len(microbatch_grads) != len(segments):
        raise ValueError("one list of micro-batch gradients per segment is required")
    ks = {len(g) for g in microbatch_grads}
    if len(ks) != 1:
        raise ValueError("every segment needs the same number of micro-batches")
    k = ks.pop()
    ptrs = []
    for i, (gs, s) in enumerate(zip(microbatch_grads, segments)):
        if s.grad is not None:
            raise ValueError(f"segment {i}: grad must be None with micro-batch gradients")
        ptrs += [_check(g, torch.bfloat16, s.master.numel(), f"microbatch_grads[{i}][{j}]")
                 for j, g in enumerate(gs)]
    return (ctypes.c_void_p * max(1, len(ptrs)))(*ptrs), k


def adamw_step(segments: Sequence[AdamwSegment], *, lr, beta1=0.9, beta2=0.999, eps=1e-8,
               weight_decay=0.01, step, stream=None,
               last_grads: Optional[Sequence[torch.Tensor]] = None,
               microbatch_grads: Optional[Sequence[Sequence[torch.Tensor]]] = None) -> None:
    """One AdamW step over `segments` on the GPU (asynchronous on `stream`).

    With `last_grads` (one bf16 tensor per segment) each segment's grad is an
    fp32 accumulator and the step adds the last micro-batch to it on the fly
    (lema_adamw_step_accum); the accumulator is not updated.  With
    `microbatch_grads` (per segment, the K bf16 micro-batch gradients; the
    segments' grad None) the step sums them in fp32 in order
    (lema_adamw_step_microbatches).
    """
    if microbatch_grads is not None:
        AdamwPlan(segments, microbatch_grads=microbatch_grads).step(
            lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay, step=step,
            stream=stream)
        return
    lib = N.load()
    segs = (N.AdamwSeg * max(1, len(segments)))(*[s.to_c() for s in segments])
    args = _args(lr, beta1, beta2, eps, weight_decay, step, _grad_dtype(segments))
    if last_grads is None:
        N.check(lib.lema_adamw_step(segs, len(segments), ctypes.byref(args),
                                    _stream_handle(stream)), "lema_adamw_step")
        return
    if len(last_grads) != len(segments):
        raise ValueError("one last-micro-batch gradient per segment is required")
    ptrs = (ctypes.c_void_p * max(1, len(segments)))(
        *[_check(g, torch.bfloat16, s.master.numel(), f"last_grads[{i}]")
          for i, (g, s) in enumerate(zip(last_grads, segments))])
    N.check(lib.lema_adamw_step_accum(segs, ptrs, len(segments), ctypes.byref(args),
                                      _stream_handle(stream)), "lema_adamw_step_accum")


def adamw_step_noalloc(segments: Sequence[AdamwSegment], *, lr, beta1=0.9, beta2=0.999,
                       eps=1e-8, weight_decay=0.01, step, stream=None) -> None:
    """adamw_step for callers that cannot allocate device memory
    (lema_adamw_step_noalloc): the launch table goes into the library's fixed
    per-GPU array; at most LEMA_NOALLOC_MAX_SEGMENTS segments, and calls that
    overlap on one GPU from different streams race for that array."""
    lib = N.load()
    segs = (N.AdamwSeg * max(1, len(segments)))(*[s.to_c() for s in segments])
    args = _args(lr, beta1, beta2, eps, weight_decay, step, _grad_dtype(segments))
    N.check(lib.lema_adamw_step_noalloc(segs, len(segments), ctypes.byref(args),
                                        _stream_handle(stream)), "lema_adamw_step_noalloc")


class AdamwPlan:
    """A segment list marshalled once for repeated steps.

    A training loop steps the same tensors every iteration; the plan keeps
    the C descriptor array (and, for the fused mode, the last-micro-batch
    pointer array) so that each step is one call into the library.  The
    tensors must stay alive and in place while the plan is used.
    """

    def __init__(self, segments: Sequence[AdamwSegment],
                 last_grads: Optional[Sequence[torch.Tensor]] = None,
                 microbatch_grads: Optional[Sequence[Sequence[torch.Tensor]]] = None):
        self.lib = N.load()
        self.segments = list(segments)
        self.n = len(self.segments)
        self.c_segs = (N.AdamwSeg * max(1, self.n))(*[s.to_c() for s in self.segments])
        self.grad_dtype = _grad_dtype(self.segments)
        self.microbatch_grads = None if microbatch_grads is None else [list(g) for g in
                                                                       microbatch_grads]
        self.c_mb, self.nmb = (None, 0)
        if self.microbatch_grads is not None:
            self.c_mb, self.nmb = _microbatch_pointers(self.segments, self.microbatch_grads)
        self.last_grads = None if last_grads is None else list(last_grads)
        self.c_last = None
        if self.last_grads is not None:
            if len(self.last_grads) != self.n:
                raise ValueError("one last-micro-batch gradient per segment is required")
            self.c_last = (ctypes.c_void_p * max(1, self.n))(
                *[_check(g, torch.bfloat16, s.master.numel(), f"last_grads[{i}]")
                  for i, (g, s) in enumerate(zip(self.last_grads, self.segments))])

    def step(self, *, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step,
             stream=None) -> None:
        args = _args(lr, beta1, beta2, eps, weight_decay, step, self.grad_dtype)
        if self.c_mb is not None:
            N.check(self.lib.lema_adamw_step_microbatches(self.c_segs, self.c_mb, self.n,
                                                          self.nmb, ctypes.byref(args),
                                                          _stream_handle(stream)),
                    "lema_adamw_step_microbatches")
        elif self.c_last is None:
            N.check(self.lib.lema_adamw_step(self.c_segs, self.n, ctypes.byref(args),
                                             _stream_handle(stream)), "lema_adamw_step")
        else:
            N.check(self.lib.lema_adamw_step_accum(self.c_segs, self.c_last, self.n,
                                                   ctypes.byref(args), _stream_handle(stream)),
                    "lema_adamw_step_accum")


class FlatState:
    """Flat device buffers, one per array kind, holding that array of every
    tensor of a segment list.

    Tensor i's array of kind k is the view of buffer k at the same element
    offset for every kind; offsets are rounded up to `align` elements (256 B
    of fp32), so every view is vector-aligned for the kernels.  This is the
    layout of flat parameter and optimizer-state buffers in ZeRO/FSDP-style
    training.  It also places the arrays that one AdamW launch streams side by
    side a whole buffer apart in HBM; allocating them tensor by tensor instead
    puts one tensor's arrays next to each other, which measured slower on
    MI355X for the same launch (about 1.5% with the step's occupancy cap,
    10-15% at full occupancy).

    The buffer of the k-th kind starts `stagger` * k bytes into an allocation
    that much larger (a multiple of 256 B, so views stay vector-aligned).
    Without it every kind starts at the allocator's large alignment, and one
    tile's accesses to all arrays share their low address bits.  Measured on
    one MI355X (three interleaved runs each), 4 KiB per kind against none:
    the Llama-2-7B attention step 1.386 against 1.409 ms, one rank's share
    of the 7B shape 4.37 against 4.49 ms, 8 resident micro-batches 1.515
    against 1.535 ms; the whole 7B shape the same within the runs' spread;
    the rank-16 LoRA step 0.233 against 0.229 ms.
    """

    def __init__(self, numels: Sequence[int], kinds: dict, device="cuda", align: int = 64,
                 stagger: int = 4096):
        if align < 1:
            raise ValueError("align must be >= 1")
        if stagger < 0 or stagger % 256:
            raise ValueError("stagger must be a non-negative multiple of 256 bytes")
        self.numels = [int(n) for n in numels]
        if any(n < 0 for n in self.numels):
            raise ValueError("numels must be >= 0")
        self.offsets = []
        total = 0
        for n in self.numels:
            self.offsets.append(total)
            total += -(-n // align) * align
        self.total = total
        self.buffers = {}
        for k, (name, dt) in enumerate(kinds.items()):
            shift = k * stagger // torch.empty(0, dtype=dt).element_size()
            self.buffers[name] = torch.empty(total + shift, dtype=dt, device=device)[shift:]

    def __len__(self) -> int:
        return len(self.numels)

    def view(self, kind: str, i: int) -> torch.Tensor:
        o = self.offsets[i]
        return self.buffers[kind][o:o + self.numels[i]]

    def views(self, kind: str) -> list:
        return [self.view(kind, i) for i in range(len(self.numels))]


def flat_adamw_state(numels: Sequence[int], *, grad: Optional[torch.dtype] = torch.bfloat16,
                     delta: bool = False, microbatches: int = 0,
                     device="cuda", stagger: int = 4096) -> tuple[FlatState, list]:
    """AdamW state for tensors of the given sizes in flat buffers.

    Kinds: master, exp_avg, exp_avg_sq (fp32), weight (bf16 output), grad
    (bf16, or the fp32 accumulator; None for no gradient buffer), orig and
    delta when `delta`, and mb0 .. mb{K-1} (bf16) for K resident micro-batch
    gradients.  Returns the buffers and the AdamwSegment list over their
    views; the contents are uninitialised except m and v, which start at 0.
    """
    kinds = {"master": torch.float32, "exp_avg": torch.float32, "exp_avg_sq": torch.float32,
             "weight": torch.bfloat16}
    if grad is not None:
        if grad not in (torch.bfloat16, torch.float32):
            raise TypeError("grad must be torch.bfloat16, torch.float32 or None")
        kinds["grad"] = grad
    if delta:
        kinds["orig"] = torch.bfloat16
        kinds["delta"] = torch.float32
    for k in range(microbatches):
        kinds[f"mb{k}"] = torch.bfloat16
    fs = FlatState(numels, kinds, device=device, stagger=stagger)
    fs.buffers["exp_avg"].zero_()
    fs.buffers["exp_avg_sq"].zero_()
    segs = [AdamwSegment(fs.view("master", i), fs.view("exp_avg", i), fs.view("exp_avg_sq", i),
                         fs.view("grad", i) if grad is not None else None, fs.view("weight", i),
                         fs.view("orig", i) if delta else None,
                         fs.view("delta", i) if delta else None)
            for i in range(len(fs))]
    return fs, segs


@dataclass
class AccumSegment:
    acc: torch.Tensor
    grad: torch.Tensor


def grad_accum(segments: Sequence[AccumSegment], *, overwrite: bool, stream=None) -> None:
    """acc = f32(g) (overwrite) or acc += f32(g) for every segment, on the GPU."""
    lib = N.load()
    cs = []
    for s in segments:
        n = s.acc.numel()
        cs.append(N.AccumSeg(_check(s.acc, torch.float32, n, "acc"),
                             _check(s.grad, torch.bfloat16, n, "grad"), n))
    arr = (N.AccumSeg * max(1, len(cs)))(*cs)
    N.check(lib.lema_grad_accum(arr, len(cs), 1 if overwrite else 0, _stream_handle(stream)),
            "lema_grad_accum")


@dataclass
class MergeSegment:
    base: torch.Tensor       # bf16
    delta: torch.Tensor      # fp32
    merged: torch.Tensor     # bf16 output


def merge_delta(segments: Sequence[MergeSegment], stream=None) -> None:
    """merged = bf16(f32(base) + delta) for every segment, on the GPU."""
    lib = N.load()
    cs = []
    for s in segments:
        n = s.base.numel()
        cs.append(N.MergeSeg(_check(s.base, torch.bfloat16, n, "base"),
                             _check(s.delta, torch.float32, n, "delta"),
                             _check(s.merged, torch.bfloat16, n, "merged"), n))
    arr = (N.MergeSeg * max(1, len(cs)))(*cs)
    N.check(lib.lema_merge_delta(arr, len(cs), _stream_handle(stream)), "lema_merge_delta")


class AccumPlan:
    """An accumulation segment list marshalled once for repeated calls."""

    def __init__(self, segments: Sequence[AccumSegment]):
        self.lib = N.load()
        self.segments = list(segments)
        cs = []
        for s in self.segments:
            n = s.acc.numel()
            cs.append(N.AccumSeg(_check(s.acc, torch.float32, n, "acc"),
                                 _check(s.grad, torch.bfloat16, n, "grad"), n))
        self.n = len(cs)
        self.c_segs = (N.AccumSeg * max(1, self.n))(*cs)

    def run(self, *, overwrite: bool, stream=None) -> None:
        N.check(self.lib.lema_grad_accum(self.c_segs, self.n, 1 if overwrite else 0,
                                         _stream_handle(stream)), "lema_grad_accum")


# ------------------------------------------------- int8 rows with scales

@dataclass
class Q8:
    """An int8 tensor with one fp32 scale per row of ``row_len`` elements
    (README "Quantization": the int8 + per-row-scale storage of quantized
    moments and accumulators; the format is stated in include/lema.h)."""
    codes: torch.Tensor      # int8, numel elements
    scale: torch.Tensor      # fp32, ceil(numel / row_len) row scales
    row_len: int

    @property
    def numel(self) -> int:
        return self.codes.numel()

    @staticmethod
    def rows_of(numel: int, row_len: int) -> int:
        return -(-numel // row_len)

    @classmethod
    def empty(cls, numel: int, row_len: int, device="cuda") -> "Q8":
        return cls(torch.empty(numel, dtype=torch.int8, device=device),
                   torch.empty(cls.rows_of(numel, row_len), dtype=torch.float32, device=device),
                   int(row_len))

    @classmethod
    def zeros(cls, numel: int, row_len: int, device="cuda") -> "Q8":
        """A zero state: codes 0 and scales 0 dequantize to exact zeros."""
        return cls(torch.zeros(numel, dtype=torch.int8, device=device),
                   torch.zeros(cls.rows_of(numel, row_len), dtype=torch.float32, device=device),
                   int(row_len))

    def pointers(self, n: int, name: str, where: str = "cuda"):
        if self.codes.numel() != n:
            raise ValueError(f"{name}: expected {n} codes, got {self.codes.numel()}")
        codes = _check(self.codes, torch.int8, n, f"{name}.codes", where)
        scale = _check(self.scale, torch.float32, self.rows_of(n, self.row_len), f"{name}.scale",
                       where)
        return codes, scale


def _q8_tensors(pairs) -> ctypes.Array:
    cs = []
    for i, (x, q) in enumerate(pairs):
        n = x.numel()
        codes, scale = q.pointers(n, f"q[{i}]")
        cs.append(N.Q8Tensor(_check(x, torch.float32, n, f"x[{i}]"), codes, scale, n, q.row_len))
    return (N.Q8Tensor * max(1, len(cs)))(*cs), len(cs)


def quantize_rows(pairs: Sequence[tuple], stream=None) -> None:
    """For each (x fp32, q Q8): q = quantization of x, on the GPU."""
    arr, n = _q8_tensors(pairs)
    N.check(N.load().lema_quantize_rows(arr, n, _stream_handle(stream)), "lema_quantize_rows")


def dequantize_rows(pairs: Sequence[tuple], stream=None) -> None:
    """For each (x fp32, q Q8): x = dequantization of q, on the GPU."""
    arr, n = _q8_tensors(pairs)
    N.check(N.load().lema_dequantize_rows(arr, n, _stream_handle(stream)),
            "lema_dequantize_rows")


@dataclass
class AdamwQ8Segment:
    """One trainable tensor of the quantized step: int8 moments (Q8) or fp32
    ones, and a bf16 / fp32 gradient tensor or an int8 accumulator (Q8).
    Every Q8 member of a segment shares one row length."""
    master: torch.Tensor
    exp_avg: object              # Q8 or fp32 tensor
    exp_avg_sq: object           # Q8 or fp32 tensor
    grad: object                 # bf16 / fp32 tensor or Q8
    weight: torch.Tensor
    orig: Optional[torch.Tensor] = None
    delta: Optional[torch.Tensor] = None

    def row_len(self) -> int:
        lens = {q.row_len for q in (self.exp_avg, self.exp_avg_sq, self.grad) if isinstance(q, Q8)}
        if len(lens) > 1:
            raise ValueError("the int8 members of one segment must share a row length")
        return lens.pop() if lens else 1

    def kinds(self):
        mom_q8 = isinstance(self.exp_avg, Q8)
        if mom_q8 != isinstance(self.exp_avg_sq, Q8):
            raise TypeError("exp_avg and exp_avg_sq must both be Q8 or both fp32")
        if isinstance(self.grad, Q8):
            gd = N.LEMA_GRAD_Q8
        elif self.grad.dtype == torch.float32:
            gd = N.LEMA_GRAD_FP32
        elif self.grad.dtype == torch.bfloat16:
            gd = N.LEMA_GRAD_BF16
        else:
            raise TypeError(f"grad: expected bfloat16, float32 or Q8, got {self.grad.dtype}")
        return mom_q8, gd

    def to_c(self, where: str = "cuda") -> N.AdamwQ8Seg:
        n = self.master.numel()
        mom_q8, gd = self.kinds()
        if mom_q8:
            m, ms = self.exp_avg.pointers(n, "exp_avg", where)
            v, vs = self.exp_avg_sq.pointers(n, "exp_avg_sq", where)
        else:
            m, ms = _check(self.exp_avg, torch.float32, n, "exp_avg", where), 0
            v, vs = _check(self.exp_avg_sq, torch.float32, n, "exp_avg_sq", where), 0
        if gd == N.LEMA_GRAD_Q8:
            g, gs = self.grad.pointers(n, "grad", where)
        else:
            g, gs = _check(self.grad, self.grad.dtype, n, "grad", where), 0
        return N.AdamwQ8Seg(
            _check(self.master, torch.float32, n, "master", where), m, ms, v, vs, g, gs,
            _check(self.weight, torch.bfloat16, n, "weight", where),
            _check(self.orig, torch.bfloat16, n, "orig", where),
            _check(self.delta, torch.float32, n, "delta", where), n, self.row_len())


def flat_q8_state(numels: Sequence[int], row_lens: Sequence[int], *, grad: str = "bf16",
                  delta: bool = False, device="cuda",
                  stagger: int = 4096) -> tuple[FlatState, FlatState, list]:
    """int8-moment AdamW state for tensors of the given sizes in flat buffers.

    Element kinds: master (fp32), weight (bf16 output), m and v codes (int8),
    the gradient (bf16, or int8 accumulator codes when grad == "q8"), orig and
    delta when `delta`.  Row kinds, in a second FlatState over each tensor's
    row count: the m, v (and accumulator) scales.  Returns both and the
    AdamwQ8Segment list over their views; codes and scales start at zero.
    """
    if grad not in ("bf16", "q8"):
        raise ValueError('grad must be "bf16" or "q8"')
    if len(row_lens) != len(numels):
        raise ValueError("one row length per tensor is required")
    kinds = {"master": torch.float32, "weight": torch.bfloat16, "m": torch.int8,
             "v": torch.int8, "grad": torch.int8 if grad == "q8" else torch.bfloat16}
    if delta:
        kinds["orig"] = torch.bfloat16
        kinds["delta"] = torch.float32
    el = FlatState(numels, kinds, device=device, stagger=stagger)
    rows = [Q8.rows_of(int(n), int(rl)) for n, rl in zip(numels, row_lens)]
    rk = {"m": torch.float32, "v": torch.float32}
    if grad == "q8":
        rk["grad"] = torch.float32
    rw = FlatState(rows, rk, device=device, stagger=stagger)
    for fs in (el, rw):
        for k in rk:
            fs.buffers[k].zero_()
    segs = []
    for i, rl in enumerate(row_lens):
        q = lambda k: Q8(el.view(k, i), rw.view(k, i), int(rl))
        segs.append(AdamwQ8Segment(el.view("master", i), q("m"), q("v"),
                                   q("grad") if grad == "q8" else el.view("grad", i),
                                   el.view("weight", i),
                                   el.view("orig", i) if delta else None,
                                   el.view("delta", i) if delta else None))
    return el, rw, segs


def _q8_call_kinds(segments: Sequence[AdamwQ8Segment]):
    kinds = {s.kinds() for s in segments}
    if len(kinds) > 1:
        raise TypeError("all segments of one call must share moment and gradient dtypes")
    return kinds.pop() if kinds else (True, N.LEMA_GRAD_BF16)


class AdamwQ8Plan:
    """A quantized-step segment list marshalled once for repeated steps."""

    def __init__(self, segments: Sequence[AdamwQ8Segment]):
        self.lib = N.load()
        self.segments = list(segments)
        self.n = len(self.segments)
        self.mom_q8, self.grad_dtype = _q8_call_kinds(self.segments)
        self.c_segs = (N.AdamwQ8Seg * max(1, self.n))(*[s.to_c() for s in self.segments])

    def step(self, *, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step,
             stream=None) -> None:
        args = _args(lr, beta1, beta2, eps, weight_decay, step, self.grad_dtype)
        moments = N.LEMA_STATE_Q8 if self.mom_q8 else N.LEMA_STATE_FP32
        N.check(self.lib.lema_adamw_step_q8(self.c_segs, self.n, ctypes.byref(args), moments,
                                            _stream_handle(stream)), "lema_adamw_step_q8")


def adamw_step_q8(segments: Sequence[AdamwQ8Segment], *, lr, beta1=0.9, beta2=0.999, eps=1e-8,
                  weight_decay=0.01, step, stream=None) -> None:
    """One AdamW step with int8 moments and/or an int8 gradient accumulator
    (README "Quantization"): the int8 arrays are widened within the step."""
    AdamwQ8Plan(segments).step(lr=lr, beta1=beta1, beta2=beta2, eps=eps,
                               weight_decay=weight_decay, step=step, stream=stream)


@dataclass
class AccumQ8Segment:
    acc: Q8
    grad: torch.Tensor           # bf16


class AccumQ8Plan:
    """int8 accumulation segments marshalled once for repeated calls."""

    def __init__(self, segments: Sequence[AccumQ8Segment]):
        self.lib = N.load()
        self.segments = list(segments)
        cs = []
        for i, s in enumerate(self.segments):
            n = s.grad.numel()
            codes, scale = s.acc.pointers(n, f"acc[{i}]")
            cs.append(N.AccumQ8Seg(codes, scale, _check(s.grad, torch.bfloat16, n, f"grad[{i}]"),
                                   n, s.acc.row_len))
        self.n = len(cs)
        self.c_segs = (N.AccumQ8Seg * max(1, self.n))(*cs)

    def run(self, *, overwrite: bool, stream=None) -> None:
        N.check(self.lib.lema_grad_accum_q8(self.c_segs, self.n, 1 if overwrite else 0,
                                            _stream_handle(stream)), "lema_grad_accum_q8")


def grad_accum_q8(segments: Sequence[AccumQ8Segment], *, overwrite: bool, stream=None) -> None:
    """acc = Q(f32(g)) (overwrite) or acc = Q(D(acc) + f32(g)), on the GPU."""
    AccumQ8Plan(segments).run(overwrite=overwrite, stream=stream)


# ------------------------------------------------------------ host memory

class _PinnedBlock:
    """Page-locked host bytes from lema_host_alloc, freed with the last view."""

    def __init__(self, nbytes: int):
        lib = N.load()
        p = ctypes.c_void_p()
        N.check(lib.lema_host_alloc(ctypes.byref(p), max(1, nbytes)), "lema_host_alloc")
        self.ptr = p.value
        self.nbytes = nbytes

    def __del__(self):
        if getattr(self, "ptr", None):
            N.load().lema_host_free(self.ptr)
            self.ptr = None


def pinned_empty(numel: int, dtype: torch.dtype) -> torch.Tensor:
    """Exact-size page-locked host tensor (no power-of-two rounding)."""
    itemsize = torch.empty((), dtype=dtype).element_size()
    block = _PinnedBlock(numel * itemsize)
    raw = (ctypes.c_uint8 * max(1, numel * itemsize)).from_address(block.ptr)
    raw._lema_owner = block                       # keeps the block alive with the buffer
    np_view = np.frombuffer(raw, dtype=np.uint8, count=numel * itemsize)
    return torch.from_numpy(np_view).view(dtype)


# ------------------------------------------------------------ slot stream

class SlotPool:
    """A pool of `nslots` HBM slots of `slot_bytes` each, with its own copy and
    compute streams (default priority), for lema_slot_stream.  With
    duplex=True the slot -> host copies get a third stream of their own.
    In duplex, layer i's upload into slot i mod nslots waits for the
    write-back of the layer that used the slot before; with 3 slots that
    write-back is long done, and on MI355X the whole 7B shape's staged
    duplex step was 2-4% faster than with 2 and its kernels fully hidden."""

    def __init__(self, slot_bytes: int, nslots: int = 2, duplex: bool = False):
        lib = N.load()
        slot_bytes = (int(slot_bytes) + 255) // 256 * 256
        self.region = torch.empty(slot_bytes * nslots, dtype=torch.uint8, device="cuda")
        self.copy_stream = torch.cuda.Stream()
        self.compute_stream = torch.cuda.Stream()
        self.slot_bytes = slot_bytes
        self.nslots = nslots
        h = ctypes.c_void_p()
        torch.cuda.synchronize()
        N.check(lib.lema_slot_pool_create(self.region.data_ptr(), slot_bytes, nslots,
                                          self.copy_stream.cuda_stream,
                                          self.compute_stream.cuda_stream, ctypes.byref(h)),
                "lema_slot_pool_create")
        self.handle = h.value
        self.writeback_stream = None
        if duplex:
            self.writeback_stream = torch.cuda.Stream()
            N.check(lib.lema_slot_pool_set_writeback_stream(self.handle,
                                                            self.writeback_stream.cuda_stream),
                    "lema_slot_pool_set_writeback_stream")

    def stream(self, layers: Sequence[Sequence[AdamwSegment]], *, lr, beta1=0.9, beta2=0.999,
               eps=1e-8, weight_decay=0.01, step, staged: bool = False,
               host_threads: int = 0) -> dict:
        """One AdamW step for every layer, streamed host -> slot -> host.
        Blocks until done; returns the timing statistics.  With staged=True
        the host state may be ordinary or memory-mapped memory, moved through
        the pool's page-locked staging buffers (lema_slot_stream_staged)."""
        lib = N.load()
        keep = []
        c_layers = (N.Layer * max(1, len(layers)))()
        for i, segs in enumerate(layers):
            arr = (N.AdamwSeg * max(1, len(segs)))(*[s.to_c(where="cpu") for s in segs])
            keep.append(arr)
            c_layers[i] = N.Layer(ctypes.cast(arr, ctypes.POINTER(N.AdamwSeg)), len(segs))
        args = _args(lr, beta1, beta2, eps, weight_decay, step, N.LEMA_GRAD_BF16)
        st = N.StreamStats()
        if staged:
            N.check(lib.lema_slot_stream_staged(self.handle, c_layers, len(layers),
                                                ctypes.byref(args), int(host_threads),
                                                ctypes.byref(st)), "lema_slot_stream_staged")
        else:
            N.check(lib.lema_slot_stream(self.handle, c_layers, len(layers), ctypes.byref(args),
                                         ctypes.byref(st)), "lema_slot_stream")
        return {name: getattr(st, name) for name, _ in N.StreamStats._fields_}

    def stream_q8(self, layers: Sequence[Sequence[AdamwQ8Segment]], *, lr, beta1=0.9,
                  beta2=0.999, eps=1e-8, weight_decay=0.01, step, staged: bool = False,
                  host_threads: int = 0) -> dict:
        """The streamed step for quantized host state (lema_slot_stream_q8):
        int8 moments with row scales and/or an int8 accumulator stay
        quantized in host memory.  staged=False needs page-locked host
        tensors; staged=True takes any host memory."""
        lib = N.load()
        keep = []
        kinds = {s.kinds() for segs in layers for s in segs}
        if len(kinds) > 1:
            raise TypeError("all segments of one call must share moment and gradient dtypes")
        mom_q8, gd = kinds.pop() if kinds else (True, N.LEMA_GRAD_BF16)
        c_layers = (N.LayerQ8 * max(1, len(layers)))()
        for i, segs in enumerate(layers):
            arr = (N.AdamwQ8Seg * max(1, len(segs)))(*[s.to_c(where="cpu") for s in segs])
            keep.append(arr)
            c_layers[i] = N.LayerQ8(ctypes.cast(arr, ctypes.POINTER(N.AdamwQ8Seg)), len(segs))
        args = _args(lr, beta1, beta2, eps, weight_decay, step, gd)
        st = N.StreamStats()
        N.check(lib.lema_slot_stream_q8(self.handle, c_layers, len(layers), ctypes.byref(args),
                                        N.LEMA_STATE_Q8 if mom_q8 else N.LEMA_STATE_FP32,
                                        1 if staged else 0, int(host_threads), ctypes.byref(st)),
                "lema_slot_stream_q8")
        return {name: getattr(st, name) for name, _ in N.StreamStats._fields_}

    def close(self):
        if getattr(self, "handle", None):
            N.check(N.load().lema_slot_pool_destroy(self.handle), "lema_slot_pool_destroy")
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------- measurement aids

def measure_copy(src: torch.Tensor, dst: torch.Tensor, nbytes: int, stream=None) -> None:
    N.check(N.load().lema_measure_copy(src.data_ptr(), dst.data_ptr(), int(nbytes),
                                       _stream_handle(stream)), "lema_measure_copy")


def probe_fp32(a: torch.Tensor, b: torch.Tensor, stream=None):
    """(a/b, sqrt(a), bf16(a)) as compiled inside the AdamW kernel."""
    n = a.numel()
    _check(a, torch.float32, n, "a")
    _check(b, torch.float32, n, "b")
    q = torch.empty_like(a)
    r = torch.empty_like(a)
    h = torch.empty(n, dtype=torch.bfloat16, device=a.device)
    N.check(N.load().lema_probe_fp32(a.data_ptr(), b.data_ptr(), q.data_ptr(), r.data_ptr(),
                                     h.data_ptr(), n, _stream_handle(stream)), "lema_probe_fp32")
    return q, r, h


def probe_q8_reciprocal(s: torch.Tensor, stream=None) -> torch.Tensor:
    """The reciprocal the int8 kernels take of each row scale in `s`."""
    n = s.numel()
    _check(s, torch.float32, n, "s")
    r = torch.empty_like(s)
    N.check(N.load().lema_probe_q8_reciprocal(s.data_ptr(), r.data_ptr(), n,
                                              _stream_handle(stream)), "lema_probe_q8_reciprocal")
    return r


def probe_residency(lanes: int, lds_bytes: int, *, per_cu: int = 40, spin_us: int = 20,
                    stream=None) -> dict:
    """How many workgroups of `lanes` lanes with `lds_bytes` of LDS each are
    resident on one compute unit at once (lema_probe_residency): the most
    whose resident intervals overlap on one CU, over a grid of `per_cu`
    workgroups per CU.  Returns that maximum, the minimum over CUs, and the
    number of distinct CUs seen."""
    cus = device_info()["compute_units"]
    n = per_cu * cus
    rec = torch.zeros(3 * n, dtype=torch.int64, device="cuda")
    N.check(N.load().lema_probe_residency(rec.data_ptr(), n, lanes, lds_bytes, spin_us,
                                          _stream_handle(stream)), "lema_probe_residency")
    torch.cuda.synchronize()
    r = rec.view(n, 3).cpu().tolist()
    # a compute unit: its XCC and the HW_ID bits 8..15 (CU, shader array, engine)
    events = {}
    for key, t0, t1 in r:
        cu = (key >> 32, (key >> 8) & 0xFF)
        events.setdefault(cu, []).extend(((t0, 1), (t1, -1)))
    most = []
    for ev in events.values():
        ev.sort(key=lambda e: (e[0], e[1]))      # an end before a start at the same tick
        cur = best = 0
        for _, d in ev:
            cur += d
            best = max(best, cur)
        most.append(best)
    return {"max_per_cu": max(most), "min_per_cu": min(most), "cus_seen": len(events),
            "workgroups": n}


def step_occupancy(kernel: int) -> dict:
    """The occupancy plan of step kernel `kernel` (lema_step_occupancy):
    0 fp32 step, 1 fp32 step on 8 resident micro-batches, 2 int8 step, 3 fp32
    step in launches of fewer than 2^18 tiles."""
    out = (ctypes.c_int32 * 6)()
    N.check(N.load().lema_step_occupancy(kernel, out), "lema_step_occupancy")
    keys = ("lanes", "static_lds", "reserved_lds", "intended_per_cu", "per_cu_by_registers",
            "lds_granule")
    return dict(zip(keys, list(out)))


def table_cache_stats() -> dict:
    """Launch-table cache counters of the current device (since load)."""
    out = (ctypes.c_int64 * 4)()
    N.check(N.load().lema_table_cache_stats(out), "lema_table_cache_stats")
    return {"hits": out[0], "uploads": out[1], "waits": out[2], "entries": out[3]}


def device_info() -> dict:
    lib = N.load()
    cus, tile = ctypes.c_int32(), ctypes.c_int32()
    N.check(lib.lema_device_info(ctypes.byref(cus), ctypes.byref(tile)), "lema_device_info")
    lds, res, res_mb = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    N.check(lib.lema_step_lds_reservation(0, ctypes.byref(lds), ctypes.byref(res)),
            "lema_step_lds_reservation")
    N.check(lib.lema_step_lds_reservation(8, ctypes.byref(lds), ctypes.byref(res_mb)),
            "lema_step_lds_reservation")
    return {"compute_units": cus.value, "tile_elements": tile.value,
            "lds_per_cu": lds.value, "step_lds_reserved": res.value,
            "step_lds_reserved_8_microbatches": res_mb.value}


# ------------------------------------------------------------ checkpoints

_CKPT_DTYPES = {torch.float32: N.LEMA_DT_F32, torch.bfloat16: N.LEMA_DT_BF16,
                torch.int8: N.LEMA_DT_I8}


def _ckpt_array(tensors: Mapping[str, torch.Tensor]):
    arr = (N.CkptTensor * len(tensors))()
    names = []
    for k, (name, t) in enumerate(tensors.items()):
        if t.dtype not in _CKPT_DTYPES:
            raise TypeError(f"{name}: checkpoints hold float32, bfloat16 or int8, not {t.dtype}")
        ptr = _check(t, t.dtype, t.numel(), name, "cuda" if t.is_cuda else "cpu")
        b = name.encode("ascii")
        names.append(b)
        arr[k] = N.CkptTensor(b, _CKPT_DTYPES[t.dtype], 0, ptr, t.numel())
    return arr, names


def save_checkpoint(path, tensors: Mapping[str, torch.Tensor], *, step: int, stream=None) -> None:
    """Write the named tensors (GPU, or host-resident state) and the step to a safetensors file
    (lema_checkpoint_save: written under a temporary name next to `path`,
    flushed, then renamed over it).  Returns once the file is complete."""
    arr, _names = _ckpt_array(tensors)
    N.check(N.load().lema_checkpoint_save(os.fsencode(path), arr, len(arr), int(step),
                                          _stream_handle(stream)), "lema_checkpoint_save")


def load_checkpoint(path, tensors: Mapping[str, torch.Tensor], *, stream=None) -> int:
    """Fill the named tensors (GPU or host) from a safetensors file (each must be
    there with the same dtype and element count) and return its step (-1 if
    it records none).  Returns once the data is in device memory."""
    arr, _names = _ckpt_array(tensors)
    step = ctypes.c_int64(-1)
    N.check(N.load().lema_checkpoint_load(os.fsencode(path), arr, len(arr), ctypes.byref(step),
                                          _stream_handle(stream)), "lema_checkpoint_load")
    return step.value


def checkpoint_tensors(segments, *, prefix: str = "", state: bool = True,
                       delta: bool = False) -> dict:
    """Name -> tensor map of a segment list's checkpoint: with `state`, each
    segment's fp32 master and its moments (fp32 tensors, or int8 codes and
    row scales: "exp_avg.codes", "exp_avg.scale"), with `delta` its delta.
    Segment i's names start with f"{prefix}{i}."."""
    out = {}
    for i, s in enumerate(segments):
        p = f"{prefix}{i}."
        if state:
            out[p + "master"] = s.master
            for name in ("exp_avg", "exp_avg_sq"):
                m = getattr(s, name)
                if isinstance(m, Q8):
                    out[p + name + ".codes"] = m.codes
                    out[p + name + ".scale"] = m.scale
                else:
                    out[p + name] = m
        if delta:
            if s.delta is None:
                raise ValueError(f"segment {i} has no delta")
            out[p + "delta"] = s.delta
    return out
