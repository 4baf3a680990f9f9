"""ctypes declarations of liblema.so (include/lema.h, include/lema_measure.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any step in Python.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblema.so")

# Status codes (include/lema.h)
LEMA_OK = 0
LEMA_ERR_NULL = -1
LEMA_ERR_SIZE = -2
LEMA_ERR_HPARAM = -3
LEMA_ERR_DTYPE = -4
LEMA_ERR_OVERLAP = -5
LEMA_ERR_NOT_PINNED = -6
LEMA_ERR_HIP = -7
LEMA_ERR_ALIGN = -8
LEMA_ERR_CAPTURE = -9
LEMA_ERR_IO = -10
LEMA_ERR_NOT_FOUND = -11

LEMA_DT_F32 = 0
LEMA_DT_BF16 = 1
LEMA_DT_I8 = 2

LEMA_GRAD_BF16 = 0
LEMA_GRAD_FP32 = 1
LEMA_GRAD_Q8 = 2

LEMA_STATE_FP32 = 0
LEMA_STATE_Q8 = 1
LEMA_Q8_MAX_ROW = 16384
LEMA_MAX_MICROBATCHES = 16
LEMA_NOALLOC_MAX_SEGMENTS = 1024

vp = ctypes.c_void_p
i32 = ctypes.c_int32
i64 = ctypes.c_int64


class AdamwSeg(ctypes.Structure):
    _fields_ = [("master", vp), ("exp_avg", vp), ("exp_avg_sq", vp), ("grad", vp),
                ("weight_bf16", vp), ("orig_bf16", vp), ("delta", vp), ("numel", i64)]


class AdamwArgs(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double), ("step", i64),
                ("grad_dtype", i32), ("reserved", i32)]


class AdamwConsts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_float) for n in (
        "beta1", "one_minus_beta1", "beta2", "one_minus_beta2",
        "eps", "decay", "step_size", "inv_bias_correction2_root")]


class AccumSeg(ctypes.Structure):
    _fields_ = [("acc", vp), ("grad_bf16", vp), ("numel", i64)]


class MergeSeg(ctypes.Structure):
    _fields_ = [("base_bf16", vp), ("delta", vp), ("merged_bf16", vp), ("numel", i64)]


class AdamwQ8Seg(ctypes.Structure):
    _fields_ = [("master", vp), ("exp_avg", vp), ("exp_avg_scale", vp), ("exp_avg_sq", vp),
                ("exp_avg_sq_scale", vp), ("grad", vp), ("grad_scale", vp), ("weight_bf16", vp),
                ("orig_bf16", vp), ("delta", vp), ("numel", i64), ("row_len", i64)]


class AccumQ8Seg(ctypes.Structure):
    _fields_ = [("acc", vp), ("acc_scale", vp), ("grad_bf16", vp), ("numel", i64),
                ("row_len", i64)]


class Q8Tensor(ctypes.Structure):
    _fields_ = [("x", vp), ("codes", vp), ("scale", vp), ("numel", i64), ("row_len", i64)]


class Layer(ctypes.Structure):
    _fields_ = [("host_segs", ctypes.POINTER(AdamwSeg)), ("nseg", i32)]


class LayerQ8(ctypes.Structure):
    _fields_ = [("host_segs", ctypes.POINTER(AdamwQ8Seg)), ("nseg", i32)]


class CkptTensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("dtype", i32), ("reserved", i32), ("data", vp),
                ("numel", i64)]


class StreamStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_double) for n in (
        "h2d_bytes", "d2h_bytes", "h2d_ms", "d2h_ms", "kernel_ms",
        "copy_busy_ms", "wall_ms", "last_kernel_ms", "host_in_ms", "host_out_ms",
        "call_ms")]


# (name, restype, argtypes) of every exported function
SIGNATURES = [
    ("lema_status_string", ctypes.c_char_p, [i32]),
    ("lema_last_hip_error", i32, []),
    ("lema_version", i32, []),
    ("lema_adamw_constants", i32, [ctypes.POINTER(AdamwArgs), ctypes.POINTER(AdamwConsts)]),
    ("lema_adamw_step", i32, [ctypes.POINTER(AdamwSeg), i32, ctypes.POINTER(AdamwArgs), vp]),
    ("lema_adamw_step_noalloc", i32, [ctypes.POINTER(AdamwSeg), i32, ctypes.POINTER(AdamwArgs),
                                      vp]),
    ("lema_adamw_step_accum", i32, [ctypes.POINTER(AdamwSeg), ctypes.POINTER(vp), i32,
                                    ctypes.POINTER(AdamwArgs), vp]),
    ("lema_adamw_step_microbatches", i32, [ctypes.POINTER(AdamwSeg), ctypes.POINTER(vp), i32, i32,
                                           ctypes.POINTER(AdamwArgs), vp]),
    ("lema_grad_accum", i32, [ctypes.POINTER(AccumSeg), i32, i32, vp]),
    ("lema_merge_delta", i32, [ctypes.POINTER(MergeSeg), i32, vp]),
    ("lema_adamw_step_q8", i32, [ctypes.POINTER(AdamwQ8Seg), i32, ctypes.POINTER(AdamwArgs), i32,
                                 vp]),
    ("lema_grad_accum_q8", i32, [ctypes.POINTER(AccumQ8Seg), i32, i32, vp]),
    ("lema_quantize_rows", i32, [ctypes.POINTER(Q8Tensor), i32, vp]),
    ("lema_dequantize_rows", i32, [ctypes.POINTER(Q8Tensor), i32, vp]),
    ("lema_slot_pool_create", i32, [vp, ctypes.c_size_t, i32, vp, vp, ctypes.POINTER(vp)]),
    ("lema_slot_pool_destroy", i32, [vp]),
    ("lema_slot_pool_set_writeback_stream", i32, [vp, vp]),
    ("lema_slot_stream", i32, [vp, ctypes.POINTER(Layer), i32, ctypes.POINTER(AdamwArgs),
                               ctypes.POINTER(StreamStats)]),
    ("lema_slot_stream_staged", i32, [vp, ctypes.POINTER(Layer), i32, ctypes.POINTER(AdamwArgs),
                                      i32, ctypes.POINTER(StreamStats)]),
    ("lema_slot_stream_q8", i32, [vp, ctypes.POINTER(LayerQ8), i32, ctypes.POINTER(AdamwArgs),
                                  i32, i32, i32, ctypes.POINTER(StreamStats)]),
    ("lema_host_alloc", i32, [ctypes.POINTER(vp), ctypes.c_size_t]),
    ("lema_host_free", i32, [vp]),
    ("lema_checkpoint_save", i32, [ctypes.c_char_p, ctypes.POINTER(CkptTensor), i32, i64, vp]),
    ("lema_checkpoint_load", i32, [ctypes.c_char_p, ctypes.POINTER(CkptTensor), i32,
                                   ctypes.POINTER(i64), vp]),
    ("lema_measure_copy", i32, [vp, vp, ctypes.c_size_t, vp]),
    ("lema_probe_fp32", i32, [vp, vp, vp, vp, vp, i64, vp]),
    ("lema_probe_q8_reciprocal", i32, [vp, vp, i64, vp]),
    ("lema_device_info", i32, [ctypes.POINTER(i32), ctypes.POINTER(i32)]),
    ("lema_step_lds_reservation", i32, [i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]),
    ("lema_probe_residency", i32, [vp, i32, i32, i32, i32, vp]),
    ("lema_step_occupancy", i32, [i32, ctypes.POINTER(i32)]),
    ("lema_table_cache_stats", i32, [ctypes.POINTER(i64)]),
]

_lib = None


def load() -> ctypes.CDLL:
    """Load liblema.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m optimizer_step_lema_amd.build` "
            "(or __graft_entry__.build()); there is no non-HIP fallback")
    import torch  # noqa: F401  -- loads the HIP runtime the library must bind to
    lib = ctypes.CDLL(LIB_PATH)
    for name, res, args in SIGNATURES:
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class LemaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.lema_status_string(status).decode()
        hip = lib.lema_last_hip_error() if status == LEMA_ERR_HIP else 0
        super().__init__(f"{where}: {msg}" + (f" (hipError {hip})" if hip else ""))
        self.status = status
        self.hip_error = hip


def check(status: int, where: str) -> None:
    if status != LEMA_OK:
        raise LemaError(status, where)
