"""CPU oracle for the mixed-precision AdamW path.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
package ``optimizer_step_lema_amd`` never imports it, and the two share no
code.

Two independent implementations live here:

* ``lema_oracle.c`` (built into ``liblema_oracle.so`` with gcc, no FMA, no
  fast-math, OpenMP over elements), wrapped by the numpy-facing functions
  below;
* ``bruteforce.py``, a per-element loop over numpy float32 scalars, for tiny
  tensors.

What is computed follows the LEMA README ("Quick Start": torch.optim.AdamW
with lr 1e-4; "Selective Full Fine-Tuning": per-layer AdamW over fp32 states
and fp32 gradient accumulation, fp32 delta checkpoint) and the LLMScale
fine-tuning VRAM page (16 bytes per trained parameter: bf16 weight and
gradient, fp32 master, m and v).  The exact rounding points are stated in
``lema_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "lema_oracle.c")
_LIB = os.path.join(_HERE, "liblema_oracle.so")

# gcc flags: every binary32 operation rounded on its own (no contraction into
# FMA, no fast-math, no flush-to-zero), OpenMP for the element loops.
GCC_FLAGS = ["-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-fno-finite-math-only", "-frounding-math", "-fopenmp", "-std=c11"]


def build(verbose: bool = False) -> str:
    """Compile lema_oracle.c into liblema_oracle.so (always recompiles)."""
    cmd = ["gcc", *GCC_FLAGS, "-o", _LIB + ".tmp", _SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    _lib = bind(ctypes.CDLL(_LIB))
    return _lib


def bind(lib):
    """Declare the C signatures on a loaded copy of the oracle library (the
    tests also bind copies built from deliberately altered sources)."""
    i64, f64, i32 = ctypes.c_int64, ctypes.c_double, ctypes.c_int
    vp = ctypes.c_void_p
    lib.oracle_rne16.argtypes = [ctypes.c_float]
    lib.oracle_rne16.restype = ctypes.c_uint16
    lib.oracle_rne16_array.argtypes = [i64, vp, vp]
    lib.oracle_rne16_array.restype = None
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = ctypes.c_float
    lib.oracle_adamw_constants.argtypes = [f64, f64, f64, f64, f64, i64, vp]
    lib.oracle_adamw_constants.restype = None
    lib.oracle_adamw.argtypes = [i64, vp, vp, vp, vp, i32, vp, vp, vp, vp]
    lib.oracle_adamw.restype = None
    lib.oracle_accum.argtypes = [i64, vp, vp, i32]
    lib.oracle_accum.restype = None
    lib.oracle_merge_delta.argtypes = [i64, vp, vp, vp]
    lib.oracle_merge_delta.restype = None
    lib.oracle_quantize_rows.argtypes = [i64, i64, vp, vp, vp]
    lib.oracle_quantize_rows.restype = None
    lib.oracle_dequantize_rows.argtypes = [i64, i64, vp, vp, vp]
    lib.oracle_dequantize_rows.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    lib.oracle_set_num_threads.argtypes = [i32]
    lib.oracle_set_num_threads.restype = None
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(a: np.ndarray, dtype, n: int, name: str, writable: bool = False):
    if a.dtype != dtype or a.ndim != 1 or a.shape[0] != n:
        raise ValueError(f"{name}: expected 1-D {np.dtype(dtype).name}[{n}], "
                         f"got {a.dtype}{list(a.shape)}")
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError(f"{name}: must be contiguous")
    if writable and not a.flags["WRITEABLE"]:
        raise ValueError(f"{name}: must be writable")


def num_threads() -> int:
    """OpenMP threads the C oracle's loops use (OMP_NUM_THREADS governs it)."""
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for later oracle calls (results do not depend on it)."""
    _load().oracle_set_num_threads(int(n))


def rne16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(x.shape[0], dtype=np.uint16)
    _load().oracle_rne16_array(x.shape[0], _ptr(x), _ptr(out))
    return out


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to fp32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def adamw_constants(lr: float, beta1: float, beta2: float, eps: float,
                    weight_decay: float, step: int) -> np.ndarray:
    """The eight fp32 constants of AdamW step number ``step`` (>= 1).

    Order: beta1, 1-beta1, beta2, 1-beta2, eps, 1-lr*wd, lr/(1-beta1^t),
    1/sqrt(1-beta2^t).
    """
    out = np.empty(8, dtype=np.float32)
    _load().oracle_adamw_constants(float(lr), float(beta1), float(beta2),
                                   float(eps), float(weight_decay), int(step),
                                   _ptr(out))
    return out


def adamw_step(master: np.ndarray, m: np.ndarray, v: np.ndarray,
               grad: np.ndarray, consts: np.ndarray,
               orig: np.ndarray | None = None):
    """One AdamW step in place on ``master``, ``m``, ``v`` (fp32, 1-D).

    ``grad`` is uint16 (bf16 patterns) or float32 (an fp32 accumulator).
    Returns ``(weight_bf16, delta)``; ``delta`` is None unless ``orig``
    (uint16 bf16 base weight) is given.
    """
    n = master.shape[0]
    _check(master, np.float32, n, "master", True)
    _check(m, np.float32, n, "m", True)
    _check(v, np.float32, n, "v", True)
    if grad.dtype == np.uint16:
        grad_is_f32 = 0
        _check(grad, np.uint16, n, "grad")
    else:
        grad_is_f32 = 1
        _check(grad, np.float32, n, "grad")
    consts = np.ascontiguousarray(consts, dtype=np.float32)
    assert consts.shape == (8,)
    weight = np.empty(n, dtype=np.uint16)
    delta = None
    if orig is not None:
        _check(orig, np.uint16, n, "orig")
        delta = np.empty(n, dtype=np.float32)
    _load().oracle_adamw(n, _ptr(master), _ptr(m), _ptr(v), _ptr(grad),
                         grad_is_f32, _ptr(weight), _ptr(orig), _ptr(delta),
                         _ptr(consts))
    return weight, delta


def grad_accum(acc: np.ndarray, grad_bf16: np.ndarray, overwrite: bool):
    """acc = f32(g) (overwrite) or acc = acc + f32(g), in place."""
    n = acc.shape[0]
    _check(acc, np.float32, n, "acc", True)
    _check(grad_bf16, np.uint16, n, "grad_bf16")
    _load().oracle_accum(n, _ptr(acc), _ptr(grad_bf16), 1 if overwrite else 0)


def merge_delta(base_bf16: np.ndarray, delta: np.ndarray) -> np.ndarray:
    """Servable bf16 weight: rne16(f32(base) + delta) (README merge_delta)."""
    n = base_bf16.shape[0]
    _check(base_bf16, np.uint16, n, "base")
    _check(delta, np.float32, n, "delta")
    out = np.empty(n, dtype=np.uint16)
    _load().oracle_merge_delta(n, _ptr(base_bf16), _ptr(delta), _ptr(out))
    return out


# ------------------------------------------------- int8 rows with scales

def n_rows(n: int, row_len: int) -> int:
    """Rows of a tensor of n elements cut into rows of row_len (last may be short)."""
    if row_len < 1:
        raise ValueError("row_len must be >= 1")
    return (n + row_len - 1) // row_len


def quantize_rows(x: np.ndarray, row_len: int):
    """fp32 -> (int8 codes, fp32 per-row scales): symmetric absmax, 127 levels.

    LEMA README "Quantization" (int8 + per-row scale for optimizer states and
    accumulators); the exact reading is stated in ``lema_oracle.c``.
    """
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    n = x.shape[0]
    q = np.empty(n, dtype=np.int8)
    scale = np.empty(n_rows(n, row_len), dtype=np.float32)
    _load().oracle_quantize_rows(n, row_len, _ptr(x), _ptr(q), _ptr(scale))
    return q, scale


def dequantize_rows(q: np.ndarray, scale: np.ndarray, row_len: int) -> np.ndarray:
    """(int8 codes, per-row scales) -> fp32: x = f32(q) * scale[row]."""
    n = q.shape[0]
    _check(q, np.int8, n, "q")
    _check(scale, np.float32, n_rows(n, row_len), "scale")
    out = np.empty(n, dtype=np.float32)
    _load().oracle_dequantize_rows(n, row_len, _ptr(q), _ptr(scale), _ptr(out))
    return out


def adamw_step_q8(master: np.ndarray, m, v, grad, consts: np.ndarray, row_len: int,
                  orig: np.ndarray | None = None):
    """One AdamW step with int8 moments and/or an int8 gradient accumulator.

    The step of the README's "Quantization" section: quantized classes are
    dequantized, the ordinary fp32 step (``adamw_step``) runs, and the new
    moments are quantized again.
      master     : fp32, updated in place
      m, v       : each an fp32 array (updated in place) or a tuple
                   (int8 codes, fp32 row scales) whose arrays are overwritten
                   with the requantized moment
      grad       : bf16 patterns (uint16), an fp32 accumulator, or a tuple
                   (int8 codes, fp32 row scales) of a quantized accumulator
    Returns ``(weight_bf16, delta)`` as ``adamw_step``.
    """
    n = master.shape[0]
    moments = []
    for arr in (m, v):
        if isinstance(arr, tuple):
            moments.append(dequantize_rows(arr[0], arr[1], row_len))
        else:
            moments.append(arr)
    if isinstance(grad, tuple):
        grad = dequantize_rows(grad[0], grad[1], row_len)
    m32, v32 = moments
    _check(m32, np.float32, n, "m")
    weight, delta = adamw_step(master, m32, v32, grad, consts, orig=orig)
    for arr, new in ((m, m32), (v, v32)):
        if isinstance(arr, tuple):
            q, s = quantize_rows(new, row_len)
            arr[0][...] = q
            arr[1][...] = s
    return weight, delta


def grad_accum_q8(acc_q: np.ndarray, acc_scale: np.ndarray, grad_bf16: np.ndarray,
                  overwrite: bool, row_len: int) -> None:
    """int8 accumulator += bf16 micro-batch, in place: dequantize, the fp32
    accumulation of ``grad_accum``, quantize again (README "Quantization":
    grad_acc_bits = 8)."""
    n = acc_q.shape[0]
    _check(acc_q, np.int8, n, "acc_q", True)
    if overwrite:
        acc = np.zeros(n, dtype=np.float32)
    else:
        acc = dequantize_rows(acc_q, acc_scale, row_len)
    grad_accum(acc, grad_bf16, overwrite)
    q, s = quantize_rows(acc, row_len)
    acc_q[...] = q
    acc_scale[...] = s
