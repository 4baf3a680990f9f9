"""Helpers of the GPU parity tests: run the HIP path and the oracle on the
same bytes and compare element by element.

Bar (per element): the bf16 weight is bit-exact (NaN compared as a class);
fp32 master, m, v, delta and accumulators are within 2e-6 relative of the
oracle and exactly equal where the oracle value is zero.  The library is
designed to be bit-exact on every output (same operation order, no FMA,
correctly rounded sqrt and division on both sides), so the tests also count
fp32 bit mismatches and require none.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

REL_TOL = 2e-6


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def compare_f32(got: np.ndarray, ref: np.ndarray, name: str, exact: bool = True) -> dict:
    got = np.asarray(got, np.float32)
    ref = np.asarray(ref, np.float32)
    assert got.shape == ref.shape, name
    gn, rn = np.isnan(got), np.isnan(ref)
    assert np.array_equal(gn, rn), f"{name}: NaN positions differ ({int((gn != rn).sum())})"
    keep = ~rn
    g, r = got[keep].astype(np.float64), ref[keep].astype(np.float64)
    inf = np.isinf(r)
    assert np.array_equal(g[inf], r[inf]), f"{name}: infinities differ"
    fin = ~inf
    err = np.abs(g[fin] - r[fin])
    bound = REL_TOL * np.abs(r[fin])
    bad = err > bound
    assert not bad.any(), (f"{name}: {int(bad.sum())} elements beyond 2e-6 relative; worst "
                           f"{err[bad].max():.3e} at ref {r[fin][bad][np.argmax(err[bad])]:.6e}")
    bits = int((got[keep].view(np.uint32) != ref[keep].view(np.uint32)).sum())
    if exact:
        assert bits == 0, f"{name}: {bits} fp32 bit mismatches (within tolerance)"
    return {"n": int(got.size), "bit_mismatches": bits}


def compare_bf16(got: np.ndarray, ref: np.ndarray, name: str) -> None:
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    gn = (got & 0x7FFF) > 0x7F80
    rn = (ref & 0x7FFF) > 0x7F80
    assert np.array_equal(gn, rn), f"{name}: NaN positions differ"
    diff = int((got[~rn] != ref[~rn]).sum())
    assert diff == 0, f"{name}: {diff} bf16 mismatches"


def oracle_consts(hp: dict, step: int) -> np.ndarray:
    return oracle.adamw_constants(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                                  hp["weight_decay"], step)


def oracle_segment(master, m, v, grad, consts, orig=None):
    """Oracle step on host copies (numpy); returns dict of outputs."""
    master, m, v = master.copy(), m.copy(), v.copy()
    wb, delta = oracle.adamw_step(master, m, v, np.ascontiguousarray(grad), consts,
                                  orig=None if orig is None else np.ascontiguousarray(orig))
    return {"master": master, "m": m, "v": v, "weight": wb, "delta": delta}
