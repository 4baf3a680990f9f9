"""The whole Llama-2-7B shape resident in HBM (291 tensors, 6,738,415,616
parameters, ~148 GB with delta), stepped once exactly as bench.py times it
(flat state, one lema_adamw_step launch, t = 10, delta on), and compared with
the oracle on EVERY element of every output, segment by segment.

The inputs of each segment are copied to host memory before the call (16 B
per parameter, 108 GB in all); after the call each segment's outputs come
back one at a time and are compared with the oracle run on that segment's
snapshot, which is then freed.  Bar: bit-exact for every output (the bf16
weight, and fp32 master, m, v and delta), which implies the 2e-6 relative
bound; any bit mismatch is re-checked with the element-wise comparison of
tests/parity.py to name it.  The sampled test in test_gpu_parity.py is the
fast check of the same workload."""
from __future__ import annotations

import time

import numpy as np
import pytest
import torch

import synth
from parity import compare_bf16, compare_f32, oracle_consts, oracle_segment, to_np

pytestmark = pytest.mark.gpu

HP = synth.HPARAMS


def _same_bits(got: np.ndarray, ref: np.ndarray) -> bool:
    return got.shape == ref.shape and np.array_equal(got.view(np.uint8), ref.view(np.uint8))


@pytest.mark.timeout(900)
def test_llama7b_full_every_element():
    import optimizer_step_lema_amd as L

    w = synth.WORKLOADS["llama7b_full"]
    t0 = time.perf_counter()
    _, segs = L.flat_adamw_state(w.numels, delta=True, device="cuda")
    snaps = []
    for i, s in enumerate(segs):
        st = synth.make_segment_state(w, i, "cuda", with_orig=True)
        s.master.copy_(st["master"])
        s.exp_avg.copy_(st["m"])
        s.exp_avg_sq.copy_(st["v"])
        s.grad.copy_(st["grads"][0])
        s.orig.copy_(st["orig"])
        del st
        snaps.append({"master": to_np(s.master), "m": to_np(s.exp_avg),
                      "v": to_np(s.exp_avg_sq), "grad": to_np(s.grad), "orig": to_np(s.orig)})
        if i % 64 == 0:
            print(f"full 7B: snapshot of segment {i}/{len(segs)} ({time.perf_counter() - t0:.0f} s)",
                  flush=True)
    L.AdamwPlan(segs).step(step=w.step, **HP)
    torch.cuda.synchronize()
    print(f"full 7B: stepped ({time.perf_counter() - t0:.0f} s)", flush=True)

    consts = oracle_consts(HP, w.step)
    checked = 0
    for i, s in enumerate(segs):
        b = snaps[i]
        ref = oracle_segment(b["master"], b["m"], b["v"], b["grad"], consts, b["orig"])
        tag = f"7b seg{i} {w.segments[i][0]}"
        for got, name, kind in ((s.master, "master", "f"), (s.exp_avg, "m", "f"),
                                (s.exp_avg_sq, "v", "f"), (s.weight, "weight", "b"),
                                (s.delta, "delta", "f")):
            g = to_np(got)
            if not _same_bits(g, ref[name]):
                if kind == "f":
                    compare_f32(g, ref[name], f"{tag}.{name}")
                else:
                    compare_bf16(g, ref[name], f"{tag}.{name}")
            checked += g.size
        snaps[i] = None
        if i % 64 == 0:
            print(f"full 7B: segment {i}/{len(segs)} equal ({time.perf_counter() - t0:.0f} s)",
                  flush=True)
    assert checked == 5 * w.params
    print(f"full 7B: {checked} output elements bit-exact ({time.perf_counter() - t0:.0f} s)",
          flush=True)


@pytest.mark.timeout(900)
def test_llama7b_full_q8_every_element():
    """The whole 7B shape with int8 moments (rows = the weights' last
    dimension, one fp32 scale per row), bf16 gradient and delta, in the flat
    int8 state bench.py --q8 times, one lema_adamw_step_q8 call: every
    output element compared with the oracle, segment by segment (master,
    weight and delta bit for bit, every int8 code as an integer, every row
    scale bit for bit).  Host snapshots: 10 B per parameter, 67 GB."""
    import oracle
    import optimizer_step_lema_amd as L

    w = synth.WORKLOADS["llama7b_full"]
    row_lens = [shape[-1] for _, shape in w.segments]
    t0 = time.perf_counter()
    _, _, segs = L.flat_q8_state(w.numels, row_lens, grad="bf16", delta=True, device="cuda")
    snaps = []
    for i, s in enumerate(segs):
        st = synth.make_segment_state(w, i, "cuda", with_orig=True)
        s.master.copy_(st["master"])
        L.quantize_rows([(st["m"], s.exp_avg), (st["v"], s.exp_avg_sq)])
        s.grad.copy_(st["grads"][0])
        s.orig.copy_(st["orig"])
        del st
        snaps.append({"master": to_np(s.master), "grad": to_np(s.grad), "orig": to_np(s.orig),
                      "m": (to_np(s.exp_avg.codes), to_np(s.exp_avg.scale)),
                      "v": (to_np(s.exp_avg_sq.codes), to_np(s.exp_avg_sq.scale))})
        if i % 64 == 0:
            print(f"full 7B q8: snapshot of segment {i}/{len(segs)} "
                  f"({time.perf_counter() - t0:.0f} s)", flush=True)
    L.AdamwQ8Plan(segs).step(step=w.step, **HP)
    torch.cuda.synchronize()
    print(f"full 7B q8: stepped ({time.perf_counter() - t0:.0f} s)", flush=True)

    consts = oracle_consts(HP, w.step)
    checked = 0
    for i, (s, rl) in enumerate(zip(segs, row_lens)):
        b = snaps[i]
        master = b["master"].copy()
        wref, dref = oracle.adamw_step_q8(master, b["m"], b["v"], b["grad"], consts, rl,
                                          orig=b["orig"])
        tag = f"7b q8 seg{i} {w.segments[i][0]}"
        for got, ref, name, kind in ((s.master, master, "master", "f"),
                                     (s.weight, wref, "weight", "b"),
                                     (s.delta, dref, "delta", "f"),
                                     (s.exp_avg.scale, b["m"][1], "m.scale", "f"),
                                     (s.exp_avg_sq.scale, b["v"][1], "v.scale", "f")):
            g = to_np(got)
            if not _same_bits(g, ref):
                if kind == "f":
                    compare_f32(g, ref, f"{tag}.{name}")
                else:
                    compare_bf16(g, ref, f"{tag}.{name}")
            checked += g.size if name in ("master", "weight", "delta") else 0
        for got, ref, name in ((s.exp_avg.codes, b["m"][0], "m.codes"),
                               (s.exp_avg_sq.codes, b["v"][0], "v.codes")):
            bad = int(np.count_nonzero(to_np(got) != ref))
            assert bad == 0, f"{tag}.{name}: {bad} int8 codes differ"
            checked += ref.size
        snaps[i] = None
        if i % 64 == 0:
            print(f"full 7B q8: segment {i}/{len(segs)} equal ({time.perf_counter() - t0:.0f} s)",
                  flush=True)
    assert checked == 5 * w.params
    print(f"full 7B q8: {checked} output elements and every row scale bit-exact "
          f"({time.perf_counter() - t0:.0f} s)", flush=True)
