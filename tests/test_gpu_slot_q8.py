"""GPU tests of slot-pool streaming with quantized host state
(lema_slot_stream_q8).

int8 moments and accumulators are kept as codes plus row scales in host
memory (and the memory-mapped tier) and widened only inside the step (LEMA
README, "Quantization").  Host-resident fp32 master weights, int8
moments with row scales and bf16 gradients (or int8 accumulators) stream
through two HBM slots; every layer's results, copied back to the host, must
equal the oracle's on the same bytes.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import compare_bf16, compare_f32, oracle_consts, to_np

pytestmark = pytest.mark.gpu
HP = synth.HPARAMS
DEV = "cuda"


@pytest.fixture(scope="module")
def L():
    import optimizer_step_lema_amd as lema
    lema.load()
    return lema


def host_tensor(L, a: np.ndarray, pinned: bool) -> torch.Tensor:
    dt = {np.float32: torch.float32, np.int8: torch.int8, np.uint16: torch.int16}[a.dtype.type]
    t = L.pinned_empty(a.size, dt) if pinned else torch.empty(a.size, dtype=dt)
    t.copy_(torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a))
    return t.view(torch.bfloat16) if a.dtype == np.uint16 else t


def q8_layer(L, shapes, seed, *, pinned, grad="bf16"):
    """One layer of host state: segments plus host snapshots of their inputs.
    `shapes` lists (numel, row_len) pairs."""
    segs, snaps = [], []
    for i, (n, rl) in enumerate(shapes):
        s = 1000 * seed + 10 * i
        master = to_np(synth.normal(n, 0.02, s, DEV))
        mq = oracle.quantize_rows(to_np(synth.normal(n, 1e-4, s + 1, DEV)), rl)
        vq = oracle.quantize_rows(to_np(synth.normal(n, 1e-3, s + 2, DEV).square_()), rl)
        if grad == "bf16":
            g = to_np(synth.bf16_normal(n, 1e-3, s + 3, DEV))
            dg = host_tensor(L, g, pinned)
        else:
            g = oracle.quantize_rows(to_np(synth.normal(n, 3e-3, s + 3, DEV)), rl)
            dg = L.Q8(host_tensor(L, g[0], pinned), host_tensor(L, g[1], pinned), rl)
        seg = L.AdamwQ8Segment(
            host_tensor(L, master, pinned),
            L.Q8(host_tensor(L, mq[0], pinned), host_tensor(L, mq[1], pinned), rl),
            L.Q8(host_tensor(L, vq[0], pinned), host_tensor(L, vq[1], pinned), rl),
            dg,
            host_tensor(L, np.zeros(n, np.uint16), pinned))
        segs.append(seg)
        snaps.append({"master": master, "mq": mq, "vq": vq, "g": g, "row_len": rl})
    return segs, snaps


def check_layers(layers, snaps, step):
    consts = oracle_consts(HP, step)
    for li, (segs, sn) in enumerate(zip(layers, snaps)):
        for si, (s, h) in enumerate(zip(segs, sn)):
            master = h["master"].copy()
            m = (h["mq"][0].copy(), h["mq"][1].copy())
            v = (h["vq"][0].copy(), h["vq"][1].copy())
            w, _ = oracle.adamw_step_q8(master, m, v, h["g"], consts, h["row_len"])
            tag = f"layer{li}.seg{si}"
            compare_f32(to_np(s.master), master, tag + ".master")
            compare_bf16(to_np(s.weight), w, tag + ".weight")
            for name, dq, ref in (("m", s.exp_avg, m), ("v", s.exp_avg_sq, v)):
                assert np.array_equal(to_np(dq.codes), ref[0]), f"{tag}.{name}.codes"
                compare_f32(to_np(dq.scale), ref[1], f"{tag}.{name}.scale")


def slot_bytes(shapes, grad="bf16"):
    a = lambda x: (x + 255) // 256 * 256
    total = 0
    for n, rl in shapes:
        rows = -(-n // rl)
        total += a(4 * n) + 2 * (a(n) + a(4 * rows)) + a(2 * n)
        total += a(2 * n) if grad == "bf16" else a(n) + a(4 * rows)
    return total


SHAPES = [[(4096 * 3, 4096), (4096, 4096), (100, 7)], [(11008 * 2 + 5, 11008)],
          [(16 * 300, 16), (2304, 2304)], [(4096 * 5, 4096)]]


@pytest.mark.parametrize("duplex", [False, True])
def test_stream_q8_pinned(L, duplex):
    layers, snaps = zip(*[q8_layer(L, s, 40 + i, pinned=True) for i, s in enumerate(SHAPES)])
    pool = L.SlotPool(max(slot_bytes(s) for s in SHAPES), nslots=2, duplex=duplex)
    stats = pool.stream_q8(layers, step=9, **HP)
    check_layers(layers, snaps, 9)
    # 8 B per parameter each way plus 8 B of scales per row
    P = sum(n for s in SHAPES for n, _ in s)
    R = sum(-(-n // rl) for s in SHAPES for n, rl in s)
    assert stats["h2d_bytes"] == 8 * P + 8 * R
    assert stats["d2h_bytes"] == 8 * P + 8 * R
    pool.close()


def test_stream_q8_staged_pageable_with_q8_accumulators(L):
    """Ordinary (pageable) host memory through the staging buffers, with an
    int8 gradient accumulator as the gradient."""
    layers, snaps = zip(*[q8_layer(L, s, 50 + i, pinned=False, grad="q8")
                          for i, s in enumerate(SHAPES)])
    pool = L.SlotPool(max(slot_bytes(s, "q8") for s in SHAPES), nslots=2)
    stats = pool.stream_q8(layers, step=4, staged=True, host_threads=4, **HP)
    check_layers(layers, snaps, 4)
    assert stats["host_in_ms"] >= 0 and stats["h2d_bytes"] > 0
    # a second step on the evolved host state
    snaps2 = [[{"master": to_np(s.master).copy(),
                "mq": (to_np(s.exp_avg.codes).copy(), to_np(s.exp_avg.scale).copy()),
                "vq": (to_np(s.exp_avg_sq.codes).copy(), to_np(s.exp_avg_sq.scale).copy()),
                "g": (to_np(s.grad.codes).copy(), to_np(s.grad.scale).copy()),
                "row_len": h["row_len"]} for s, h in zip(segs, sn)]
              for segs, sn in zip(layers, snaps)]
    pool.stream_q8(layers, step=5, staged=True, **HP)
    check_layers(layers, snaps2, 5)
    pool.close()


def test_stream_q8_rejects(L):
    from optimizer_step_lema_amd import _native as N
    shapes = [(4096, 4096)]
    layers, _ = zip(q8_layer(L, shapes, 60, pinned=False))
    pool = L.SlotPool(slot_bytes(shapes), nslots=2)
    with pytest.raises(N.LemaError) as e:
        pool.stream_q8(layers, step=1, **HP)                 # pageable without staging
    assert e.value.status == N.LEMA_ERR_NOT_PINNED
    small = L.SlotPool(slot_bytes(shapes) - 256, nslots=2)
    with pytest.raises(N.LemaError) as e:
        small.stream_q8(layers, step=1, staged=True, **HP)   # layer does not fit
    assert e.value.status == N.LEMA_ERR_SIZE
    with pytest.raises(N.LemaError) as e:
        pool.stream_q8(layers, step=1, staged=True, host_threads=999, **HP)
    assert e.value.status == N.LEMA_ERR_SIZE
    pool.close()
    small.close()


@pytest.mark.parametrize("duplex", [True, False])
def test_stream_q8_llama_layers_staged(L, duplex):
    """Two Llama-2-7B decoder layers (404.8 M params) of int8 host state,
    staged, every element checked.  A piece spans adjacent arrays of the
    slot (master, codes, row scales and gradient of a segment going in), so
    pieces mix 4-byte, 1-byte and row-scale arrays."""
    w = synth.WORKLOADS["llama7b_layer"]
    shapes = [(n, sh[-1]) for n, (_, sh) in zip(w.numels, w.segments)]
    layers, snaps = zip(*[q8_layer(L, shapes, 70 + i, pinned=False) for i in range(2)])
    pool = L.SlotPool(slot_bytes(shapes), nslots=2, duplex=duplex)
    stats = pool.stream_q8(layers, step=w.step, staged=True, **HP)
    check_layers(layers, snaps, w.step)
    assert stats["kernel_ms"] > 0
    pool.close()


def test_stream_q8_injected_copy_failure(L, monkeypatch):
    """The int8 pipeline's failure exit: LEMA_ERR_HIP, then the pool works."""
    from optimizer_step_lema_amd import _native as N
    layers, _ = zip(*[q8_layer(L, s, 80 + i, pinned=True) for i, s in enumerate(SHAPES)])
    pool = L.SlotPool(max(slot_bytes(s) for s in SHAPES), nslots=2)
    monkeypatch.setenv("LEMA_FAULT_INJECT", "copy:9")
    with pytest.raises(N.LemaError) as e:
        pool.stream_q8(layers, step=2, **HP)
    assert e.value.status == N.LEMA_ERR_HIP
    monkeypatch.delenv("LEMA_FAULT_INJECT")
    layers2, snaps2 = zip(*[q8_layer(L, s, 90 + i, pinned=True) for i, s in enumerate(SHAPES)])
    pool.stream_q8(layers2, step=2, **HP)
    check_layers(layers2, snaps2, 2)
    pool.close()
