"""GPU tests of the slot-pool streaming engine (lema_slot_stream).

Host-resident fp32 master/m/v and bf16 gradients in page-locked memory are
streamed through two HBM slots; every layer's results, copied back to the
host, must equal the oracle's on the same bytes.  Delays injected on the
copy and compute streams from the host must not change a single bit.
"""
from __future__ import annotations

import threading

import numpy as np
import pytest
import torch

import synth
from parity import compare_bf16, compare_f32, oracle_consts, oracle_segment, to_np

pytestmark = pytest.mark.gpu
HP = synth.HPARAMS
DEV = "cuda"


@pytest.fixture(scope="module")
def L():
    import optimizer_step_lema_amd as lema
    lema.load()
    return lema


def host_layer(L, sizes, seed):
    """One layer of pinned host state plus numpy snapshots of its inputs."""
    segs, snaps = [], []
    for i, n in enumerate(sizes):
        s = 100 * seed + 10 * i
        dev = {"master": synth.normal(n, 0.02, s, DEV), "m": synth.normal(n, 1e-4, s + 1, DEV),
               "v": synth.normal(n, 1e-3, s + 2, DEV).square_(),
               "g": synth.bf16_normal(n, 1e-3, s + 3, DEV)}
        host = {k: L.pinned_empty(n, t.dtype) for k, t in dev.items()}
        for k in dev:
            host[k].copy_(dev[k])
        w = L.pinned_empty(n, torch.bfloat16)
        segs.append(L.AdamwSegment(host["master"], host["m"], host["v"], host["g"], w))
        # copies: to_np of a host tensor is a view, and the stream writes back into it
        snaps.append({"master": to_np(host["master"]).copy(), "m": to_np(host["m"]).copy(),
                      "v": to_np(host["v"]).copy(), "grad": to_np(host["g"]).copy()})
    return segs, snaps


def check_layers(layers, snaps, step, sample=None):
    consts = oracle_consts(HP, step)
    rng = np.random.default_rng(0)
    for li, (segs, sn) in enumerate(zip(layers, snaps)):
        for si, (s, h) in enumerate(zip(segs, sn)):
            n = s.master.numel()
            idx = slice(None) if sample is None or n <= sample else np.unique(
                np.concatenate([np.arange(1024), np.arange(n - 1024, n), rng.integers(0, n, sample)]))
            ref = oracle_segment(h["master"][idx], h["m"][idx], h["v"][idx], h["grad"][idx], consts)
            tag = f"layer{li}.seg{si}"
            compare_f32(to_np(s.master)[idx], ref["master"], tag + ".master")
            compare_f32(to_np(s.exp_avg)[idx], ref["m"], tag + ".m")
            compare_f32(to_np(s.exp_avg_sq)[idx], ref["v"], tag + ".v")
            compare_bf16(to_np(s.weight)[idx], ref["weight"], tag + ".weight")


def layer_bytes(sizes):
    a = lambda x: (x + 255) // 256 * 256
    return sum(a(4 * n) * 3 + a(2 * n) * 2 for n in sizes)


def test_slot_stream_small_layers(L):
    shapes = [[100003, 4096, 2048 * 3 + 1], [777, 65536], [1, 2, 3, 300000], [5000]]
    layers, snaps = zip(*[host_layer(L, s, 10 + i) for i, s in enumerate(shapes)])
    pool = L.SlotPool(max(layer_bytes(s) for s in shapes), nslots=2)
    stats = pool.stream(layers, step=7, **HP)
    check_layers(layers, snaps, 7)
    P = sum(sum(s) for s in shapes)
    assert stats["h2d_bytes"] == 14 * P and stats["d2h_bytes"] == 14 * P
    assert stats["wall_ms"] > 0 and stats["kernel_ms"] > 0
    # a second streamed step on the evolved state, with three slots
    snaps2 = [[{"master": to_np(s.master).copy(), "m": to_np(s.exp_avg).copy(),
                "v": to_np(s.exp_avg_sq).copy(), "grad": to_np(s.grad).copy()} for s in segs]
              for segs in layers]
    pool3 = L.SlotPool(max(layer_bytes(s) for s in shapes), nslots=3)
    pool3.stream(layers, step=8, **HP)
    check_layers(layers, snaps2, 8)
    pool.close()
    pool3.close()


def test_slot_stream_with_injected_delays(L):
    """Long work queued on the pool's copy stream and on its compute stream
    before the call must not change any result (ordering is by events)."""
    shapes = [[1 << 20, 4097], [1 << 20, 4097], [1 << 20, 4097], [1 << 20, 4097]]
    layers, snaps = zip(*[host_layer(L, s, 30 + i) for i, s in enumerate(shapes)])
    pool = L.SlotPool(layer_bytes(shapes[0]), nslots=2)
    big_a = torch.empty(1 << 28, device=DEV)
    big_b = torch.empty(1 << 28, device=DEV)
    x = torch.randn(4096, 4096, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(pool.copy_stream):
        for _ in range(20):
            big_b.copy_(big_a)                       # ~20 ms of copy-stream work
    with torch.cuda.stream(pool.compute_stream):
        for _ in range(10):
            x = x @ x                                # compute-stream work
            x = x / x.norm()
    pool.stream(layers, step=3, **HP)
    check_layers(layers, snaps, 3)
    pool.close()


def test_slot_stream_rejects_pageable_and_oversize(L):
    n = 4096
    pageable = L.AdamwSegment(torch.zeros(n), torch.zeros(n), torch.zeros(n),
                              torch.zeros(n, dtype=torch.bfloat16),
                              torch.zeros(n, dtype=torch.bfloat16))
    pool = L.SlotPool(layer_bytes([n]), nslots=2)
    with pytest.raises(L.LemaError) as e:
        pool.stream([[pageable]], step=1, **HP)
    assert e.value.status == -6                      # LEMA_ERR_NOT_PINNED
    assert torch.count_nonzero(pageable.master) == 0  # nothing ran
    segs, _ = host_layer(L, [2 * n], 77)
    with pytest.raises(L.LemaError) as e:
        pool.stream([segs], step=1, **HP)
    assert e.value.status == -2                      # LEMA_ERR_SIZE: layer exceeds a slot
    pool.close()


def test_slot_stream_llama_layers(L):
    """Three real Llama-2-7B decoder layers (202M params each, 3.24 GB slots),
    every element checked."""
    w = synth.WORKLOADS["llama7b_layer"]
    sizes = w.numels
    layers, snaps = zip(*[host_layer(L, sizes, 50 + i) for i in range(3)])
    pool = L.SlotPool(layer_bytes(sizes), nslots=2)
    stats = pool.stream(layers, step=10, **HP)
    check_layers(layers, snaps, 10)
    h2d_gbps = stats["h2d_bytes"] / (stats["h2d_ms"] * 1e-3) / 1e9
    d2h_gbps = stats["d2h_bytes"] / (stats["d2h_ms"] * 1e-3) / 1e9
    print(f"slot stream 3 Llama layers: H2D {h2d_gbps:.1f} GB/s, D2H {d2h_gbps:.1f} GB/s, "
          f"kernel {stats['kernel_ms']:.2f} ms, wall {stats['wall_ms']:.1f} ms, "
          f"copy busy {stats['copy_busy_ms']:.1f} ms, last kernel {stats['last_kernel_ms']:.3f} ms")
    assert stats["wall_ms"] - stats["copy_busy_ms"] <= 1.05 * stats["last_kernel_ms"] + 1.0
    pool.close()


@pytest.mark.parametrize("nslots", [2, 3])
def test_slot_stream_duplex_writeback(L, nslots):
    """Slot -> host copies on their own stream: both PCIe directions at once.
    Slot reuse then hangs on events alone; results must not change."""
    shapes = [[1 << 20, 4097, 3], [1 << 20, 4097, 3], [5000], [1 << 20, 4097, 3], [1 << 19]]
    layers, snaps = zip(*[host_layer(L, s, 70 + i) for i, s in enumerate(shapes)])
    pool = L.SlotPool(max(layer_bytes(s) for s in shapes), nslots=nslots, duplex=True)
    stats = pool.stream(layers, step=4, **HP)
    check_layers(layers, snaps, 4)
    P = sum(sum(s) for s in shapes)
    assert stats["h2d_bytes"] == 14 * P and stats["d2h_bytes"] == 14 * P
    assert stats["copy_busy_ms"] <= stats["wall_ms"] + 1e-3
    pool.close()


def test_slot_stream_duplex_llama_layers(L):
    """Four real Llama-2-7B layers through 2 slots with the duplex write-back."""
    w = synth.WORKLOADS["llama7b_layer"]
    sizes = w.numels
    layers, snaps = zip(*[host_layer(L, sizes, 90 + i) for i in range(4)])
    pool = L.SlotPool(layer_bytes(sizes), nslots=2, duplex=True)
    stats = pool.stream(layers, step=10, **HP)
    check_layers(layers, snaps, 10)
    h2d_gbps = stats["h2d_bytes"] / (stats["h2d_ms"] * 1e-3) / 1e9
    d2h_gbps = stats["d2h_bytes"] / (stats["d2h_ms"] * 1e-3) / 1e9
    print(f"duplex slot stream 4 Llama layers: H2D {h2d_gbps:.1f} GB/s, D2H {d2h_gbps:.1f} GB/s, "
          f"kernel {stats['kernel_ms']:.2f} ms, wall {stats['wall_ms']:.1f} ms, "
          f"copy busy {stats['copy_busy_ms']:.1f} ms, last kernel {stats['last_kernel_ms']:.3f} ms")
    assert stats["wall_ms"] - stats["copy_busy_ms"] <= 1.05 * stats["last_kernel_ms"] + 1.0
    pool.close()


# --------------------------------------------------- staged (pageable / mmap)

def pageable_layer(sizes, seed, alloc=None):
    """One layer in ordinary (pageable) host memory, or in tensors from alloc(n, dtype)."""
    segs, snaps = [], []
    for i, n in enumerate(sizes):
        s = 100 * seed + 10 * i
        dev = {"master": synth.normal(n, 0.02, s, DEV), "m": synth.normal(n, 1e-4, s + 1, DEV),
               "v": synth.normal(n, 1e-3, s + 2, DEV).square_(),
               "g": synth.bf16_normal(n, 1e-3, s + 3, DEV)}
        make = alloc or (lambda k, dt: torch.empty(k, dtype=dt))
        host = {k: make(n, t.dtype) for k, t in dev.items()}
        for k in dev:
            host[k].copy_(dev[k])
        import optimizer_step_lema_amd as lema
        segs.append(lema.AdamwSegment(host["master"], host["m"], host["v"], host["g"],
                                      make(n, torch.bfloat16)))
        snaps.append({"master": to_np(host["master"]).copy(), "m": to_np(host["m"]).copy(),
                      "v": to_np(host["v"]).copy(), "grad": to_np(host["g"]).copy()})
    return segs, snaps


@pytest.mark.parametrize("duplex,threads,nslots", [(False, 0, 2), (True, 3, 2), (False, 1, 2),
                                                   (False, 0, 3), (True, 2, 3)])
def test_slot_stream_staged_pageable(L, duplex, threads, nslots):
    """Pageable host state through the page-locked staging buffers."""
    shapes = [[100003, 4096, 2048 * 3 + 1], [777, 1 << 20], [1, 2, 3, 300000], [5000],
              [1 << 20, 17]]
    layers, snaps = zip(*[pageable_layer(s, 110 + i) for i, s in enumerate(shapes)])
    pool = L.SlotPool(max(layer_bytes(s) for s in shapes), nslots=nslots, duplex=duplex)
    stats = pool.stream(layers, step=6, staged=True, host_threads=threads, **HP)
    check_layers(layers, snaps, 6)
    P = sum(sum(s) for s in shapes)
    assert stats["h2d_bytes"] == 14 * P and stats["d2h_bytes"] == 14 * P
    assert stats["call_ms"] >= stats["wall_ms"] > 0
    # a second step on the evolved state: the staging buffers are reused
    snaps2 = [[{"master": to_np(s.master).copy(), "m": to_np(s.exp_avg).copy(),
                "v": to_np(s.exp_avg_sq).copy(), "grad": to_np(s.grad).copy()} for s in segs]
              for segs in layers]
    pool.stream(layers, step=7, staged=True, host_threads=threads, **HP)
    check_layers(layers, snaps2, 7)
    pool.close()


def test_slot_stream_staged_memory_mapped(L, tmp_path):
    """Host state in memory-mapped files (the disk tier): results land in the files."""
    files = []

    def mapped(n, dtype):
        np_dtype = {torch.float32: np.float32, torch.bfloat16: np.uint16}[dtype]
        path = tmp_path / f"arr{len(files)}.bin"
        mm = np.memmap(path, dtype=np_dtype, mode="w+", shape=(n,))
        files.append((path, mm))
        t = torch.from_numpy(mm)
        return t.view(torch.bfloat16) if dtype == torch.bfloat16 else t

    shapes = [[65536 * 3 + 5, 4096], [300001], [4096, 4096, 7]]
    layers, snaps = zip(*[pageable_layer(s, 130 + i, alloc=mapped) for i, s in enumerate(shapes)])
    pool = L.SlotPool(max(layer_bytes(s) for s in shapes), nslots=2)
    pool.stream(layers, step=3, staged=True, **HP)
    check_layers(layers, snaps, 3)
    # re-read one array from its file: the update reached the mapped pages
    for _, mm in files:
        mm.flush()
    path0 = files[0][0]
    again = np.fromfile(path0, dtype=np.float32)
    assert np.array_equal(again.view(np.uint32), to_np(layers[0][0].master).view(np.uint32))
    pool.close()


@pytest.mark.parametrize("duplex", [True, False])
def test_slot_stream_staged_llama_layers(L, duplex):
    """Four real Llama-2-7B layers from pageable memory: each direction of a
    layer moves in 45 pieces, more than a ring holds, in groups of 4
    with a ragged last group."""
    w = synth.WORKLOADS["llama7b_layer"]
    sizes = w.numels
    layers, snaps = zip(*[pageable_layer(sizes, 150 + i) for i in range(4)])
    pool = L.SlotPool(layer_bytes(sizes), nslots=2, duplex=duplex)
    stats = pool.stream(layers, step=10, staged=True, **HP)
    check_layers(layers, snaps, 10)
    print(f"staged slot stream 4 Llama layers: call {stats['call_ms']:.1f} ms, GPU span "
          f"{stats['wall_ms']:.1f} ms, host in {stats['host_in_ms']:.1f} ms, host out "
          f"{stats['host_out_ms']:.1f} ms, H2D {stats['h2d_ms']:.1f} ms, D2H {stats['d2h_ms']:.1f} ms, "
          f"kernel {stats['kernel_ms']:.2f} ms")
    pool.close()


@pytest.mark.parametrize("staged,fail_at", [(False, 6), (False, 13), (True, 2), (True, 9)])
def test_injected_copy_failure_then_recovery(L, monkeypatch, staged, fail_at):
    """A copy that fails in the middle of a streamed call (forced from the
    host with LEMA_FAULT_INJECT) returns LEMA_ERR_HIP after the pool's streams
    have drained; the same pool then streams fresh layers correctly and can
    be destroyed."""
    from optimizer_step_lema_amd import _native as N
    shapes = [[5000, 777], [4096], [300, 20000]]
    layers, _ = zip(*[host_layer(L, s, 80 + i) for i, s in enumerate(shapes)])
    pool = L.SlotPool(max(layer_bytes(s) for s in shapes), nslots=2)
    monkeypatch.setenv("LEMA_FAULT_INJECT", f"copy:{fail_at}")
    with pytest.raises(N.LemaError) as e:
        pool.stream(layers, step=3, staged=staged, **HP)
    assert e.value.status == N.LEMA_ERR_HIP and e.value.hip_error != 0
    monkeypatch.delenv("LEMA_FAULT_INJECT")
    layers2, snaps2 = zip(*[host_layer(L, s, 90 + i) for i, s in enumerate(shapes)])
    pool.stream(layers2, step=3, staged=staged, **HP)
    check_layers(layers2, snaps2, 3)
    pool.close()


def _in_fresh_thread(fn):
    """Runs fn on a new thread (whose last-HIP-error slot starts at 0) and
    returns the exception it raised, or None."""
    out = {}

    def run():
        try:
            fn()
        except BaseException as ex:    # handed to the test thread
            out["e"] = ex

    t = threading.Thread(target=run)
    t.start()
    t.join()
    return out.get("e")


HIP_ERROR_UNKNOWN = 999     # what the injected copy failure returns


@pytest.mark.parametrize("duplex,fail_at", [(False, 40), (False, 125), (True, 60), (True, 130)])
def test_staged_failure_mid_stream_then_recovery(L, monkeypatch, duplex, fail_at):
    """A copy that fails while a staged call over real Llama-2-7B layers is
    well under way (each direction of a layer moves in 45 pieces, so both
    rings are full and completion groups are pending in both threads):
    LEMA_ERR_HIP once the streams have drained, with the injected failure's
    raw HIP code on the calling thread whichever of the call's threads hit
    it, then the same pool streams the layers again and every element
    matches the oracle."""
    from optimizer_step_lema_amd import _native as N
    w = synth.WORKLOADS["llama7b_layer"]
    sizes = w.numels
    layers, snaps = zip(*[pageable_layer(sizes, 170 + i) for i in range(3)])
    pool = L.SlotPool(layer_bytes(sizes), nslots=2, duplex=duplex)
    monkeypatch.setenv("LEMA_FAULT_INJECT", f"copy:{fail_at}")
    err = _in_fresh_thread(lambda: pool.stream(layers, step=10, staged=True, **HP))
    assert isinstance(err, N.LemaError), err
    assert err.status == N.LEMA_ERR_HIP and err.hip_error == HIP_ERROR_UNKNOWN
    monkeypatch.delenv("LEMA_FAULT_INJECT")
    layers2, snaps2 = zip(*[pageable_layer(sizes, 180 + i) for i in range(3)])
    pool.stream(layers2, step=10, staged=True, **HP)
    check_layers(layers2, snaps2, 10, sample=20000)    # the full check is the tests above
    pool.close()
