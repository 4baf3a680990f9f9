"""GPU tests of checkpoint files (lema_checkpoint_save / lema_checkpoint_load).

LEMA README, "Features" (interval-based checkpointing of the full
fine-tuning delta with the optimizer states) and "Selective Full
Fine-Tuning" (a checkpoint holds the fp32 delta plus the optimizer state;
training resumes from it; merge_delta turns base + delta into a servable
model).  Files are checked against the safetensors library, an independent
reader and writer of the format, and a resumed run must equal an
uninterrupted one bit for bit.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch
from safetensors import safe_open
from safetensors.torch import load_file, save_file

import oracle
import synth
from parity import to_np

pytestmark = pytest.mark.gpu
HP = synth.HPARAMS
DEV = "cuda"


@pytest.fixture(scope="module")
def L():
    import optimizer_step_lema_amd as lema
    lema.load()
    return lema


def same(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality (NaN payloads included)."""
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def test_save_reads_back_with_safetensors(L, tmp_path):
    """Every dtype, an empty tensor, and a 100 MB tensor that crosses several
    staging buffers: the safetensors library reads the same bytes and the
    step; the file is exactly header + data."""
    t = {"big": synth.normal(25_000_000, 1.0, 3, DEV),
         "w.bf16": synth.bf16_normal(70_001, 1e-3, 4, DEV),
         "codes": torch.randint(-127, 128, (12_345,), dtype=torch.int8, device=DEV),
         "empty": torch.empty(0, device=DEV),
         "tail": synth.normal(3, 1.0, 5, DEV)}
    p = str(tmp_path / "c.safetensors")
    L.save_checkpoint(p, t, step=42)
    assert sorted(os.listdir(tmp_path)) == ["c.safetensors"]
    back = load_file(p)
    assert sorted(back) == sorted(t)
    for k, v in t.items():
        assert same(back[k], v.cpu()), k
    with safe_open(p, "pt") as f:
        assert f.metadata() == {"format": "lema-checkpoint", "step": "42"}
    data_bytes = sum(v.numel() * v.element_size() for v in t.values())
    with open(p, "rb") as f:
        hlen = int.from_bytes(f.read(8), "little")
    assert os.path.getsize(p) == 8 + hlen + data_bytes


def test_load_a_file_written_by_safetensors(L, tmp_path):
    """A file of the safetensors library (other tensors in it, 2-D shapes)
    loads into device buffers bit for bit, with its step."""
    host = {"a": torch.randn(3000, 7), "b": torch.randn(50_000).to(torch.bfloat16),
            "c": torch.randint(-128, 128, (999,), dtype=torch.int8), "unused": torch.ones(4)}
    p = str(tmp_path / "ref.safetensors")
    save_file(host, p, metadata={"step": "7", "note": "from another writer"})
    dev = {"a": torch.empty(21000, device=DEV), "b": torch.empty(50_000, dtype=torch.bfloat16,
                                                                   device=DEV),
           "c": torch.empty(999, dtype=torch.int8, device=DEV)}
    assert L.load_checkpoint(p, dev) == 7
    for k, v in dev.items():
        assert same(v.cpu(), host[k].reshape(-1)), k


def test_failed_load_writes_nothing(L, tmp_path):
    from optimizer_step_lema_amd import _native as N
    p = str(tmp_path / "c.safetensors")
    L.save_checkpoint(p, {"x": torch.ones(10, device=DEV)}, step=1)
    y = torch.full((10,), 5.0, device=DEV)
    z = torch.full((3,), 6.0, device=DEV)
    with pytest.raises(N.LemaError) as e:
        L.load_checkpoint(p, {"x": y, "zz": z})
    assert e.value.status == N.LEMA_ERR_NOT_FOUND
    with pytest.raises(N.LemaError) as e:
        L.load_checkpoint(p, {"x": torch.empty(10, dtype=torch.bfloat16, device=DEV)})
    assert e.value.status == N.LEMA_ERR_DTYPE
    torch.cuda.synchronize()
    assert torch.all(y == 5.0) and torch.all(z == 6.0)


def test_save_replaces_an_earlier_file_only_when_complete(L, tmp_path):
    from optimizer_step_lema_amd import _native as N
    p = str(tmp_path / "c.safetensors")
    L.save_checkpoint(p, {"x": torch.ones(10, device=DEV)}, step=1)
    with pytest.raises(N.LemaError):
        L.save_checkpoint(p, {"x": torch.ones(10, device=DEV), "x\\": torch.ones(1, device=DEV)},
                          step=2)
    assert L.load_checkpoint(p, {"x": torch.empty(10, device=DEV)}) == 1
    L.save_checkpoint(p, {"x": torch.zeros(10, device=DEV)}, step=2)
    assert L.load_checkpoint(p, {"x": torch.empty(10, device=DEV)}) == 2
    assert sorted(os.listdir(tmp_path)) == ["c.safetensors"]


def _fp32_state(L, sizes, seed, delta=False):
    segs = []
    for i, n in enumerate(sizes):
        k = seed + 10 * i
        master = synth.normal(n, 0.02, k, DEV)
        orig = master.to(torch.bfloat16) if delta else None
        segs.append(L.AdamwSegment(master, synth.normal(n, 1e-4, k + 1, DEV),
                                   synth.normal(n, 1e-3, k + 2, DEV).square_(),
                                   torch.empty(n, dtype=torch.bfloat16, device=DEV),
                                   torch.empty(n, dtype=torch.bfloat16, device=DEV),
                                   orig, torch.empty(n, device=DEV) if delta else None))
    return segs


def _blank_like(L, segs):
    """Fresh buffers of the same shapes, filled with garbage."""
    out = []
    for s in segs:
        def junk(t):
            return torch.full_like(t, 7) if t.dtype == torch.int8 else torch.full_like(t, 3.5)

        def q8(m):
            return L.Q8(junk(m.codes), junk(m.scale), m.row_len) if isinstance(m, L.Q8) else junk(m)
        out.append(type(s)(junk(s.master), q8(s.exp_avg), q8(s.exp_avg_sq), s.grad,
                           torch.empty_like(s.weight)))
    return out


@pytest.mark.parametrize("moments", ["fp32", "q8"])
def test_resume_from_checkpoint_is_bit_exact(L, tmp_path, moments):
    """Six steps straight equal three steps, a checkpoint of master, m and v
    (int8 codes and row scales for int8 moments), a load into fresh buffers
    and three more steps, bit for bit; the step number comes back from the
    file."""
    sizes = [4096 * 5, 11008 * 2, 333, 64 * 9]
    row_lens = [4096, 11008, 333, 64]
    grads = [[synth.bf16_normal(n, 1e-3, 700 + 10 * t + i, DEV) for i, n in enumerate(sizes)]
             for t in range(6)]

    def build():
        segs = _fp32_state(L, sizes, 610)
        if moments == "q8":
            q = []
            for s, rl in zip(segs, row_lens):
                m, v = L.Q8.empty(s.master.numel(), rl), L.Q8.empty(s.master.numel(), rl)
                L.quantize_rows([(s.exp_avg, m), (s.exp_avg_sq, v)])
                q.append(L.AdamwQ8Segment(s.master, m, v, s.grad, s.weight))
            segs = q
        return segs

    def run(segs, t):
        for s, g in zip(segs, grads[t]):
            s.grad.copy_(g)
        if moments == "q8":
            L.adamw_step_q8(segs, step=t + 1, **HP)
        else:
            L.adamw_step(segs, step=t + 1, **HP)

    straight = build()
    for t in range(6):
        run(straight, t)
    resumed = build()
    for t in range(3):
        run(resumed, t)
    p = str(tmp_path / "ckpt.safetensors")
    L.save_checkpoint(p, L.checkpoint_tensors(resumed), step=3)
    fresh = _blank_like(L, resumed)
    assert L.load_checkpoint(p, L.checkpoint_tensors(fresh)) == 3
    for t in range(3, 6):
        run(fresh, t)
    torch.cuda.synchronize()
    for a, b in zip(straight, fresh):
        assert same(a.master, b.master) and same(a.weight, b.weight)
        for x, y in ((a.exp_avg, b.exp_avg), (a.exp_avg_sq, b.exp_avg_sq)):
            if moments == "q8":
                assert same(x.codes, y.codes) and same(x.scale, y.scale)
            else:
                assert same(x, y)


def test_delta_checkpoint_feeds_merge_delta(L, tmp_path):
    """A step with delta on; the delta alone is saved (the pages' small
    checkpoint), loaded into a fresh buffer, and merged with the base: the
    same bytes as merging the delta that never left the device, and the
    oracle's merge of the loaded delta."""
    sizes = [4096 * 3 + 7, 2304]
    segs = _fp32_state(L, sizes, 630, delta=True)
    for s, n in zip(segs, sizes):
        s.grad.copy_(synth.bf16_normal(n, 1e-3, 640 + n, DEV))
    L.adamw_step(segs, step=5, **HP)
    p = str(tmp_path / "delta.safetensors")
    L.save_checkpoint(p, L.checkpoint_tensors(segs, state=False, delta=True), step=5)
    loaded = {k: torch.empty_like(v)
              for k, v in L.checkpoint_tensors(segs, state=False, delta=True).items()}
    assert L.load_checkpoint(p, loaded) == 5
    for i, s in enumerate(segs):
        d = loaded[f"{i}.delta"]
        assert same(d, s.delta)
        m1 = torch.empty_like(s.orig)
        m2 = torch.empty_like(s.orig)
        L.merge_delta([L.MergeSegment(s.orig, d, m1), L.MergeSegment(s.orig, s.delta, m2)])
        torch.cuda.synchronize()
        assert same(m1, m2)
        ref = oracle.merge_delta(to_np(s.orig), to_np(d))
        assert np.array_equal(to_np(m1), ref)


def test_concurrent_saves_to_one_path(L, tmp_path):
    """Four threads save different contents to one path at once: each writes
    its own temporary file, the last rename wins, the file is whole (its
    data matches its own step) and no temporary file is left."""
    import threading
    p = str(tmp_path / "c.safetensors")
    xs = [torch.full((1 << 22,), float(k), device=DEV) for k in range(4)]
    torch.cuda.synchronize()
    errs = []

    def run(k):
        try:
            L.save_checkpoint(p, {"x": xs[k]}, step=k)
        except Exception as e:          # reported below
            errs.append(e)

    threads = [threading.Thread(target=run, args=(k,)) for k in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errs
    assert sorted(os.listdir(tmp_path)) == ["c.safetensors"]
    y = torch.empty(1 << 22, device=DEV)
    step = L.load_checkpoint(p, {"x": y})
    assert 0 <= step < 4 and bool(torch.all(y == float(step)))


def test_host_resident_state(L, tmp_path):
    """The host-resident state of a streamed run (page-locked and ordinary
    host tensors) is saved and loaded in place, mixed with device tensors in
    one file."""
    n = 3_000_017
    pinned = L.pinned_empty(n, torch.float32)
    pinned.copy_(torch.randn(n))
    pageable = torch.randn(n // 3).to(torch.bfloat16)
    codes = torch.randint(-127, 128, (12_345,), dtype=torch.int8)
    dev = synth.normal(777, 1.0, 9, DEV)
    p = str(tmp_path / "host.safetensors")
    L.save_checkpoint(p, {"m": pinned, "g": pageable, "c": codes, "d": dev}, step=11)
    back = load_file(p)
    for k, v in (("m", pinned), ("g", pageable), ("c", codes), ("d", dev.cpu())):
        assert same(back[k], v), k
    out = {"m": L.pinned_empty(n, torch.float32), "g": torch.empty(n // 3, dtype=torch.bfloat16),
           "c": torch.empty(12_345, dtype=torch.int8), "d": torch.empty(777, device=DEV)}
    assert L.load_checkpoint(p, out) == 11
    assert same(out["m"], pinned) and same(out["g"], pageable) and same(out["c"], codes)
    assert same(out["d"], dev)
