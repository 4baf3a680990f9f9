"""Host-side checks of the flat state buffers (FlatState, flat_adamw_state,
flat_q8_state): offsets, alignment and views, on CPU tensors.  No kernel runs
here; the GPU parity tests step segments built by the same helpers."""
import pytest
import torch

import optimizer_step_lema_amd as L


def test_offsets_aligned_and_disjoint():
    numels = [5, 64, 0, 130, 1, 4096 * 3 + 5]
    fs = L.FlatState(numels, {"a": torch.float32, "b": torch.bfloat16}, device="cpu")
    assert fs.offsets[0] == 0 and all(o % 64 == 0 for o in fs.offsets)
    for i in range(1, len(numels)):
        assert fs.offsets[i] >= fs.offsets[i - 1] + numels[i - 1]
    assert fs.total >= fs.offsets[-1] + numels[-1] and fs.total % 64 == 0
    for k, esz in (("a", 4), ("b", 2)):
        base = fs.buffers[k].data_ptr()
        for i, n in enumerate(numels):
            v = fs.view(k, i)
            assert v.numel() == n and v.is_contiguous()
            if n == 0:
                continue                       # empty views carry no address
            assert (v.data_ptr() - base) == fs.offsets[i] * esz
            assert (v.data_ptr() - base) % (64 * esz) == 0


def test_kinds_are_staggered():
    kinds = {"a": torch.float32, "b": torch.bfloat16, "c": torch.int8, "d": torch.float32}
    fs = L.FlatState([100, 7], kinds, device="cpu")
    for k, (name, dt) in enumerate(kinds.items()):
        b = fs.buffers[name]
        assert b.numel() == fs.total and b.is_contiguous()
        assert b.storage_offset() * b.element_size() == 4096 * k
    fs0 = L.FlatState([100], kinds, device="cpu", stagger=0)
    assert all(b.storage_offset() == 0 for b in fs0.buffers.values())
    fs1 = L.FlatState([100], kinds, device="cpu", stagger=768)
    assert fs1.buffers["d"].storage_offset() * 4 == 3 * 768
    for bad in (-256, 100, 4097):
        with pytest.raises(ValueError):
            L.FlatState([1], kinds, device="cpu", stagger=bad)


def test_views_share_the_buffer():
    fs = L.FlatState([3, 7], {"x": torch.float32}, device="cpu")
    fs.buffers["x"].zero_()
    fs.view("x", 1).fill_(2.0)
    assert fs.buffers["x"][64:71].eq(2.0).all() and fs.buffers["x"][:64].eq(0).all()


def test_rejects_bad_sizes():
    with pytest.raises(ValueError):
        L.FlatState([-1], {"x": torch.float32}, device="cpu")
    with pytest.raises(ValueError):
        L.FlatState([1], {"x": torch.float32}, device="cpu", align=0)


def test_flat_adamw_state_kinds():
    fs, segs = L.flat_adamw_state([10, 300], delta=True, microbatches=3, device="cpu")
    assert set(fs.buffers) == {"master", "exp_avg", "exp_avg_sq", "weight", "grad", "orig",
                               "delta", "mb0", "mb1", "mb2"}
    assert fs.buffers["grad"].dtype == torch.bfloat16
    for i, s in enumerate(segs):
        assert s.master.numel() == s.weight.numel() == s.delta.numel() == fs.numels[i]
        assert s.exp_avg.eq(0).all() and s.exp_avg_sq.eq(0).all()
    fs2, segs2 = L.flat_adamw_state([10], grad=torch.float32, device="cpu")
    assert segs2[0].grad.dtype == torch.float32 and segs2[0].delta is None
    _, segs3 = L.flat_adamw_state([10], grad=None, device="cpu")
    assert segs3[0].grad is None
    with pytest.raises(TypeError):
        L.flat_adamw_state([10], grad=torch.float16, device="cpu")


def test_flat_q8_state_rows():
    numels, row_lens = [5, 4096 * 3, 0, 130], [5, 4096, 7, 13]
    el, rw, segs = L.flat_q8_state(numels, row_lens, grad="q8", delta=True, device="cpu")
    assert rw.numels == [1, 3, 0, 10]
    for i, s in enumerate(segs):
        assert s.row_len() == row_lens[i]
        assert s.exp_avg.codes.numel() == numels[i] and s.exp_avg.scale.numel() == rw.numels[i]
        assert s.grad.codes.dtype == torch.int8 and s.grad.scale.numel() == rw.numels[i]
        assert s.exp_avg.codes.eq(0).all() and s.exp_avg_sq.scale.eq(0).all()
    _, _, segs_b = L.flat_q8_state([8], [4], device="cpu")
    assert segs_b[0].grad.dtype == torch.bfloat16 and segs_b[0].orig is None
    with pytest.raises(ValueError):
        L.flat_q8_state([8], [4, 4], device="cpu")
