"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every test compares element by element on the same seeded bytes: the inputs
are drawn on the GPU (synth), copied to the host for the oracle, then the
GPU runs the step in place.  See tests/parity.py for the bar.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (compare_bf16, compare_f32, oracle_consts, oracle_segment, to_np)

pytestmark = pytest.mark.gpu
HP = synth.HPARAMS
DEV = "cuda"


@pytest.fixture(scope="module")
def L():
    import optimizer_step_lema_amd as lema
    lema.load()
    return lema


def _f32(n, sigma, seed, offset=0, square=False):
    t = synth.normal(n + offset, sigma, seed, DEV)
    if square:
        t.mul_(t)
    return t[offset:]


def _bf16(n, sigma, seed, offset=0):
    return synth.normal(n + offset, sigma, seed, DEV).to(torch.bfloat16)[offset:]


def _empty(n, dtype, offset=0):
    return torch.empty(n + offset, dtype=dtype, device=DEV)[offset:]


def build_segments(L, sizes, seed, *, grad_f32=False, delta=(), offset=0, fresh=False,
                   grad_sigma=1e-3):
    """Device segments plus host snapshots of their inputs."""
    segs, snaps = [], []
    for i, n in enumerate(sizes):
        s = seed * 1000 + 10 * i
        master = _f32(n, 0.02, s + 0, offset)
        if fresh:
            m = torch.zeros(n + offset, device=DEV)[offset:]
            v = torch.zeros(n + offset, device=DEV)[offset:]
        else:
            m = _f32(n, 1e-4, s + 1, offset)
            v = _f32(n, 1e-3, s + 2, offset, square=True)
        grad = _f32(n, 3e-3, s + 3, offset) if grad_f32 else _bf16(n, grad_sigma, s + 3, offset)
        weight = _empty(n, torch.bfloat16, offset)
        orig = dl = None
        if delta == "all" or i in delta:
            orig = master.to(torch.bfloat16)
            if offset:
                o2 = _empty(n, torch.bfloat16, offset)
                o2.copy_(orig)
                orig = o2
            dl = _empty(n, torch.float32, offset)
        segs.append(L.AdamwSegment(master, m, v, grad, weight, orig, dl))
        snaps.append({"master": to_np(master), "m": to_np(m), "v": to_np(v), "grad": to_np(grad),
                      "orig": None if orig is None else to_np(orig)})
    return segs, snaps


def check_segments(segs, snaps, consts, label=""):
    for i, (s, h) in enumerate(zip(segs, snaps)):
        ref = oracle_segment(h["master"], h["m"], h["v"], h["grad"], consts, h["orig"])
        tag = f"{label}seg{i}(n={s.master.numel()})"
        compare_f32(to_np(s.master), ref["master"], tag + ".master")
        compare_f32(to_np(s.exp_avg), ref["m"], tag + ".m")
        compare_f32(to_np(s.exp_avg_sq), ref["v"], tag + ".v")
        compare_bf16(to_np(s.weight), ref["weight"], tag + ".weight")
        if s.delta is not None:
            compare_f32(to_np(s.delta), ref["delta"], tag + ".delta")


# ------------------------------------------------------------ primitives

def test_fp32_primitives_are_ieee(L):
    """Division, sqrt and bf16 rounding as compiled in the kernel vs the host's IEEE ops."""
    rng = np.random.default_rng(0)
    n = 1 << 22
    a_bits = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    b_bits = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    # structured cases: subnormals, near-one, powers of two, rounding ties for bf16
    k = 1 << 16
    a_bits[:k] = rng.integers(0, 1 << 23, k)                       # positive subnormals
    b_bits[k:2 * k] = rng.integers(0, 1 << 23, k)                  # subnormal divisors
    a_bits[2 * k:3 * k] = (0x3F800000 + rng.integers(-4096, 4096, k)).astype(np.uint32)
    a_bits[3 * k:4 * k] = (rng.integers(0, 1 << 16, k) << 16 | 0x8000).astype(np.uint32)
    a = a_bits.view(np.float32)
    b = b_bits.view(np.float32)
    q, r, h = L.probe_fp32(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV))
    with np.errstate(all="ignore"):
        q_ref = a / b
        r_ref = np.sqrt(a)
    compare_f32(to_np(q), q_ref, "a/b")
    compare_f32(to_np(r), r_ref, "sqrt(a)")
    compare_bf16(to_np(h), oracle.rne16(a), "bf16(a)")


# ---------------------------------------------------------- ragged lists

RAGGED = [0, 1, 3, 4, 5, 7, 8, 9, 255, 256, 257, 1023, 1024, 1025, 2047, 2048, 2049, 4095,
          4096, 4097, 100003, 3 * 65536 + 17]


@pytest.mark.parametrize("offset", [0, 1, 3])
@pytest.mark.parametrize("grad_f32", [False, True])
def test_ragged_segments(L, offset, grad_f32):
    delta = {i for i in range(len(RAGGED)) if i % 2 == 0}
    segs, snaps = build_segments(L, RAGGED, 7 + offset, grad_f32=grad_f32, delta=delta,
                                 offset=offset)
    L.adamw_step(segs, step=37, **HP)
    torch.cuda.synchronize()
    check_segments(segs, snaps, oracle_consts(HP, 37))


def test_many_segments_with_empty_ones(L):
    """300 segments of mixed sizes in one call, empty ones in between: the
    binary search over the launch table's tile prefix sums finds each."""
    rng = np.random.default_rng(3)
    sizes = [int(x) for x in rng.choice([0, 1, 17, 2048, 5000, 40000], size=300)]
    segs, snaps = build_segments(L, sizes, 11, delta=set(range(0, 300, 3)))
    L.adamw_step(segs, step=5, **HP)
    torch.cuda.synchronize()
    check_segments(segs, snaps, oracle_consts(HP, 5))


@pytest.mark.parametrize("hp", [dict(HP, lr=0.0), dict(HP, beta1=0.0, beta2=0.0),
                                dict(HP, lr=3e-3, weight_decay=0.1, eps=1e-6)])
def test_hyperparameter_variants(L, hp):
    segs, snaps = build_segments(L, [4096 * 3 + 5, 777], 21, delta="all")
    L.adamw_step(segs, step=3, **hp)
    torch.cuda.synchronize()
    check_segments(segs, snaps, oracle_consts(hp, 3))


def test_special_values(L):
    """NaN, infinities, subnormals and signed zeros flow as in the oracle."""
    n = 4096 + 19
    segs, snaps = build_segments(L, [n], 31, delta="all")
    s = segs[0]
    specials = torch.tensor([float("nan"), float("inf"), -float("inf"), 0.0, -0.0, 1e-40, -1e-42,
                             3.4e38], device=DEV)
    k = len(specials)
    for t, stride in ((s.master, 3), (s.exp_avg, 5), (s.exp_avg_sq, 7)):
        t[1:1 + k * stride:stride] = specials
    s.exp_avg_sq.abs_()                          # the caller keeps v >= 0
    pats = np.array([0x7FC0, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x8001, 0x7F7F], np.uint16)
    gb = torch.from_numpy(pats.view(np.int16)).to(DEV).view(torch.bfloat16)
    s.grad[2:2 + 11 * k:11] = gb
    snaps[0] = {"master": to_np(s.master), "m": to_np(s.exp_avg), "v": to_np(s.exp_avg_sq),
                "grad": to_np(s.grad), "orig": to_np(s.orig)}
    L.adamw_step(segs, step=2, **HP)
    torch.cuda.synchronize()
    check_segments(segs, snaps, oracle_consts(HP, 2))


def test_golden_fixture(L):
    import json
    import os
    doc = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "adamw_small.json")))
    hp = doc["hyperparameters"]

    def arr(hx):
        if len(hx[0]) == 8:
            return torch.tensor(np.array([int(h, 16) for h in hx], np.uint32).view(np.int32),
                                device=DEV).view(torch.float32)
        return torch.tensor(np.array([int(h, 16) for h in hx], np.uint16).view(np.int16),
                            device=DEV).view(torch.bfloat16)

    case = doc["cases"][0]
    ins, exp = case["inputs"], case["expect"]
    sizes = doc["segment_sizes"]
    full = {k: arr(v) for k, v in ins.items()}
    outs_w = torch.empty(sum(sizes), dtype=torch.bfloat16, device=DEV)
    outs_d = torch.empty(sum(sizes), dtype=torch.float32, device=DEV)
    segs, o = [], 0
    for n in sizes:
        sl = slice(o, o + n)
        segs.append(L.AdamwSegment(full["master"][sl], full["m"][sl], full["v"][sl],
                                   full["grad"][sl], outs_w[sl], full["orig"][sl], outs_d[sl]))
        o += n
    L.adamw_step(segs, step=case["step"], **hp)
    torch.cuda.synchronize()
    for name, t in (("master", full["master"]), ("m", full["m"]), ("v", full["v"]),
                    ("delta", outs_d)):
        compare_f32(to_np(t), to_np(arr(exp[name])), name)
    compare_bf16(to_np(outs_w), to_np(arr(exp["weight"])), "weight")

    # the accumulated-gradient case: three micro-batches then an fp32-grad step
    case = doc["cases"][1]
    ins, exp = case["inputs"], case["expect"]
    acc = torch.empty(sum(sizes), dtype=torch.float32, device=DEV)
    for k, mb in enumerate(ins["micro_batches"]):
        L.grad_accum([L.AccumSegment(acc, arr(mb))], overwrite=(k == 0))
    torch.cuda.synchronize()
    compare_f32(to_np(acc), to_np(arr(exp["acc"])), "acc")
    master, m, v = arr(ins["master"]), arr(ins["m"]), arr(ins["v"])
    w = torch.empty(sum(sizes), dtype=torch.bfloat16, device=DEV)
    L.adamw_step([L.AdamwSegment(master, m, v, acc, w)], step=case["step"], **hp)
    torch.cuda.synchronize()
    for name, t in (("master", master), ("m", m), ("v", v)):
        compare_f32(to_np(t), to_np(arr(exp[name])), "acc-case " + name)
    compare_bf16(to_np(w), to_np(arr(exp["weight"])), "acc-case weight")


# ------------------------------------------------------------ accumulation

@pytest.mark.parametrize("offset", [0, 1])
def test_accumulation_eight_microbatches(L, offset):
    sizes = [1, 2048, 2049, 65536 + 3, 0, 300001]
    accs = [_empty(n, torch.float32, offset) for n in sizes]
    grads = [[_bf16(n, 1e-3, 500 + 10 * i + k, offset) for i, n in enumerate(sizes)]
             for k in range(8)]
    grads[0][1][:4] = torch.tensor([-0.0, 0.0, float("inf"), -1e-40], device=DEV).to(torch.bfloat16)
    for k in range(8):
        L.grad_accum([L.AccumSegment(a, g) for a, g in zip(accs, grads[k])], overwrite=(k == 0))
        if k == 0:
            torch.cuda.synchronize()
            assert to_np(accs[1]).view(np.uint32)[0] == 0x80000000      # -0 kept
    torch.cuda.synchronize()
    for i, n in enumerate(sizes):
        ref = np.empty(n, np.float32)
        oracle.grad_accum(ref, to_np(grads[0][i]), overwrite=True)
        for k in range(1, 8):
            oracle.grad_accum(ref, to_np(grads[k][i]), overwrite=False)
        compare_f32(to_np(accs[i]), ref, f"acc{i}")


@pytest.mark.parametrize("offset", [0, 1])
def test_fused_last_microbatch(L, offset):
    """Step on acc + f32(last) in one pass == accumulate(last) then step, bit for bit;
    the accumulator itself is left untouched."""
    sizes = [5, 256, 257, 4097, 100003, 0, 3 * 65536 + 17]
    segs, _ = build_segments(L, sizes, 81, grad_f32=True, delta={0, 3, 4}, offset=offset)
    lasts = [_bf16(n, 1e-3, 7000 + i, offset) for i, n in enumerate(sizes)]
    twin = _clone_segs(L, segs)
    acc_before = [to_np(s.grad).copy() for s in segs]
    snaps = [{"master": to_np(s.master), "m": to_np(s.exp_avg), "v": to_np(s.exp_avg_sq),
              "orig": None if s.orig is None else to_np(s.orig)} for s in segs]
    L.adamw_step(segs, step=9, last_grads=lasts, **HP)
    # the two-call path on the twin
    L.grad_accum([L.AccumSegment(t.grad, g) for t, g in zip(twin, lasts)], overwrite=False)
    L.adamw_step(twin, step=9, **HP)
    torch.cuda.synchronize()
    consts = oracle_consts(HP, 9)
    for i, (s, t) in enumerate(zip(segs, twin)):
        assert np.array_equal(to_np(s.grad).view(np.uint32), acc_before[i].view(np.uint32))
        g = acc_before[i].copy()
        oracle.grad_accum(g, to_np(lasts[i]), overwrite=False)
        ref = oracle_segment(snaps[i]["master"], snaps[i]["m"], snaps[i]["v"], g, consts,
                             snaps[i]["orig"])
        tag = f"fused seg{i}"
        compare_f32(to_np(s.master), ref["master"], tag + ".master")
        compare_f32(to_np(s.exp_avg), ref["m"], tag + ".m")
        compare_f32(to_np(s.exp_avg_sq), ref["v"], tag + ".v")
        compare_bf16(to_np(s.weight), ref["weight"], tag + ".weight")
        if s.delta is not None:
            compare_f32(to_np(s.delta), ref["delta"], tag + ".delta")
        for f in ("master", "exp_avg", "exp_avg_sq", "weight"):
            assert _same(getattr(s, f), getattr(t, f)), (i, f)


# ------------------------------------------------------------ merge delta

@pytest.mark.parametrize("offset", [0, 1, 2])
def test_merge_delta_ragged(L, offset):
    sizes = [0, 1, 3, 255, 256, 257, 4097, 100003]
    bases = [_bf16(n, 0.02, 8100 + i, offset) for i, n in enumerate(sizes)]
    deltas = [_f32(n, 1e-4, 8200 + i, offset) for i, n in enumerate(sizes)]
    deltas[7][:6] = torch.tensor([float("nan"), float("inf"), -float("inf"), 0.0, -0.0, 1e-42],
                                 device=DEV)
    outs = [_empty(n, torch.bfloat16, offset) for n in sizes]
    L.merge_delta([L.MergeSegment(b, d, o) for b, d, o in zip(bases, deltas, outs)])
    torch.cuda.synchronize()
    for i, (b, d, o) in enumerate(zip(bases, deltas, outs)):
        compare_bf16(to_np(o), oracle.merge_delta(to_np(b), to_np(d)), f"merge{i}")


def test_merge_delta_reproduces_step_weight(L):
    """A step's delta merged onto its base gives the step's bf16 weight back
    wherever the subtraction was exact (README merge_delta), and equals the
    oracle's merge everywhere."""
    w = synth.WORKLOADS["llama7b_attn_last4"]
    segs = _workload_segments(L, w, True)[:4]
    L.adamw_step(segs, step=w.step, **HP)
    merged = [torch.empty_like(s.weight) for s in segs]
    L.merge_delta([L.MergeSegment(s.orig, s.delta, m) for s, m in zip(segs, merged)])
    torch.cuda.synchronize()
    for i, (s, m) in enumerate(zip(segs, merged)):
        b = to_np(s.orig)
        d = to_np(s.delta)
        got = to_np(m)
        compare_bf16(got, oracle.merge_delta(b, d), f"merge{i}")
        wgt = to_np(s.weight)
        base = oracle.bf16_to_f32(b).astype(np.float64)
        new = to_np(s.master).astype(np.float64)
        exact = (np.sign(new) == np.sign(base)) & (np.abs(new) <= 2 * np.abs(base)) & \
                (np.abs(base) <= 2 * np.abs(new))
        assert exact.mean() > 0.99
        assert np.array_equal(got[exact], wgt[exact])
    del segs
    torch.cuda.empty_cache()


# ------------------------------------------------------- invariances

def _clone_segs(L, segs):
    out = []
    for s in segs:
        out.append(L.AdamwSegment(s.master.clone(), s.exp_avg.clone(), s.exp_avg_sq.clone(),
                                  s.grad.clone(), torch.empty_like(s.weight),
                                  None if s.orig is None else s.orig.clone(),
                                  None if s.delta is None else torch.empty_like(s.delta)))
    return out


def _same(a, b):
    return torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a.view(torch.int16),
                       b.view(torch.int32) if b.dtype == torch.float32 else b.view(torch.int16))


def test_resume_invariance(L):
    """P11: T steps straight == T1 steps, host round trip of the state, T-T1 steps."""
    sizes = [5000, 2048 * 7, 333]
    segs, _ = build_segments(L, sizes, 41)
    twin = _clone_segs(L, segs)
    grads = [[_bf16(n, 1e-3, 900 + 10 * t + i) for i, n in enumerate(sizes)] for t in range(6)]
    for t in range(6):
        for s, g in zip(segs, grads[t]):
            s.grad.copy_(g)
        L.adamw_step(segs, step=t + 1, **HP)
    for t in range(6):
        if t == 2:   # checkpoint: state to the host and back into fresh buffers
            torch.cuda.synchronize()
            host = [(s.master.cpu(), s.exp_avg.cpu(), s.exp_avg_sq.cpu()) for s in twin]
            twin = [L.AdamwSegment(h[0].to(DEV), h[1].to(DEV), h[2].to(DEV), s.grad,
                                   torch.empty_like(s.weight)) for h, s in zip(host, twin)]
        for s, g in zip(twin, grads[t]):
            s.grad.copy_(g)
        L.adamw_step(twin, step=t + 1, **HP)
    torch.cuda.synchronize()
    for a, b in zip(segs, twin):
        for x, y in ((a.master, b.master), (a.exp_avg, b.exp_avg), (a.exp_avg_sq, b.exp_avg_sq),
                     (a.weight, b.weight)):
            assert _same(x, y)


def test_split_permute_pack_invariance(L):
    """P12: one call == per-segment calls == permuted == split == packed == unaligned views."""
    sizes = [768 * 2304, 2304, 4099, 1]
    segs, _ = build_segments(L, sizes, 51, delta="all")
    variants = {k: _clone_segs(L, segs) for k in ("one", "each", "perm", "split", "packed")}
    L.adamw_step(variants["one"], step=1, **HP)
    for s in variants["each"]:
        L.adamw_step([s], step=1, **HP)
    L.adamw_step(list(reversed(variants["perm"])), step=1, **HP)
    halves = []
    for s in variants["split"]:
        h = s.master.numel() // 2
        for sl in (slice(0, h), slice(h, None)):
            halves.append(L.AdamwSegment(s.master[sl], s.exp_avg[sl], s.exp_avg_sq[sl], s.grad[sl],
                                         s.weight[sl], s.orig[sl], s.delta[sl]))
    L.adamw_step([x for x in halves if x.master.numel() > 0], step=1, **HP)
    # packed: W and b of the first "layer" in one contiguous buffer, one descriptor
    p = variants["packed"]
    cat = lambda a, b: torch.cat([a, b])
    packed = L.AdamwSegment(cat(p[0].master, p[1].master), cat(p[0].exp_avg, p[1].exp_avg),
                            cat(p[0].exp_avg_sq, p[1].exp_avg_sq), cat(p[0].grad, p[1].grad),
                            torch.empty(sizes[0] + sizes[1], dtype=torch.bfloat16, device=DEV),
                            cat(p[0].orig, p[1].orig),
                            torch.empty(sizes[0] + sizes[1], device=DEV))
    L.adamw_step([packed] + p[2:], step=1, **HP)
    torch.cuda.synchronize()
    ref = variants["one"]
    for name in ("each", "perm", "split"):
        for a, b in zip(ref, variants[name]):
            for f in ("master", "exp_avg", "exp_avg_sq", "weight", "delta"):
                assert _same(getattr(a, f), getattr(b, f)), (name, f)
    for f in ("master", "exp_avg", "exp_avg_sq", "weight", "delta"):
        assert _same(cat(getattr(ref[0], f), getattr(ref[1], f)), getattr(packed, f)), f


def test_rank_shards_equal_whole_call(L):
    """Data-parallel ownership: eight calls, call k over rank k's contiguous
    eighth of every tensor (views; where numel % 8 != 0 the ranks after the
    first start unaligned), give the same bytes as one call over the whole
    tensors, which itself matches the oracle."""
    sizes = [4096 * 4096, 11008 * 512, 4096, 4096 * 3 + 5, 13, 7]
    segs, snaps = build_segments(L, sizes, 61, delta="all")
    sharded = _clone_segs(L, segs)
    L.adamw_step(segs, step=10, **HP)
    for k in range(8):
        views = []
        for s in sharded:
            b, e = synth.shard_range(s.master.numel(), 8, k)
            if e > b:
                sl = slice(b, e)
                views.append(L.AdamwSegment(s.master[sl], s.exp_avg[sl], s.exp_avg_sq[sl],
                                            s.grad[sl], s.weight[sl], s.orig[sl], s.delta[sl]))
        L.adamw_step(views, step=10, **HP)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(segs, sharded)):
        for f in ("master", "exp_avg", "exp_avg_sq", "weight", "delta"):
            assert _same(getattr(a, f), getattr(b, f)), (i, f)
    check_segments(segs[2:], snaps[2:], oracle_consts(HP, 10), "whole ")


def _fill_flat(segs, sizes, seed):
    snaps = []
    for i, (s, n) in enumerate(zip(segs, sizes)):
        k = seed + 10 * i
        s.master.copy_(_f32(n, 0.02, k))
        s.exp_avg.copy_(_f32(n, 1e-4, k + 1))
        s.exp_avg_sq.copy_(_f32(n, 1e-3, k + 2, square=True))
        if s.grad is not None:
            s.grad.copy_(_bf16(n, 1e-3, k + 3))
        if s.orig is not None:
            s.orig.copy_(s.master.to(torch.bfloat16))
        snaps.append({"master": to_np(s.master), "m": to_np(s.exp_avg), "v": to_np(s.exp_avg_sq),
                      "grad": None if s.grad is None else to_np(s.grad),
                      "orig": None if s.orig is None else to_np(s.orig)})
    return snaps


FLAT_SIZES = [70001, 4096, 5, 1, 0, 3 * 4096 + 5, 256]


def test_flat_state_step_matches_oracle(L):
    """Segments that are views of flat per-kind buffers (flat_adamw_state):
    ragged sizes including an empty tensor, delta on, every element."""
    fs, segs = L.flat_adamw_state(FLAT_SIZES, delta=True, device=DEV)
    snaps = _fill_flat(segs, FLAT_SIZES, 71000)
    L.adamw_step(segs, step=7, **HP)
    torch.cuda.synchronize()
    check_segments(segs, snaps, oracle_consts(HP, 7), "flat ")


def test_flat_state_resident_microbatches(L):
    """Flat state with three resident micro-batch gradient buffers, stepped
    through an AdamwPlan: K accumulations then the step, bit for bit."""
    K = 3
    fs, segs = L.flat_adamw_state(FLAT_SIZES, grad=None, delta=True, microbatches=K, device=DEV)
    snaps = _fill_flat(segs, FLAT_SIZES, 72000)
    mbs = []
    for i, n in enumerate(FLAT_SIZES):
        views = [fs.view(f"mb{k}", i) for k in range(K)]
        for k, v in enumerate(views):
            v.copy_(_bf16(n, 1e-3, 72500 + 10 * i + k))
        mbs.append(views)
    L.AdamwPlan(segs, microbatch_grads=mbs).step(step=12, **HP)
    torch.cuda.synchronize()
    c = oracle_consts(HP, 12)
    for i, (seg, h, gs) in enumerate(zip(segs, snaps, mbs)):
        if FLAT_SIZES[i] == 0:
            continue
        ref = _accumulate_then_step(h, [to_np(g) for g in gs], c, h["orig"])
        compare_f32(to_np(seg.master), ref["master"], f"flat mb seg{i}.master")
        compare_f32(to_np(seg.exp_avg), ref["m"], f"flat mb seg{i}.m")
        compare_f32(to_np(seg.exp_avg_sq), ref["v"], f"flat mb seg{i}.v")
        compare_bf16(to_np(seg.weight), ref["weight"], f"flat mb seg{i}.weight")
        compare_f32(to_np(seg.delta), ref["delta"], f"flat mb seg{i}.delta")


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")   # the refusal leaves it empty
def test_rejects_graph_capture(L):
    """A stream capturing a HIP graph is refused before anything is enqueued:
    the launch tables live in a cache a captured graph would outlive."""
    from optimizer_step_lema_amd import _native as N
    segs, snaps = build_segments(L, [4099], 96)
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(N.LemaError) as e:
        with torch.cuda.graph(graph, stream=side):
            L.adamw_step(segs, step=3, **HP)
    assert e.value.status == N.LEMA_ERR_CAPTURE
    torch.cuda.synchronize()
    # nothing ran: the state is still the input, and an ordinary call works
    assert np.array_equal(to_np(segs[0].master).view(np.uint32), snaps[0]["master"].view(np.uint32))
    L.adamw_step(segs, step=3, **HP)
    torch.cuda.synchronize()
    check_segments(segs, snaps, oracle_consts(HP, 3), "after capture ")


def test_concurrent_host_threads(L):
    """Eight host threads, each with its own stream and segment list, call the
    library at once (ctypes releases the GIL, so the calls really overlap in
    the launch-table cache); every thread's five steps must match the oracle."""
    import threading
    groups = [build_segments(L, [4099 + 64 * i, 300, 70001], 200 + i, delta="all")
              for i in range(8)]
    streams = [torch.cuda.Stream() for _ in groups]
    torch.cuda.synchronize()
    errors = []

    def worker(i):
        try:
            segs, _ = groups[i]
            for t in range(1, 6):
                L.adamw_step(segs, step=t, stream=streams[i], **HP)
        except Exception as e:  # reported below
            errors.append((i, e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(groups))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (segs, snaps) in enumerate(groups):
        for s, h in zip(segs, snaps):
            master, m, v = h["master"].copy(), h["m"].copy(), h["v"].copy()
            for t in range(1, 6):
                ref = oracle_segment(master, m, v, h["grad"], oracle_consts(HP, t), h["orig"])
                master, m, v = ref["master"], ref["m"], ref["v"]
            tag = f"thread{i} n={s.master.numel()}"
            compare_f32(to_np(s.master), ref["master"], tag + ".master")
            compare_f32(to_np(s.exp_avg), ref["m"], tag + ".m")
            compare_f32(to_np(s.exp_avg_sq), ref["v"], tag + ".v")
            compare_bf16(to_np(s.weight), ref["weight"], tag + ".weight")
            compare_f32(to_np(s.delta), ref["delta"], tag + ".delta")


def test_step_lds_reservation(L):
    """The step reserves LDS it does not use, in whole allocation granules,
    so that 12 of its workgroups (9 with >= 4 resident micro-batches) share
    a CU (test_gpu_occupancy.py measures the counts)."""
    info = L.device_info()
    lds, res, res_mb = info["lds_per_cu"], info["step_lds_reserved"], \
        info["step_lds_reserved_8_microbatches"]
    g = L.step_occupancy(0)["lds_granule"]
    assert lds >= 64 * 1024, info
    assert res % g == 0 and res_mb % g == 0 and res_mb <= 65536, info
    assert lds // res == 12 and lds // res_mb == 9, info


def test_plans_match_direct_calls(L):
    """AdamwPlan / AccumPlan (arguments marshalled once) == the direct calls."""
    sizes = [4099, 256, 70001]
    segs, _ = build_segments(L, sizes, 91, grad_f32=True, delta={1})
    twin = _clone_segs(L, segs)
    lasts = [_bf16(n, 1e-3, 9100 + i) for i, n in enumerate(sizes)]
    plan = L.AdamwPlan(segs)
    fused = L.AdamwPlan(segs, last_grads=lasts)
    acc_plan = L.AccumPlan([L.AccumSegment(s.grad, g) for s, g in zip(segs, lasts)])
    for t in (1, 2, 3):
        plan.step(step=t, **HP)
        L.adamw_step(twin, step=t, **HP)
    fused.step(step=4, **HP)
    L.adamw_step(twin, step=4, last_grads=lasts, **HP)
    acc_plan.run(overwrite=False)
    L.grad_accum([L.AccumSegment(s.grad, g) for s, g in zip(twin, lasts)], overwrite=False)
    torch.cuda.synchronize()
    for a, b in zip(segs, twin):
        for f in ("master", "exp_avg", "exp_avg_sq", "grad", "weight"):
            assert _same(getattr(a, f), getattr(b, f)), f
        if a.delta is not None:
            assert _same(a.delta, b.delta)


# Tables of more than 2048 bytes go through the device cache; smaller ones
# travel in the kernel arguments.  The cache tests pad every call with
# PAD_SEGS one-element segments of their own tensor so that each table is
# large enough for the cache.
PAD_SEGS = 25


def _pad_segments(L, pad):
    return [L.AdamwSegment(pad.master[k:k + 1], pad.exp_avg[k:k + 1], pad.exp_avg_sq[k:k + 1],
                           pad.grad[k:k + 1], pad.weight[k:k + 1]) for k in range(PAD_SEGS)]


def test_table_cache_many_lists_and_streams(L):
    """More distinct segment lists than cached tables, alternating two streams.

    Call j steps a prefix of segment j % 3 whose length shrinks with j, so
    nearly every call has a table of its own and the cache must evict."""
    s2 = torch.cuda.Stream()
    base, snaps = build_segments(L, [3000, 70001, 2048, PAD_SEGS], 61)
    pad = _pad_segments(L, base[3])
    calls = []
    before = L.table_cache_stats()
    for j in range(48):
        i = j % 3
        n = base[i].master.numel() - (j % 24)
        b = base[i]
        seg = L.AdamwSegment(b.master[:n], b.exp_avg[:n], b.exp_avg_sq[:n], b.grad[:n],
                             b.weight[:n])
        extra = [] if j % 5 else [L.AdamwSegment(base[(i + 1) % 3].master[:7],
                                                 base[(i + 1) % 3].exp_avg[:7],
                                                 base[(i + 1) % 3].exp_avg_sq[:7],
                                                 base[(i + 1) % 3].grad[:7],
                                                 base[(i + 1) % 3].weight[:7])]
        if j % 2:
            s2.wait_stream(torch.cuda.current_stream())
            L.adamw_step([seg] + extra + pad, step=j + 1, stream=s2, **HP)
            torch.cuda.current_stream().wait_stream(s2)
        else:
            L.adamw_step([seg] + extra + pad, step=j + 1, **HP)
        calls.append(([(i, n)] + ([((i + 1) % 3, 7)] if extra else []) + [(3, PAD_SEGS)], j + 1))
    after = L.table_cache_stats()
    assert after["hits"] + after["uploads"] - before["hits"] - before["uploads"] == 48
    torch.cuda.synchronize()
    state = [{k: h[k].copy() for k in ("master", "m", "v", "grad")} for h in snaps]
    for w in state:
        w["w"] = None
    wout = [np.zeros(len(h["master"]), np.uint16) for h in snaps]
    touched = [np.zeros(len(h["master"]), bool) for h in snaps]
    for items, t in calls:
        c = oracle_consts(HP, t)
        for i, n in items:
            st = state[i]
            out = oracle_segment(st["master"][:n], st["m"][:n], st["v"][:n], st["grad"][:n], c)
            st["master"][:n], st["m"][:n], st["v"][:n] = out["master"], out["m"], out["v"]
            wout[i][:n] = out["weight"]
            touched[i][:n] = True
    for i, s in enumerate(base):
        compare_f32(to_np(s.master), state[i]["master"], f"cache seg{i} master")
        compare_f32(to_np(s.exp_avg_sq), state[i]["v"], f"cache seg{i} v")
        compare_bf16(to_np(s.weight)[touched[i]], wout[i][touched[i]], f"cache seg{i} weight")


def test_table_cache_beyond_capacity(L):
    """More distinct tables than the cache may hold (512): 600 back-to-back
    calls on prefixes of one tensor, each its own table, with no host wait in
    between, so that the cache both grows and, at its cap, reuses entries whose
    launches have finished.  Results follow the oracle's sequence of steps."""
    base, snaps = build_segments(L, [4096, PAD_SEGS], 62)
    b = base[0]
    pad = _pad_segments(L, base[1])
    lengths = [4096 - j for j in range(600)]
    before = L.table_cache_stats()
    for j, n in enumerate(lengths):
        seg = L.AdamwSegment(b.master[:n], b.exp_avg[:n], b.exp_avg_sq[:n], b.grad[:n],
                             b.weight[:n])
        L.adamw_step([seg] + pad, step=j + 1, **HP)
    torch.cuda.synchronize()
    after = L.table_cache_stats()
    assert after["hits"] + after["uploads"] - before["hits"] - before["uploads"] == 600
    assert after["entries"] <= 512
    sts = [{k: h[k].copy() for k in ("master", "m", "v", "grad")} for h in snaps]
    for j, n in enumerate(lengths):
        for st, k in ((sts[0], n), (sts[1], PAD_SEGS)):
            out = oracle_segment(st["master"][:k], st["m"][:k], st["v"][:k], st["grad"][:k],
                                 oracle_consts(HP, j + 1))
            st["master"][:k], st["m"][:k], st["v"][:k] = out["master"], out["m"], out["v"]
    for t, st, tag in ((b, sts[0], "cache cap"), (base[1], sts[1], "cache cap pad")):
        compare_f32(to_np(t.master), st["master"], tag + " master")
        compare_f32(to_np(t.exp_avg), st["m"], tag + " m")
        compare_f32(to_np(t.exp_avg_sq), st["v"], tag + " v")


# The largest launch table carried in the kernel arguments is 2048 bytes:
# 24 segment records (a 128-byte tile prefix and 24 x 80 bytes), or, for the
# step over 8 resident micro-batches, 13 records with their pointer lists.
@pytest.mark.parametrize("nseg", [24, 25])
def test_tables_in_kernel_arguments_and_in_cache(L, nseg):
    """The step, the accumulation and the merge on 24 segments (table in the
    kernel arguments, cache untouched) and on 25 (table through the cache):
    every element equals the oracle's either way."""
    rng = np.random.default_rng(90 + nseg)
    sizes = [int(x) for x in rng.choice([1, 17, 255, 256, 2048, 5000, 40001], size=nseg)]
    segs, snaps = build_segments(L, sizes, 90 + nseg, delta=set(range(0, nseg, 2)))
    accs = [_empty(n, torch.float32) for n in sizes]
    g1 = [_bf16(n, 1e-3, 9100 + i) for i, n in enumerate(sizes)]
    g2 = [_bf16(n, 1e-3, 9200 + i) for i, n in enumerate(sizes)]
    bases = [_bf16(n, 0.02, 9300 + i) for i, n in enumerate(sizes)]
    deltas = [_f32(n, 1e-4, 9400 + i) for i, n in enumerate(sizes)]
    merged = [_empty(n, torch.bfloat16) for n in sizes]
    torch.cuda.synchronize()
    before = L.table_cache_stats()
    L.adamw_step(segs, step=9, **HP)
    L.grad_accum([L.AccumSegment(a, g) for a, g in zip(accs, g1)], overwrite=True)
    L.grad_accum([L.AccumSegment(a, g) for a, g in zip(accs, g2)], overwrite=False)
    L.merge_delta([L.MergeSegment(b, d, o) for b, d, o in zip(bases, deltas, merged)])
    torch.cuda.synchronize()
    after = L.table_cache_stats()
    cached = after["hits"] + after["uploads"] - before["hits"] - before["uploads"]
    assert cached == (0 if nseg <= 24 else 4), (before, after)
    check_segments(segs, snaps, oracle_consts(HP, 9), f"n{nseg}.")
    for i, n in enumerate(sizes):
        acc = np.empty(n, np.float32)
        oracle.grad_accum(acc, to_np(g1[i]), overwrite=True)
        oracle.grad_accum(acc, to_np(g2[i]), overwrite=False)
        compare_f32(to_np(accs[i]), acc, f"n{nseg}.accum{i}")
        compare_bf16(to_np(merged[i]), oracle.merge_delta(to_np(bases[i]), to_np(deltas[i])),
                     f"n{nseg}.merge{i}")


@pytest.mark.parametrize("nseg", [13, 14])
def test_microbatch_tables_in_kernel_arguments_and_in_cache(L, nseg):
    """8 resident micro-batches: 13 segments fit the kernel arguments with
    their pointer lists, 14 go through the cache; both equal accumulate-then-
    step on every element."""
    nmb = 8
    rng = np.random.default_rng(110 + nseg)
    sizes = [int(x) for x in rng.choice([1, 255, 256, 4099, 30000], size=nseg)]
    segs, snaps = build_segments(L, sizes, 110 + nseg, delta=set(range(1, nseg, 2)))
    mbs = [[_bf16(n, 1e-3, 11000 + 100 * i + k) for k in range(nmb)] for i, n in enumerate(sizes)]
    for seg in segs:
        seg.grad = None
    torch.cuda.synchronize()
    before = L.table_cache_stats()
    L.adamw_step(segs, step=4, microbatch_grads=mbs, **HP)
    torch.cuda.synchronize()
    after = L.table_cache_stats()
    cached = after["hits"] + after["uploads"] - before["hits"] - before["uploads"]
    assert cached == (0 if nseg <= 13 else 1), (before, after)
    c = oracle_consts(HP, 4)
    for i, (seg, h, gs) in enumerate(zip(segs, snaps, mbs)):
        ref = _accumulate_then_step(h, [to_np(g) for g in gs], c, h["orig"])
        tag = f"mb.n{nseg}.seg{i}"
        compare_f32(to_np(seg.master), ref["master"], tag + ".master")
        compare_f32(to_np(seg.exp_avg), ref["m"], tag + ".m")
        compare_f32(to_np(seg.exp_avg_sq), ref["v"], tag + ".v")
        compare_bf16(to_np(seg.weight), ref["weight"], tag + ".weight")
        if seg.delta is not None:
            compare_f32(to_np(seg.delta), ref["delta"], tag + ".delta")


def _accumulate_then_step(snap, grads_np, consts, orig=None):
    """The oracle's separate calls: K accumulations (the first overwriting),
    then the step on the fp32 accumulator."""
    acc = np.empty(len(snap["master"]), np.float32)
    for k, g in enumerate(grads_np):
        oracle.grad_accum(acc, g, overwrite=(k == 0))
    return oracle_segment(snap["master"], snap["m"], snap["v"], acc, consts, orig)


@pytest.mark.parametrize("nmb", [1, 2, 3, 8, 16])
@pytest.mark.parametrize("offset", [0, 1])
def test_microbatch_sum_step(L, nmb, offset):
    """lema_adamw_step_microbatches equals K accumulations then the step on
    the accumulator, bit for bit: ragged sizes, misaligned arrays, delta on
    some segments only, planted -0 / inf / NaN gradients."""
    sizes = [4096 * 3 + 17, 255, 1, 70001]
    segs, snaps = build_segments(L, sizes, 70 + nmb, delta=(0, 3), offset=offset)
    mbs = []
    for i, (seg, n) in enumerate(zip(segs, sizes)):
        gs = [_bf16(n, 1e-3, 7000 + 100 * nmb + 10 * i + k, offset) for k in range(nmb)]
        if n > 40:
            gs[0][5] = -0.0
            gs[-1][9] = float("inf")
            gs[nmb // 2][13] = float("nan")
        mbs.append(gs)
        seg.grad = None
    L.adamw_step(segs, step=11, microbatch_grads=mbs, **HP)
    torch.cuda.synchronize()
    c = oracle_consts(HP, 11)
    for i, (seg, h, gs) in enumerate(zip(segs, snaps, mbs)):
        ref = _accumulate_then_step(h, [to_np(g) for g in gs], c, h["orig"])
        tag = f"mb{nmb}.seg{i}"
        compare_f32(to_np(seg.master), ref["master"], tag + ".master")
        compare_f32(to_np(seg.exp_avg), ref["m"], tag + ".m")
        compare_f32(to_np(seg.exp_avg_sq), ref["v"], tag + ".v")
        compare_bf16(to_np(seg.weight), ref["weight"], tag + ".weight")
        if seg.delta is not None:
            compare_f32(to_np(seg.delta), ref["delta"], tag + ".delta")


def test_microbatch_sum_llama7b_layer_full(L):
    """One Llama-2-7B layer with its 8 micro-batch gradients resident, summed
    inside the step: every element equals accumulate-then-step."""
    w = synth.WORKLOADS["llama7b_layer"]
    c = oracle_consts(HP, w.step)
    segs, mbs, hosts = [], [], []
    for i in range(len(w.segments)):
        st = synth.make_segment_state(w, i, DEV, with_orig=True)
        n = w.numels[i]
        seg = L.AdamwSegment(st["master"], st["m"], st["v"], None,
                             torch.empty(n, dtype=torch.bfloat16, device=DEV), st["orig"],
                             torch.empty(n, device=DEV))
        hosts.append({"master": to_np(st["master"]), "m": to_np(st["m"]), "v": to_np(st["v"]),
                      "orig": to_np(st["orig"])})
        segs.append(seg)
        mbs.append(st["grads"])
    plan = L.AdamwPlan(segs, microbatch_grads=mbs)
    plan.step(step=w.step, **HP)
    torch.cuda.synchronize()
    for i, (seg, h, gs) in enumerate(zip(segs, hosts, mbs)):
        ref = _accumulate_then_step(h, [to_np(g) for g in gs], c, h["orig"])
        compare_f32(to_np(seg.master), ref["master"], f"layer.seg{i}.master")
        compare_f32(to_np(seg.exp_avg), ref["m"], f"layer.seg{i}.m")
        compare_f32(to_np(seg.exp_avg_sq), ref["v"], f"layer.seg{i}.v")
        compare_bf16(to_np(seg.weight), ref["weight"], f"layer.seg{i}.weight")
        compare_f32(to_np(seg.delta), ref["delta"], f"layer.seg{i}.delta")


# ------------------------------------------------------ full workloads

def _workload_segments(L, w, with_orig, device_grads=1):
    segs = []
    for i in range(len(w.segments)):
        st = synth.make_segment_state(w, i, DEV, with_orig=with_orig, grads=device_grads)
        n = w.numels[i]
        segs.append(L.AdamwSegment(st["master"], st["m"], st["v"], st["grads"][0],
                                   torch.empty(n, dtype=torch.bfloat16, device=DEV),
                                   st.get("orig"),
                                   torch.empty(n, device=DEV) if with_orig else None))
    return segs


@pytest.mark.parametrize("with_delta", [False, True])
def test_gpt2_cattn_full(L, with_delta):
    """GPT-2-small c_attn, first two layers, t=1 from m=v=0: every element."""
    w = synth.WORKLOADS["gpt2_cattn_first2"]
    segs = _workload_segments(L, w, with_delta)
    snaps = [{"master": to_np(s.master), "m": to_np(s.exp_avg), "v": to_np(s.exp_avg_sq),
              "grad": to_np(s.grad), "orig": None if s.orig is None else to_np(s.orig)}
             for s in segs]
    L.adamw_step(segs, step=w.step, **HP)
    torch.cuda.synchronize()
    check_segments(segs, snaps, oracle_consts(HP, w.step), "gpt2 ")


def test_llama7b_lora_r16_full(L):
    """448 rank-16 LoRA adapter tensors in one call (t=10): every element."""
    w = synth.WORKLOADS["llama7b_lora_r16"]
    segs = _workload_segments(L, w, True)
    snaps = [{"master": to_np(s.master), "m": to_np(s.exp_avg), "v": to_np(s.exp_avg_sq),
              "grad": to_np(s.grad), "orig": to_np(s.orig)} for s in segs]
    L.adamw_step(segs, step=w.step, **HP)
    torch.cuda.synchronize()
    check_segments(segs, snaps, oracle_consts(HP, w.step), "lora ")


def test_llama7b_attn_last4_full(L):
    """Llama-2-7B q,k,v,o of the last 4 layers, t=100: all 268M elements."""
    w = synth.WORKLOADS["llama7b_attn_last4"]
    segs = _workload_segments(L, w, True)
    snaps = [{"master": to_np(s.master), "m": to_np(s.exp_avg), "v": to_np(s.exp_avg_sq),
              "grad": to_np(s.grad), "orig": to_np(s.orig)} for s in segs]
    L.adamw_step(segs, step=w.step, **HP)
    torch.cuda.synchronize()
    consts = oracle_consts(HP, w.step)
    for i in range(len(segs)):
        check_segments(segs[i:i + 1], snaps[i:i + 1], consts, f"attn{i} ")
        snaps[i] = None
    del segs
    torch.cuda.empty_cache()


def test_llama7b_layer_accumulate_then_step(L):
    """One Llama-2-7B layer: 8 bf16 micro-batches into fp32, then the step (t=50)."""
    w = synth.WORKLOADS["llama7b_layer"]
    accs, segs, snaps = [], [], []
    for i in range(len(w.segments)):
        st = synth.make_segment_state(w, i, DEV)
        n = w.numels[i]
        acc = torch.empty(n, device=DEV)
        accs.append((acc, st["grads"]))
        segs.append(L.AdamwSegment(st["master"], st["m"], st["v"], acc,
                                   torch.empty(n, dtype=torch.bfloat16, device=DEV)))
        snaps.append({"master": to_np(st["master"]), "m": to_np(st["m"]), "v": to_np(st["v"]),
                      "orig": None})
    for k in range(w.microbatches):
        L.grad_accum([L.AccumSegment(a, g[k]) for a, g in accs], overwrite=(k == 0))
    torch.cuda.synchronize()
    for i, (acc, grads) in enumerate(accs):
        ref = np.empty(acc.numel(), np.float32)
        for k, g in enumerate(grads):
            oracle.grad_accum(ref, to_np(g), overwrite=(k == 0))
        compare_f32(to_np(acc), ref, f"layer acc{i}")
        snaps[i]["grad"] = ref
    L.adamw_step(segs, step=w.step, **HP)
    torch.cuda.synchronize()
    check_segments(segs, snaps, oracle_consts(HP, w.step), "layer ")
    del accs, segs
    torch.cuda.empty_cache()


def _boundary_samples(n, rng):
    """Element indices around every power of two from 2^20 up to n, where a
    32-bit element or byte offset would wrap, plus both ends and random ones."""
    idx = [np.arange(2048), np.arange(n - 2048, n), rng.integers(0, n, 16384)]
    e = 20
    while (1 << e) < n:
        b = 1 << e
        idx.append(np.arange(max(0, b - 600), min(n, b + 600)))
        e += 1
    return np.unique(np.concatenate(idx))


def test_single_segment_beyond_2_31_elements(L):
    """One tensor of 2^31 + 4099 elements (73 GB of state with delta): every
    offset computation past 2, 4 and 8 GiB inside one segment, checked against
    the oracle on the elements around each power of two and at both ends."""
    n = (1 << 31) + 4099
    k = 90000
    master = synth.normal(n, 0.02, k, DEV)
    m = synth.normal(n, 1e-4, k + 1, DEV)
    v = synth.normal(n, 1e-3, k + 2, DEV).square_()
    grad = synth.bf16_normal(n, 1e-3, k + 3, DEV)
    orig = master.to(torch.bfloat16)
    weight = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    delta = torch.empty(n, device=DEV)
    idx = torch.from_numpy(_boundary_samples(n, np.random.default_rng(7))).to(DEV)
    before = {name: to_np(t[idx]) for name, t in
              (("master", master), ("m", m), ("v", v), ("grad", grad), ("orig", orig))}
    L.adamw_step([L.AdamwSegment(master, m, v, grad, weight, orig, delta)], step=10, **HP)
    torch.cuda.synchronize()
    ref = oracle_segment(before["master"], before["m"], before["v"], before["grad"],
                         oracle_consts(HP, 10), before["orig"])
    compare_f32(to_np(master[idx]), ref["master"], "2^31+ master")
    compare_f32(to_np(m[idx]), ref["m"], "2^31+ m")
    compare_f32(to_np(v[idx]), ref["v"], "2^31+ v")
    compare_bf16(to_np(weight[idx]), ref["weight"], "2^31+ weight")
    compare_f32(to_np(delta[idx]), ref["delta"], "2^31+ delta")
    del master, m, v, grad, orig, weight, delta
    torch.cuda.empty_cache()


@pytest.mark.parametrize("workload", ["llama7b_full", "llama7b_full_shard8"])
def test_llama7b_full_resident_sampled(L, workload):
    """Whole 7B shape resident (291 tensors, ~148 GB with delta), and one of 8
    data-parallel ranks' share of it: two steps (t=10 with delta, t=11
    without), checked on sampled elements of every tensor, including each
    tensor's first and last 2048."""
    w = synth.WORKLOADS[workload]
    segs = _workload_segments(L, w, True)
    rng = np.random.default_rng(4)
    idx = []
    for n in w.numels:
        i = np.unique(np.concatenate([np.arange(min(n, 2048)), np.arange(max(0, n - 2048), n),
                                      rng.integers(0, n, 8192)]))
        idx.append(torch.from_numpy(i).to(DEV))

    def gather(s, i, fields):
        return {f: to_np(getattr(s, f)[i]) for f in fields}

    for step, with_delta in ((w.step, True), (w.step + 1, False)):
        before = [gather(s, i, ("master", "exp_avg", "exp_avg_sq", "grad", "orig"))
                  for s, i in zip(segs, idx)]
        run = segs if with_delta else [L.AdamwSegment(s.master, s.exp_avg, s.exp_avg_sq, s.grad,
                                                      s.weight) for s in segs]
        L.adamw_step(run, step=step, **HP)
        torch.cuda.synchronize()
        consts = oracle_consts(HP, step)
        for k, (s, i, b) in enumerate(zip(segs, idx, before)):
            ref = oracle_segment(b["master"], b["exp_avg"], b["exp_avg_sq"], b["grad"], consts,
                                 b["orig"] if with_delta else None)
            after = gather(s, i, ("master", "exp_avg", "exp_avg_sq", "weight", "delta"))
            tag = f"7b t={step} seg{k}"
            compare_f32(after["master"], ref["master"], tag + ".master")
            compare_f32(after["exp_avg"], ref["m"], tag + ".m")
            compare_f32(after["exp_avg_sq"], ref["v"], tag + ".v")
            compare_bf16(after["weight"], ref["weight"], tag + ".weight")
            if with_delta:
                compare_f32(after["delta"], ref["delta"], tag + ".delta")
    del segs
    torch.cuda.empty_cache()
