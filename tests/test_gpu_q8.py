"""GPU parity of the int8 + per-row-scale path against the CPU oracle.

int8 moments and int8 gradient accumulators with a scale per row, widened
to fp32 within the step alone (LEMA README, "Quantization": the 8-bit
optimizer-state and accumulator settings).  Initial int8 state is
quantized by the oracle on the host and uploaded, so every comparison here
checks the HIP path against oracle-made inputs and oracle-made outputs.  The
bar is bit-exact for codes, scales (NaN compared as a class), the fp32
master and delta and the bf16 weight.
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


def up(a: np.ndarray, offset: int = 0) -> torch.Tensor:
    """Host array -> device tensor starting `offset` elements into its buffer."""
    dt = {np.float32: torch.float32, np.int8: torch.int8, np.uint16: torch.int16}[a.dtype.type]
    buf = torch.empty(a.size + offset, dtype=dt, device=DEV)
    t = buf[offset:]
    src = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    t.copy_(src)
    return t.view(torch.bfloat16) if a.dtype == np.uint16 else t


def host_f32(n, sigma, seed, square=False):
    t = synth.normal(n, sigma, seed, DEV)
    if square:
        t.mul_(t)
    return to_np(t)


def host_bf16(n, sigma, seed):
    return to_np(synth.normal(n, sigma, seed, DEV).to(torch.bfloat16))


def compare_codes(got: torch.Tensor, ref: np.ndarray, name: str):
    g = to_np(got)
    bad = int((g != ref).sum())
    assert bad == 0, f"{name}: {bad} int8 codes differ"


class Case:
    """One segment: host inputs, device tensors, and the oracle's outputs."""

    def __init__(self, L, n, row_len, seed, *, grad="bf16", moments="q8", delta=False,
                 offset=0, specials=False):
        self.n, self.row_len = n, row_len
        h = {"master": host_f32(n, 0.02, seed)}
        m32 = host_f32(n, 1e-4, seed + 1)
        v32 = host_f32(n, 1e-3, seed + 2, square=True)
        if grad == "bf16":
            g = host_bf16(n, 1e-3, seed + 3)
        elif grad == "fp32":
            g = host_f32(n, 3e-3, seed + 3)
        else:
            g = oracle.quantize_rows(host_f32(n, 3e-3, seed + 3), row_len)
        if specials and n > 40:
            gv = g[0] if isinstance(g, tuple) else g
            if gv.dtype == np.uint16:
                gv[3], gv[17] = 0x7FC0, 0x7F80          # NaN, +inf (bf16 patterns)
            elif gv.dtype == np.float32:
                gv[3], gv[17] = np.nan, np.inf
            m32[5:5 + min(row_len, n - 5)] = 0.0        # a zero stretch of m
        self.h = h
        self.mom_q8 = moments == "q8"
        if self.mom_q8:
            self.mq = oracle.quantize_rows(m32, row_len)
            self.vq = oracle.quantize_rows(v32, row_len)
        else:
            self.m32, self.v32 = m32, v32
        self.g = g
        self.orig = oracle.rne16(h["master"]) if delta else None

        # device tensors
        self.master = up(h["master"], offset)
        if self.mom_q8:
            self.m = L.Q8(up(self.mq[0], offset), up(self.mq[1]), row_len)
            self.v = L.Q8(up(self.vq[0], offset), up(self.vq[1]), row_len)
        else:
            self.m, self.v = up(m32, offset), up(v32, offset)
        self.grad = L.Q8(up(g[0], offset), up(g[1]), row_len) if isinstance(g, tuple) else up(g, offset)
        self.weight = torch.empty(n + offset, dtype=torch.bfloat16, device=DEV)[offset:]
        self.dev_orig = None if self.orig is None else up(self.orig, offset)
        self.delta = None if self.orig is None else torch.empty(n + offset, device=DEV)[offset:]

    def segment(self, L):
        return L.AdamwQ8Segment(self.master, self.m, self.v, self.grad, self.weight,
                                self.dev_orig, self.delta)

    def run_oracle(self, consts):
        master = self.h["master"].copy()
        if self.mom_q8:
            m = (self.mq[0].copy(), self.mq[1].copy())
            v = (self.vq[0].copy(), self.vq[1].copy())
        else:
            m, v = self.m32.copy(), self.v32.copy()
        w, d = oracle.adamw_step_q8(master, m, v, self.g, consts, self.row_len, orig=self.orig)
        return master, m, v, w, d

    def check(self, consts, tag):
        master, m, v, w, d = self.run_oracle(consts)
        compare_f32(to_np(self.master), master, tag + ".master")
        compare_bf16(to_np(self.weight), w, tag + ".weight")
        if d is not None:
            compare_f32(to_np(self.delta), d, tag + ".delta")
        if self.mom_q8:
            for name, dev, ref in (("m", self.m, m), ("v", self.v, v)):
                compare_codes(dev.codes, ref[0], f"{tag}.{name}.codes")
                compare_f32(to_np(dev.scale), ref[1], f"{tag}.{name}.scale")
        else:
            compare_f32(to_np(self.m), m, tag + ".m")
            compare_f32(to_np(self.v), v, tag + ".v")
        return master, m, v


def step(L, cases, t, stream=None):
    L.adamw_step_q8([c.segment(L) for c in cases], step=t, stream=stream, **HP)


# ------------------------------------------------------------ conversions

@pytest.mark.parametrize("row_len", [1, 3, 4, 16, 100, 256, 4096, 4100, 11008, 16384])
@pytest.mark.parametrize("offset", [0, 1])
def test_quantize_dequantize_rows(L, row_len, offset):
    """Codes and scales of lema_quantize_rows and the values of
    lema_dequantize_rows against the oracle, with a ragged last row, zero,
    NaN, infinite and subnormal rows, on vector and element paths."""
    # short rows: several workgroups' worth (packed rows for 4, 16, 256)
    rows = 5 if row_len > 256 else 2 * (4 * 256 * 4 // max(row_len, 4)) + 5
    n = row_len * rows + max(1, row_len // 3)
    x = host_f32(n, 1e-3, 7000 + row_len)
    x[:row_len] = 0.0                                   # an all-zero row
    x[row_len] = np.nan                                 # a NaN row
    x[2 * row_len] = np.inf                             # an infinite row
    x[3 * row_len:4 * row_len] = np.float32(1e-42)      # a subnormal row
    q = L.Q8(torch.empty(n + offset, dtype=torch.int8, device=DEV)[offset:],
             torch.empty(L.Q8.rows_of(n, row_len), device=DEV), row_len)
    xd = up(x, offset)
    L.quantize_rows([(xd, q)])
    rq, rs = oracle.quantize_rows(x, row_len)
    compare_codes(q.codes, rq, "codes")
    compare_f32(to_np(q.scale), rs, "scale")
    back = torch.empty(n + offset, device=DEV)[offset:]
    L.dequantize_rows([(back, q)])
    compare_f32(to_np(back), oracle.dequantize_rows(rq, rs, row_len), "dequantized")


def test_quantize_near_half_integers(L):
    """Rows whose values divide by the row scale to half-integers or a few
    ulps off them (where the kernels fall back from x*(1/s) to the IEEE
    division), over scales from 2^-120 to 2^120."""
    rng = np.random.default_rng(77)
    rows = []
    for e in range(-120, 121, 8):
        a = np.float32(rng.uniform(1, 2) * 2.0 ** e)
        s = np.float32(a / np.float32(127))
        k = rng.integers(-127, 127, 256).astype(np.float64) + 0.5
        j = rng.integers(-6, 7, 256) * 2.0 ** -19
        x = ((k + j) * float(s)).astype(np.float32)
        x = np.where(np.abs(x) <= a, x, np.float32(0))
        x[0] = a
        x[1:3] = np.nextafter(x[5:7], np.float32(np.inf))
        rows.append(x)
    x = np.concatenate(rows)
    q = L.Q8.empty(x.size, 256)
    L.quantize_rows([(up(x), q)])
    rq, rs = oracle.quantize_rows(x, 256)
    compare_codes(q.codes, rq, "codes")
    compare_f32(to_np(q.scale), rs, "scale")


# ------------------------------------------------------------------ step

@pytest.mark.parametrize("grad", ["bf16", "fp32", "q8"])
@pytest.mark.parametrize("delta", [False, True])
@pytest.mark.parametrize("row_len", [1, 7, 64, 4096, 11008])
def test_q8_step_matches_oracle(L, grad, delta, row_len):
    """int8 moments with each gradient kind, ragged last rows, narrow teams
    (row_len 1, 7: element path), one-workgroup rows (4096) and the wide
    workgroup (11008)."""
    n = row_len * 6 + (row_len // 2 or 1)
    c = Case(L, n, row_len, 9000 + row_len, grad=grad, delta=delta)
    step(L, [c], 100)
    torch.cuda.synchronize()
    c.check(oracle_consts(HP, 100), f"q8[{grad},{delta},{row_len}]")


@pytest.mark.parametrize("row_len", [4, 8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("kinds", [("q8", "bf16"), ("q8", "q8"), ("fp32", "q8")])
def test_q8_step_packed_rows(L, row_len, kinds):
    """Rows of 4*S elements (S a power of two up to 64) run packed: each
    lane's chunks belong to different rows, so a wavefront's accesses stay
    contiguous.  Two and a bit workgroups of rows, a ragged last row, delta on."""
    moments, grad = kinds
    rows_per_block = 4 * 256 * 4 // row_len
    n = row_len * (2 * rows_per_block + 37) + row_len // 2 + 1
    c = Case(L, n, row_len, 9500 + row_len, grad=grad, moments=moments, delta=True)
    step(L, [c], 100)
    torch.cuda.synchronize()
    c.check(oracle_consts(HP, 100), f"packed[{moments},{grad},{row_len}]")


@pytest.mark.parametrize("offset", [1, 3])
def test_q8_step_misaligned(L, offset):
    """Arrays starting off their vector alignment take the element path."""
    cases = [Case(L, 4096 * 3 + 5, 4096, 9100, delta=True, offset=offset),
             Case(L, 333, 16, 9200, grad="q8", offset=offset)]
    L.adamw_step_q8([cases[0].segment(L)], step=7, **HP)
    L.adamw_step_q8([cases[1].segment(L)], step=7, **HP)
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        c.check(oracle_consts(HP, 7), f"misaligned{i}")


def test_q8_step_mixed_segments_one_call(L):
    """One call over segments of both workgroup sizes, different row lengths,
    empty segments and delta on only some of them."""
    spec = [(4096 * 4, 4096, True), (11008 * 2 + 9, 11008, False), (16 * 100, 16, True),
            (2304, 2304, False), (5, 3, False), (16384 * 2, 16384, True), (777, 1, False)]
    cases = [Case(L, n, rl, 9300 + 10 * i, delta=d) for i, (n, rl, d) in enumerate(spec)]
    segs = [c.segment(L) for c in cases]
    empty = L.AdamwQ8Segment(torch.empty(0, device=DEV), L.Q8.zeros(0, 4), L.Q8.zeros(0, 4),
                             torch.empty(0, dtype=torch.bfloat16, device=DEV),
                             torch.empty(0, dtype=torch.bfloat16, device=DEV))
    L.adamw_step_q8(segs[:3] + [empty] + segs[3:], step=50, **HP)
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        c.check(oracle_consts(HP, 50), f"mixed{i}")


@pytest.mark.parametrize("kinds", [("q8", "bf16", True), ("q8", "q8", True), ("q8", "fp32", False),
                                   ("fp32", "q8", True)])
def test_q8_step_one_mixed_launch(L, kinds):
    """Packed rows (16, 256), wave rows of 4096 and rows of 11,008, 11,260
    and 11,264 elements (one 256-lane team each, up to 11 chunks per lane,
    ragged ends) go into one mixed launch, next to segments that keep their
    own launch groups (rows of 1, and misaligned rows); every element."""
    moments, grad, delta = kinds
    spec = [(11008 * 3, 11008, 0), (11264 * 2, 11264, 0), (11260 * 2 + 4, 11260, 0),
            (4096 * 3 + 256, 4096, 0), (16 * 1000 + 8, 16, 0), (256 * 50, 256, 0),
            (777, 1, 0), (4096 * 2 + 12, 4096, 1)]
    cases = [Case(L, n, rl, 9600 + 10 * i, grad=grad, moments=moments, delta=delta, offset=off)
             for i, (n, rl, off) in enumerate(spec)]
    for t in (60, 61):
        step(L, cases, t)
        torch.cuda.synchronize()
        for i, c in enumerate(cases):
            master, m, v = c.check(oracle_consts(HP, t), f"mixed-launch[{kinds}] t={t} seg{i}")
            # the next step starts from the oracle's outputs (equal to the device's)
            c.h["master"] = master
            if c.mom_q8:
                c.mq, c.vq = m, v
            else:
                c.m32, c.v32 = m, v


def test_fp32_moments_with_q8_accumulator(L):
    """fp32 moments with an int8 gradient accumulator (grad_acc_bits = 8 alone)."""
    cases = [Case(L, 4096 * 3 + 100, 4096, 9400, grad="q8", moments="fp32", delta=True),
             Case(L, 11008 * 2, 11008, 9410, grad="q8", moments="fp32")]
    step(L, cases, 12)
    torch.cuda.synchronize()
    for i, c in enumerate(cases):
        c.check(oracle_consts(HP, 12), f"fp32mom{i}")


def test_q8_three_consecutive_steps(L):
    """State carried over three steps (new bf16 gradients each time) stays
    bit-identical to the oracle's."""
    n, rl = 4096 * 5 + 300, 4096
    c = Case(L, n, rl, 9500, delta=True)
    master, m, v = c.h["master"].copy(), (c.mq[0].copy(), c.mq[1].copy()), (c.vq[0].copy(), c.vq[1].copy())
    for t in (20, 21, 22):
        g = host_bf16(n, 1e-3, 9600 + t)
        c.grad = up(g)
        step(L, [c], t)
        w, d = oracle.adamw_step_q8(master, m, v, g, oracle_consts(HP, t), rl, orig=c.orig)
        torch.cuda.synchronize()
        compare_f32(to_np(c.master), master, f"t{t}.master")
        compare_bf16(to_np(c.weight), w, f"t{t}.weight")
        compare_f32(to_np(c.delta), d, f"t{t}.delta")
        compare_codes(c.m.codes, m[0], f"t{t}.m")
        compare_codes(c.v.codes, v[0], f"t{t}.v")
        compare_f32(to_np(c.m.scale), m[1], f"t{t}.ms")
        compare_f32(to_np(c.v.scale), v[1], f"t{t}.vs")


def test_q8_step_special_values(L):
    """NaN and infinite gradients: their rows get NaN or infinite scales and
    zero codes, other rows are untouched; a zero stretch of m is exact."""
    for grad in ("bf16", "fp32"):
        c = Case(L, 64 * 10 + 3, 64, 9700, grad=grad, specials=True, delta=True)
        step(L, [c], 3)
        torch.cuda.synchronize()
        _, m, _ = c.check(oracle_consts(HP, 3), f"specials[{grad}]")
        assert np.isnan(m[1][0])                      # the NaN lands in row 0


# ----------------------------------------------------------- accumulation

@pytest.mark.parametrize("row_len", [3, 16, 64, 256, 4096, 11008])
@pytest.mark.parametrize("offset", [0, 1])
def test_q8_accumulation(L, row_len, offset):
    """Four bf16 micro-batches into an int8 accumulator: overwrite, then
    dequantize-add-requantize, bit-exact after every micro-batch."""
    rows = 4 if row_len > 256 else 2 * (4 * 256 * 4 // row_len) + 5   # packed: several workgroups
    n = row_len * rows + row_len // 2 + 1
    acc = L.Q8(torch.full((n + offset,), 77, dtype=torch.int8, device=DEV)[offset:],
               torch.full((L.Q8.rows_of(n, row_len),), 5.0, device=DEV), row_len)
    ref_q = np.zeros(n, np.int8)
    ref_s = np.zeros(L.Q8.rows_of(n, row_len), np.float32)
    for k in range(4):
        g = host_bf16(n, 1e-3, 9800 + 10 * row_len + k)
        L.grad_accum_q8([L.AccumQ8Segment(acc, up(g, offset))], overwrite=k == 0)
        oracle.grad_accum_q8(ref_q, ref_s, g, k == 0, row_len)
        torch.cuda.synchronize()
        compare_codes(acc.codes, ref_q, f"acc{k}.codes")
        compare_f32(to_np(acc.scale), ref_s, f"acc{k}.scale")


def test_q8_plans_match_direct_calls(L):
    """AdamwQ8Plan / AccumQ8Plan reuse one marshalled list; results equal a
    direct call on cloned state."""
    a = Case(L, 4096 * 2 + 10, 4096, 9900, delta=True)
    b = Case(L, 4096 * 2 + 10, 4096, 9900, delta=True)
    plan = L.AdamwQ8Plan([a.segment(L)])
    plan.step(step=9, **HP)
    step(L, [b], 9)
    torch.cuda.synchronize()
    for x, y in ((a.master, b.master), (a.m.codes, b.m.codes), (a.v.scale, b.v.scale),
                 (a.weight, b.weight), (a.delta, b.delta)):
        assert torch.equal(x, y)


def test_repeated_calls_reuse_cached_tables(L):
    """A plan stepped again and again uploads its launch tables once: step
    calls over rows of 4096 and of 11,008 launch one mixed table per call,
    accumulation calls (both row lengths in 256-lane wave rows) one, and
    all stay cached."""
    cases = [Case(L, 4096 * 2, 4096, 9950), Case(L, 11008 * 2, 11008, 9960)]
    plan = L.AdamwQ8Plan([c.segment(L) for c in cases])
    accs = [L.Q8.empty(c.n, c.row_len) for c in cases]
    grads = [up(host_bf16(c.n, 1e-3, 9970 + i)) for i, c in enumerate(cases)]
    acc_plan = L.AccumQ8Plan([L.AccumQ8Segment(a, g) for a, g in zip(accs, grads)])
    acc_plan.run(overwrite=True)
    plan.step(step=1, **HP)
    torch.cuda.synchronize()
    before = L.table_cache_stats()
    for t in range(2, 12):
        acc_plan.run(overwrite=False)
        plan.step(step=t, **HP)
    torch.cuda.synchronize()
    after = L.table_cache_stats()
    assert after["uploads"] == before["uploads"], (before, after)
    assert after["hits"] - before["hits"] == 10 * (1 + 1), (before, after)


# ------------------------------------------------------------ wave rows
#
# Rows of 256 elements and more (other than the packed ones) on
# vector-aligned arrays whose element count is a multiple of 4 run as wave
# rows: teams of whole wavefronts, through row-sized buffer resources.  The
# step's teams (4 chunks per lane) covered here: 64 lanes (300 with two
# chunks, 1000 with four: four rows per workgroup), 128 (2000), 256 (3000,
# 4096), 512 and 1024 in wide workgroups (5000; 11,008 and 16,384).
# Accumulation and conversions hold up to 16 chunks per lane in 256-lane
# workgroups: 64 lanes for rows up to 4096, 128 for 5000, 256 for 11,008 and
# 16,384.  Every case has a ragged last row and, for the narrower teams,
# workgroups with teams past the last row.

WAVE_ROWS = [300, 1000, 2000, 3000, 4096, 5000, 11008, 16384]


def wave_numel(row_len: int) -> int:
    rows = 9 if row_len <= 2000 else 3          # 9 rows of 1000: the third workgroup holds one
    return row_len * rows + (row_len // 3) // 4 * 4 + 4


@pytest.mark.parametrize("row_len", WAVE_ROWS)
def test_wave_rows_quantize_dequantize(L, row_len):
    """Zero, NaN, infinite and subnormal rows, a ragged last row."""
    n = wave_numel(row_len)
    assert n % 4 == 0
    x = host_f32(n, 1e-3, 7100 + row_len)
    x[:row_len] = 0.0
    x[row_len + 5] = np.nan
    x[2 * row_len - 1] = -np.inf
    if n >= 4 * row_len:
        x[3 * row_len:4 * row_len] = np.float32(-3e-42)
    q = L.Q8.empty(n, row_len)
    L.quantize_rows([(up(x), q)])
    rq, rs = oracle.quantize_rows(x, row_len)
    compare_codes(q.codes, rq, "codes")
    compare_f32(to_np(q.scale), rs, "scale")
    back = torch.empty(n, device=DEV)
    L.dequantize_rows([(back, q)])
    compare_f32(to_np(back), oracle.dequantize_rows(rq, rs, row_len), "dequantized")


@pytest.mark.parametrize("row_len", WAVE_ROWS)
@pytest.mark.parametrize("kinds", [("q8", "bf16", True), ("q8", "q8", True), ("q8", "fp32", False),
                                   ("fp32", "q8", True)])
def test_wave_rows_step(L, row_len, kinds):
    moments, grad, delta = kinds
    c = Case(L, wave_numel(row_len), row_len, 9050 + row_len, grad=grad, moments=moments,
             delta=delta)
    step(L, [c], 30)
    torch.cuda.synchronize()
    c.check(oracle_consts(HP, 30), f"wave[{moments},{grad},{delta},{row_len}]")


def nonzero_codes(n, seed):
    rng = np.random.default_rng(seed)
    k = rng.integers(1, 128, n) * rng.choice([-1, 1], n)
    return k.astype(np.int8)


@pytest.mark.parametrize("row_len", WAVE_ROWS)
def test_wave_rows_step_special_scales(L, row_len):
    """Old row scales of +inf (over codes that are all nonzero, so every
    element of the row dequantizes to an infinity) and NaN: lanes whose
    chunks lie past the row's end must stay out of the new absmax."""
    c = Case(L, wave_numel(row_len), row_len, 9150 + row_len, delta=True)
    rows = L.Q8.rows_of(c.n, row_len)
    last = slice((rows - 1) * row_len, c.n)
    c.mq[0][last] = nonzero_codes(c.n - (rows - 1) * row_len, 1)
    c.mq[1][rows - 1] = np.inf
    c.vq[1][1] = np.nan
    c.m = L.Q8(up(c.mq[0]), up(c.mq[1]), row_len)
    c.v = L.Q8(up(c.vq[0]), up(c.vq[1]), row_len)
    step(L, [c], 4)
    torch.cuda.synchronize()
    _, m, v = c.check(oracle_consts(HP, 4), f"wave_specials[{row_len}]")
    assert np.isinf(m[1][rows - 1]) and np.isnan(v[1][1])


@pytest.mark.parametrize("row_len", WAVE_ROWS)
def test_wave_rows_accumulation(L, row_len):
    """Overwrite, then three dequantize-add-requantize micro-batches; then
    one more onto old scales of +inf (all codes nonzero) and NaN."""
    n = wave_numel(row_len)
    rows = L.Q8.rows_of(n, row_len)
    acc = L.Q8.empty(n, row_len)
    ref_q = np.zeros(n, np.int8)
    ref_s = np.zeros(rows, np.float32)
    for k in range(5):
        if k == 4:
            ref_q[(rows - 1) * row_len:] = nonzero_codes(n - (rows - 1) * row_len, 2)
            ref_s[rows - 1], ref_s[0] = np.inf, np.nan
            acc = L.Q8(up(ref_q), up(ref_s), row_len)
        g = host_bf16(n, 1e-3, 9850 + 10 * row_len + k)
        L.grad_accum_q8([L.AccumQ8Segment(acc, up(g))], overwrite=k == 0)
        oracle.grad_accum_q8(ref_q, ref_s, g, k == 0, row_len)
        torch.cuda.synchronize()
        compare_codes(acc.codes, ref_q, f"acc{k}.codes")
        compare_f32(to_np(acc.scale), ref_s, f"acc{k}.scale")
    assert np.isinf(ref_s[rows - 1]) and np.isnan(ref_s[0])


# -------------------------------------------------- workloads at full size

def _workload_q8(L, w, row_len_of, *, delta, grad="bf16"):
    cases = []
    for i, (label, shape) in enumerate(w.segments):
        n = w.numels[i]
        cases.append(Case(L, n, row_len_of(shape), 100000 + 1000 * w.wid + i, grad=grad,
                          delta=delta))
    return cases


def last_dim(shape):
    return shape[-1]


def test_flat_q8_state_step_matches_oracle(L):
    """int8-moment segments that are views of flat buffers (flat_q8_state):
    codes at 64-element offsets of shared buffers, scales at row offsets of
    another; bf16 gradient, delta on; every element against the oracle."""
    numels, row_lens = [4096 * 3, 11008 * 2 + 5, 100, 16 * 30, 0, 4099], [4096, 11008, 7, 16, 5, 4099]
    el, rw, segs = L.flat_q8_state(numels, row_lens, grad="bf16", delta=True, device=DEV)
    refs = []
    for i, (s, n, rl) in enumerate(zip(segs, numels, row_lens)):
        k = 73000 + 10 * i
        master = host_f32(n, 0.02, k)
        mq = oracle.quantize_rows(host_f32(n, 1e-4, k + 1), rl)
        vq = oracle.quantize_rows(host_f32(n, 1e-3, k + 2, square=True), rl)
        g = host_bf16(n, 1e-3, k + 3)
        orig = oracle.rne16(master)
        s.master.copy_(torch.from_numpy(master))
        s.exp_avg.codes.copy_(torch.from_numpy(mq[0]))
        s.exp_avg.scale.copy_(torch.from_numpy(mq[1]))
        s.exp_avg_sq.codes.copy_(torch.from_numpy(vq[0]))
        s.exp_avg_sq.scale.copy_(torch.from_numpy(vq[1]))
        s.grad.copy_(torch.from_numpy(g.view(np.int16)).view(torch.bfloat16))
        s.orig.copy_(torch.from_numpy(orig.view(np.int16)).view(torch.bfloat16))
        refs.append((master, mq, vq, g, orig))
    L.adamw_step_q8(segs, step=9, **HP)
    torch.cuda.synchronize()
    consts = oracle_consts(HP, 9)
    for i, (s, (master, mq, vq, g, orig)) in enumerate(zip(segs, refs)):
        m, v = (mq[0].copy(), mq[1].copy()), (vq[0].copy(), vq[1].copy())
        w, d = oracle.adamw_step_q8(master, m, v, g, consts, row_lens[i], orig=orig)
        tag = f"flat q8 seg{i}"
        compare_f32(to_np(s.master), master, tag + ".master")
        compare_bf16(to_np(s.weight), w, tag + ".weight")
        compare_f32(to_np(s.delta), d, tag + ".delta")
        for name, dq, ref in (("m", s.exp_avg, m), ("v", s.exp_avg_sq, v)):
            compare_codes(dq.codes, ref[0], f"{tag}.{name}.codes")
            compare_f32(to_np(dq.scale), ref[1], f"{tag}.{name}.scale")


def test_q8_single_segment_beyond_2_31_elements(L):
    """int8 moments on one tensor of 2^31 + 4096 elements in rows of 4096
    (524,289 rows): row and element offsets past 2^31, checked against the
    oracle on whole rows around every power-of-two element index and at both
    ends (a row is the unit the oracle quantizes)."""
    rl = 4096
    n = (1 << 31) + rl
    rows = n // rl
    k = 91000
    master = synth.normal(n, 0.02, k, DEV)
    m32 = synth.normal(n, 1e-4, k + 1, DEV)
    v32 = synth.normal(n, 1e-3, k + 2, DEV).square_()
    mq, vq = L.Q8.empty(n, rl), L.Q8.empty(n, rl)
    L.quantize_rows([(m32, mq), (v32, vq)])
    del m32, v32
    grad = synth.bf16_normal(n, 1e-3, k + 3, DEV)
    weight = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    pick = {0, 1, rows - 2, rows - 1}
    e = 20
    while (1 << e) < n:
        pick |= {max(0, (1 << e) // rl - 1), min(rows - 1, (1 << e) // rl)}
        e += 1
    pick = sorted(pick)
    elems = torch.from_numpy(np.concatenate([np.arange(r * rl, (r + 1) * rl) for r in pick])).to(DEV)
    ridx = torch.tensor(pick, device=DEV)
    before = {"master": to_np(master[elems]), "mq": to_np(mq.codes[elems]), "ms": to_np(mq.scale[ridx]),
              "vq": to_np(vq.codes[elems]), "vs": to_np(vq.scale[ridx]), "g": to_np(grad[elems])}
    L.adamw_step_q8([L.AdamwQ8Segment(master, mq, vq, grad, weight)], step=10, **HP)
    torch.cuda.synchronize()
    mref, vref = (before["mq"].copy(), before["ms"].copy()), (before["vq"].copy(), before["vs"].copy())
    mref_master = before["master"].copy()
    w, _ = oracle.adamw_step_q8(mref_master, mref, vref, before["g"], oracle_consts(HP, 10), rl)
    compare_f32(to_np(master[elems]), mref_master, "2^31+ q8 master")
    compare_bf16(to_np(weight[elems]), w, "2^31+ q8 weight")
    compare_codes(mq.codes[elems], mref[0], "2^31+ q8 m codes")
    compare_codes(vq.codes[elems], vref[0], "2^31+ q8 v codes")
    compare_f32(to_np(mq.scale[ridx]), mref[1], "2^31+ q8 m scales")
    compare_f32(to_np(vq.scale[ridx]), vref[1], "2^31+ q8 v scales")
    del master, mq, vq, grad, weight
    torch.cuda.empty_cache()


def test_llama7b_full_rows_shard8_q8_sampled(L):
    """One of 8 data-parallel ranks' share of the whole 7B shape split on
    whole rows (842.5 M params in 291 tensors), with int8 moments, in the flat
    state bench.py times: one step with delta, checked against the oracle on
    whole sampled rows of every tensor (the first, the last and 14 random
    ones; a row is the unit the oracle quantizes)."""
    w = synth.WORKLOADS["llama7b_full_rows_shard8"]
    row_lens = [shape[-1] for _, shape in w.segments]
    el, rw, segs = L.flat_q8_state(w.numels, row_lens, grad="bf16", delta=True, device=DEV)
    for i, s in enumerate(segs):
        st = synth.make_segment_state(w, i, DEV, with_orig=True)
        s.master.copy_(st["master"])
        L.quantize_rows([(st["m"], s.exp_avg), (st["v"], s.exp_avg_sq)])
        s.orig.copy_(st["orig"])
        s.grad.copy_(st["grads"][0])
        del st
    torch.cuda.synchronize()
    rng = np.random.default_rng(21)
    picks = []
    for n, rl in zip(w.numels, row_lens):
        rows = n // rl
        r = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 14)]))
        el_idx = (r[:, None] * rl + np.arange(rl)[None, :]).reshape(-1)
        picks.append((torch.from_numpy(r).to(DEV), torch.from_numpy(el_idx).to(DEV)))

    def take(t, i):
        return to_np(t[i])

    before = []
    for s, (ri, ei) in zip(segs, picks):
        before.append({
            "master": take(s.master, ei), "grad": take(s.grad, ei), "orig": take(s.orig, ei),
            "m": (take(s.exp_avg.codes, ei), take(s.exp_avg.scale, ri)),
            "v": (take(s.exp_avg_sq.codes, ei), take(s.exp_avg_sq.scale, ri))})
    L.adamw_step_q8(segs, step=w.step, **HP)
    torch.cuda.synchronize()
    consts = oracle_consts(HP, w.step)
    for k, (s, (ri, ei), b, rl) in enumerate(zip(segs, picks, before, row_lens)):
        master, m, v = b["master"].copy(), b["m"], b["v"]
        wref, dref = oracle.adamw_step_q8(master, m, v, b["grad"], consts, rl, orig=b["orig"])
        tag = f"rows shard seg{k}"
        compare_f32(take(s.master, ei), master, tag + ".master")
        compare_bf16(take(s.weight, ei), wref, tag + ".weight")
        compare_f32(take(s.delta, ei), dref, tag + ".delta")
        for name, q, ref in (("m", s.exp_avg, m), ("v", s.exp_avg_sq, v)):
            bad = int((take(q.codes, ei) != ref[0]).sum())
            assert bad == 0, f"{tag}.{name}: {bad} int8 codes differ"
            compare_f32(take(q.scale, ri), ref[1], f"{tag}.{name}.scale")
    del segs, el, rw
    torch.cuda.empty_cache()


def test_llama7b_attn_last4_q8_full(L):
    """Llama-2-7B q,k,v,o of the last 4 layers (268 M parameters, rows of
    4096) with int8 moments, bf16 gradient and delta: every element checked."""
    w = synth.WORKLOADS["llama7b_attn_last4"]
    cases = _workload_q8(L, w, last_dim, delta=True)
    step(L, cases, w.step)
    torch.cuda.synchronize()
    consts = oracle_consts(HP, w.step)
    for i, c in enumerate(cases):
        c.check(consts, f"attn{i}")
        del c.master, c.m, c.v, c.grad, c.weight, c.dev_orig, c.delta


def test_llama7b_layer_q8_accumulate_then_step(L):
    """One Llama-2-7B layer (rows of 4096 and 11008, 1-D norms): 8 micro-
    batches into int8 accumulators, then the step with int8 moments and the
    int8 accumulator as its gradient; every element checked."""
    w = synth.WORKLOADS["llama7b_layer"]
    consts = oracle_consts(HP, w.step)
    for i, (label, shape) in enumerate(w.segments):
        n, rl = w.numels[i], shape[-1]
        c = Case(L, n, rl, 200000 + i, grad="bf16", delta=True)
        acc = L.Q8.empty(n, rl)
        ref_q = np.zeros(n, np.int8)
        ref_s = np.zeros(L.Q8.rows_of(n, rl), np.float32)
        for k in range(w.microbatches):
            g = host_bf16(n, 1e-3, synth.seed_of(w.wid, synth.ARRAY_GRAD0 + k, i))
            L.grad_accum_q8([L.AccumQ8Segment(acc, up(g))], overwrite=k == 0)
            oracle.grad_accum_q8(ref_q, ref_s, g, k == 0, rl)
        c.grad, c.g = acc, (ref_q, ref_s)
        step(L, [c], w.step)
        torch.cuda.synchronize()
        compare_codes(acc.codes, ref_q, f"{label}.acc")
        compare_f32(to_np(acc.scale), ref_s, f"{label}.acc_scale")
        c.check(consts, label)


def test_llama7b_lora_r16_q8_full(L):
    """The 448 rank-16 LoRA adapters with int8 moments: A matrices have rows
    of 4096 or 11,008, B matrices rows of 16 (256 rows per workgroup, one lane
    per row); every element checked."""
    w = synth.WORKLOADS["llama7b_lora_r16"]
    cases = _workload_q8(L, w, last_dim, delta=True)
    step(L, cases, w.step)
    torch.cuda.synchronize()
    consts = oracle_consts(HP, w.step)
    for i, c in enumerate(cases):
        c.check(consts, f"lora{i}")


def test_gpt2_cattn_q8_full(L):
    """GPT-2 c_attn of the first two layers with int8 moments from a fresh
    state at t = 1 (all-zero rows to start); the 1-D biases are one row each."""
    w = synth.WORKLOADS["gpt2_cattn_first2"]
    cases = []
    for i, (label, shape) in enumerate(w.segments):
        c = Case(L, w.numels[i], shape[-1], 300000 + i, delta=True)
        zq = (np.zeros(c.n, np.int8), np.zeros(-(-c.n // c.row_len), np.float32))
        c.mq, c.vq = (zq[0].copy(), zq[1].copy()), (zq[0].copy(), zq[1].copy())
        c.m = L.Q8(up(c.mq[0]), up(c.mq[1]), c.row_len)
        c.v = L.Q8(up(c.vq[0]), up(c.vq[1]), c.row_len)
        cases.append(c)
    step(L, cases, 1)
    torch.cuda.synchronize()
    consts = oracle_consts(HP, 1)
    for i, c in enumerate(cases):
        c.check(consts, f"gpt2_{i}")
