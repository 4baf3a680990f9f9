"""Seeded synthetic inputs for the AdamW path: shapes, distributions, seeds.

This module serves both the GPU path (tests, bench) and the CPU oracle (via
host copies of the very same bytes).  It holds none of the optimizer's
arithmetic: it only draws random tensors and lays out segment lists.

Workloads (tensor shapes from the models the LEMA README trains):

* ``gpt2_cattn_first2``  -- GPT-2-small ``c_attn`` of the first 2 layers
  (README, "Selective Full Fine-Tuning", selection ``["c_attn"] x
  ["first:2"]``): per layer W [768 x 2304] and bias [2304]; 4 segments,
  3,543,552 parameters; step t = 1 from m = v = 0.
* ``llama7b_attn_last4``  -- Llama-2-7B q, k, v, o projections of the last
  4 decoder layers (README, same section, ``["q_proj", ...] x ["last:4"]``):
  16 segments of [4096 x 4096], 268,435,456 parameters; t = 100.
* ``llama7b_layer``  -- one Llama-2-7B decoder layer: q, k, v, o
  [4096 x 4096], gate and up [11008 x 4096], down [4096 x 11008], two RMSNorm
  weights [4096]; 9 segments, 202,383,360 parameters; 8 bf16 micro-batch
  gradients accumulated in fp32, then one step at t = 50.
* ``llama7b_full``  -- the whole Llama-2-7B shape: embedding [32000 x 4096],
  32 decoder layers as above, final RMSNorm [4096], LM head [32000 x 4096];
  291 segments, 6,738,415,616 parameters; t = 10.
* ``llama7b_lora_r16``  -- rank-16 LoRA adapters (README "Quick Start":
  ``lora_rank=16`` with torch.optim.AdamW over the adapters) on all seven
  linear projections of the 32 Llama-2-7B layers: per projection A
  [16 x in] and B [out x 16]; 448 segments, 39,976,960 parameters; t = 10.
* ``llama7b_full_shard8``  -- one data-parallel rank's share of the whole
  7B shape when each tensor's flat element range is split 8 ways (ZeRO-1/2
  style ownership): the first eighth of each of the 291 tensors, as 1-D
  segments; 842,301,952 parameters; t = 10.

Distributions: gradient bf16 = bf16(N(0, 1e-3)) (drawn in fp32, converted
by torch), master ~ N(0, 0.02), m ~ N(0, 1e-4), v = N(0, 1e-3)^2 (square of
an independent draw); the GPT-2 workload starts from m = v = 0.  sigma is a
standard deviation.  Hyperparameters: lr 1e-4, betas (0.9, 0.999), eps 1e-8,
weight decay 0.01 (README "Quick Start" sets lr; the rest are the defaults
of torch.optim.AdamW that it calls).

Seeds: tensor (workload w, array a, segment s) uses
``torch.Generator(device).manual_seed(1000*w + 100*a + s)`` with array ids
0 master, 1 m, 2 v, 30+k gradient of micro-batch k.  Segments beyond 99
fold into the same formula (the seed only has to be fixed, not unique).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

HPARAMS = dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)

ARRAY_MASTER, ARRAY_M, ARRAY_V = 0, 1, 2
ARRAY_GRAD0 = 30


@dataclass
class Workload:
    name: str
    wid: int                      # numeric id used in seeds
    segments: list                # [(label, shape tuple)]
    step: int                     # AdamW step number t being taken
    microbatches: int = 1         # bf16 gradients accumulated before the step
    fresh_state: bool = False     # m = v = 0
    description: str = ""
    sigma: dict = field(default_factory=lambda: dict(
        grad=1e-3, master=0.02, m=1e-4, v_root=1e-3))

    @property
    def numels(self):
        n = []
        for _, shape in self.segments:
            k = 1
            for d in shape:
                k *= d
            n.append(k)
        return n

    @property
    def params(self) -> int:
        return sum(self.numels)


def _llama_layer(prefix: str):
    h, f = 4096, 11008
    return [
        (f"{prefix}.self_attn.q_proj", (h, h)),
        (f"{prefix}.self_attn.k_proj", (h, h)),
        (f"{prefix}.self_attn.v_proj", (h, h)),
        (f"{prefix}.self_attn.o_proj", (h, h)),
        (f"{prefix}.mlp.gate_proj", (f, h)),
        (f"{prefix}.mlp.up_proj", (f, h)),
        (f"{prefix}.mlp.down_proj", (h, f)),
        (f"{prefix}.input_layernorm", (h,)),
        (f"{prefix}.post_attention_layernorm", (h,)),
    ]


def _gpt2_first2():
    segs = []
    for layer in range(2):
        segs.append((f"h.{layer}.attn.c_attn.weight", (768, 2304)))
        segs.append((f"h.{layer}.attn.c_attn.bias", (2304,)))
    return segs


def _llama_attn_last4():
    segs = []
    for layer in range(28, 32):
        for p in ("q_proj", "k_proj", "v_proj", "o_proj"):
            segs.append((f"layers.{layer}.self_attn.{p}", (4096, 4096)))
    return segs


def _llama_lora_r16():
    h, f, r = 4096, 11008, 16
    shapes = {"q_proj": (h, h), "k_proj": (h, h), "v_proj": (h, h), "o_proj": (h, h),
              "gate_proj": (f, h), "up_proj": (f, h), "down_proj": (h, f)}
    segs = []
    for layer in range(32):
        for name, (out_f, in_f) in shapes.items():
            segs.append((f"layers.{layer}.{name}.lora_A", (r, in_f)))
            segs.append((f"layers.{layer}.{name}.lora_B", (out_f, r)))
    return segs


def _llama_full():
    segs = [("embed_tokens", (32000, 4096))]
    for layer in range(32):
        segs += _llama_layer(f"layers.{layer}")
    segs.append(("norm", (4096,)))
    segs.append(("lm_head", (32000, 4096)))
    return segs


def shard_range(numel: int, ranks: int, rank: int) -> tuple[int, int]:
    """[begin, end) of the elements rank owns when a tensor's flat range is
    split into `ranks` contiguous pieces (the first numel % ranks get one
    extra element)."""
    q, r = divmod(numel, ranks)
    begin = rank * q + min(rank, r)
    return begin, begin + q + (1 if rank < r else 0)


def _llama_full_shard(ranks: int, rank: int):
    segs = []
    for label, shape in _llama_full():
        n = 1
        for d in shape:
            n *= d
        b, e = shard_range(n, ranks, rank)
        segs.append((f"{label}[{b}:{e}]", (e - b,)))
    return segs


def _llama_full_row_shard(ranks: int, rank: int):
    """Rank `rank`'s share when every tensor is split on whole rows (its last
    dimension is the row): int8 state keeps each row's codes with that row's
    scale, so a rank owns complete rows.  The row index range is split like
    shard_range splits elements; a 1-D tensor is one row and goes whole to
    rank 0."""
    segs = []
    for label, shape in _llama_full():
        rows = 1
        for d in shape[:-1]:
            rows *= d
        b, e = shard_range(rows, ranks, rank)
        if e > b:
            segs.append((f"{label}[rows {b}:{e}]", (e - b, shape[-1])))
    return segs


WORKLOADS = {
    "gpt2_cattn_first2": Workload(
        "gpt2_cattn_first2", 1, _gpt2_first2(), step=1, fresh_state=True,
        description="GPT-2-small c_attn of layers 0-1: 2x W[768x2304] + "
                    "2x b[2304], bf16 grad, t=1 from m=v=0"),
    "llama7b_attn_last4": Workload(
        "llama7b_attn_last4", 2, _llama_attn_last4(), step=100,
        description="Llama-2-7B q,k,v,o of the last 4 layers: 16x "
                    "[4096x4096], bf16 grad, t=100"),
    "llama7b_layer": Workload(
        "llama7b_layer", 3, _llama_layer("layers.0"), step=50, microbatches=8,
        description="one Llama-2-7B decoder layer (9 tensors), 8 bf16 "
                    "micro-batches accumulated in fp32, then the step, t=50"),
    "llama7b_full": Workload(
        "llama7b_full", 4, _llama_full(), step=10,
        description="whole Llama-2-7B shape, 291 tensors resident, bf16 "
                    "grad, t=10"),
    "llama7b_lora_r16": Workload(
        "llama7b_lora_r16", 5, _llama_lora_r16(), step=10,
        description="rank-16 LoRA adapters on all 7 linear projections of 32 "
                    "Llama-2-7B layers: 448 tensors, bf16 grad, t=10"),
    "llama7b_full_shard8": Workload(
        "llama7b_full_shard8", 6, _llama_full_shard(8, 0), step=10,
        description="one of 8 data-parallel ranks' share of the whole "
                    "Llama-2-7B shape: the first eighth of each of the 291 "
                    "tensors, bf16 grad, t=10"),
    "llama7b_full_rows_shard8": Workload(
        "llama7b_full_rows_shard8", 7, _llama_full_row_shard(8, 0), step=10,
        description="rank 0 of 8 data-parallel ranks' share of the whole "
                    "Llama-2-7B shape split on whole rows (the layout int8 "
                    "state shards in): the first eighth of each tensor's "
                    "rows, the 1-D norm weights whole, bf16 grad, t=10"),
}


def seed_of(wid: int, array: int, seg: int) -> int:
    return 1000 * wid + 100 * array + seg


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(n: int, sigma: float, seed: int, device) -> torch.Tensor:
    """fp32 N(0, sigma) of length n from a fixed seed."""
    out = torch.empty(n, dtype=torch.float32, device=device)
    out.normal_(mean=0.0, std=sigma, generator=_gen(device, seed))
    return out


def bf16_normal(n: int, sigma: float, seed: int, device) -> torch.Tensor:
    """bf16 tensor drawn as fp32 N(0, sigma) then converted by torch."""
    return normal(n, sigma, seed, device).to(torch.bfloat16)


def make_segment_state(w: Workload, seg: int, device, with_orig: bool = False,
                       grads: int | None = None):
    """Tensors of one segment: dict with master, m, v, grads [list], orig."""
    n = w.numels[seg]
    s = w.sigma
    out = {"master": normal(n, s["master"], seed_of(w.wid, ARRAY_MASTER, seg), device)}
    if w.fresh_state:
        out["m"] = torch.zeros(n, dtype=torch.float32, device=device)
        out["v"] = torch.zeros(n, dtype=torch.float32, device=device)
    else:
        out["m"] = normal(n, s["m"], seed_of(w.wid, ARRAY_M, seg), device)
        root = normal(n, s["v_root"], seed_of(w.wid, ARRAY_V, seg), device)
        out["v"] = root.mul_(root)
    k = w.microbatches if grads is None else grads
    out["grads"] = [bf16_normal(n, s["grad"], seed_of(w.wid, ARRAY_GRAD0 + j, seg), device)
                    for j in range(k)]
    if with_orig:
        # base checkpoint weight: the bf16 copy of the starting master
        out["orig"] = out["master"].to(torch.bfloat16)
    return out


def random_normal_like_sizes(sizes, sigma, seed, device, dtype=torch.float32):
    """A list of independent N(0, sigma) tensors with the given sizes."""
    outs = []
    for i, n in enumerate(sizes):
        t = normal(n, sigma, seed + i, device)
        outs.append(t.to(dtype) if dtype != torch.float32 else t)
    return outs
