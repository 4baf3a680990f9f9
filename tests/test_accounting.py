"""P10: the 16-bytes-per-parameter state layout and the workload sizes.

The LLMScale fine-tuning VRAM page fixes mixed-precision Adam at 16 bytes per
trained parameter (bf16 weight 2 + bf16 gradient 2 + fp32 master, m, v 12)
and prints worked totals; tests/golden/accounting.json holds them.
"""
import json
import os

import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accounting.json")


def test_page_examples():
    g = json.load(open(GOLDEN))
    parts = g["bytes_per_trained_param"]
    assert parts["total"] == sum(v for k, v in parts.items() if k != "total") == 16
    f = g["formula_bytes_per_param"]
    assert f["grads"] + f["adam"] + f["base_bf16"] == parts["total"]
    for ex in g["examples"]:
        gib = ex["params"] * ex["bytes_per_param"] / 2 ** 30
        assert abs(gib - ex["gib"]) <= ex["tol_gib"], ex


def test_state_layout_is_16_bytes():
    # arrays the AdamW path keeps per trained parameter (dtype sizes)
    layout = {"weight_bf16": 2, "grad_bf16": 2, "master_f32": 4, "m_f32": 4, "v_f32": 4}
    assert sum(layout.values()) == json.load(open(GOLDEN))["bytes_per_trained_param"]["total"]


@pytest.mark.parametrize("name,params,nseg", [
    ("gpt2_cattn_first2", 3_543_552, 4),
    ("llama7b_attn_last4", 268_435_456, 16),
    ("llama7b_layer", 202_383_360, 9),
    ("llama7b_full", 6_738_415_616, 291),
    ("llama7b_lora_r16", 39_976_960, 448),
    ("llama7b_full_shard8", 842_301_952, 291),
    ("llama7b_full_rows_shard8", 842_534_912, 291),
])
def test_workload_sizes(name, params, nseg):
    w = synth.WORKLOADS[name]
    assert w.params == params and len(w.segments) == nseg


def test_resident_and_slot_footprints():
    full = synth.WORKLOADS["llama7b_full"].params * 16
    assert abs(full / 1e9 - 107.81) < 0.01                 # about 108 GB resident
    slot = synth.WORKLOADS["llama7b_layer"].params * 16
    assert abs(slot / 1e9 - 3.238) < 0.001                 # one layer slot
    assert full < 288e9 / 1.3                              # room for orig + delta on one GPU


@pytest.mark.parametrize("numel", [0, 1, 7, 8, 9, 4096 * 3 + 5, 32000 * 4096])
@pytest.mark.parametrize("ranks", [1, 2, 3, 8])
def test_shard_ranges_partition(numel, ranks):
    """Rank ranges are contiguous, in order, cover every element once and
    differ in length by at most one."""
    ranges = [synth.shard_range(numel, ranks, k) for k in range(ranks)]
    assert ranges[0][0] == 0 and ranges[-1][1] == numel
    assert all(a[1] == b[0] for a, b in zip(ranges, ranges[1:]))
    lens = [e - b for b, e in ranges]
    assert min(lens) >= 0 and max(lens) - min(lens) <= 1 and sum(lens) == numel


def test_shard_workload_is_the_first_eighth():
    full, shard = synth.WORKLOADS["llama7b_full"], synth.WORKLOADS["llama7b_full_shard8"]
    assert shard.numels == [synth.shard_range(n, 8, 0)[1] for n in full.numels]
    assert shard.params * 8 == full.params


def test_row_shards_are_whole_rows_and_partition_the_model():
    """Splitting on whole rows: every rank's segments are complete rows of
    their tensor, the 8 ranks together hold every parameter once, and rank 0
    holds an eighth of every 2-D tensor (all of them split evenly) plus the
    65 norm weights whole: 6,738,415,616 / 8 + 7/8 * 65 * 4096."""
    full = synth.WORKLOADS["llama7b_full"]
    shapes = dict(full.segments)
    total = 0
    for rank in range(8):
        segs = synth._llama_full_row_shard(8, rank)
        for label, (rows, row_len) in segs:
            assert row_len == shapes[label.split("[")[0]][-1]
        total += sum(rows * row_len for _, (rows, row_len) in segs)
        if rank:
            assert len(segs) == 291 - 65           # the norm rows stay on rank 0
    assert total == full.params
    w = synth.WORKLOADS["llama7b_full_rows_shard8"]
    assert w.segments == synth._llama_full_row_shard(8, 0)
    assert w.params == full.params // 8 + 7 * 65 * 4096 // 8
