"""The counter record bench.py reads for `roofline.traffic`
(profiles/adamw_counters.json): every entry's algorithmic bytes follow from
its workload's shapes, its bytes follow from the recorded counters and the
copy kernel's scale factors, and bench.py hands out an entry only for the
kernel sources and state layout it was measured on."""
from __future__ import annotations

import json

import pytest

import bench
import synth

REC = json.load(open(bench.COUNTERS))
COPY_KIB = 2 * (1 << 30) / 1024        # lema_measure_copy: 2 GiB read, 2 GiB written


def algorithmic(key: str) -> int:
    wl, *mode = key.split(":")
    w = synth.WORKLOADS[wl]
    if mode == ["merge"]:
        return 8 * w.params                 # bf16 base + fp32 delta in, bf16 out
    if mode[0] == "q8":
        return sum(bench.q8_step_bytes(n, -(-n // sh[-1]), "bf16", mode[1] == "delta")
                   for n, (_, sh) in zip(w.numels, w.segments))
    return w.params * bench.adamw_bytes_per_param(False, mode[0] == "delta")


@pytest.mark.parametrize("key", sorted(REC["workloads"]))
def test_entry_is_consistent(key):
    e = REC["workloads"][key]
    assert e["algorithmic_bytes_per_launch"] == algorithmic(key)
    assert e["fetch_factor"] == pytest.approx(e["copy_fetch_kib"] / COPY_KIB)
    assert e["write_factor"] == pytest.approx(e["copy_write_kib"] / COPY_KIB)
    assert e["read_bytes"] == pytest.approx(e["fetch_kib"] * 1024 / e["fetch_factor"])
    assert e["written_bytes"] == pytest.approx(e["write_kib"] * 1024 / e["write_factor"])
    total = e["read_bytes"] + e["written_bytes"]
    assert e["traffic_bytes_per_launch"] == pytest.approx(total)
    assert e["traffic_over_algorithmic"] == pytest.approx(total / algorithmic(key))
    # a streaming kernel moves each byte once: within 1% of the algorithmic bytes
    assert 0.99 < e["traffic_over_algorithmic"] < 1.01


def test_lookup_checks_layout_and_sources(monkeypatch):
    key = "llama7b_attn_last4:delta"
    if REC["kernel_digest"] != bench.kernel_digest():
        assert bench.traffic_for(key, "flat") is None
        return
    assert bench.traffic_for(key, "flat") == REC["workloads"][key]["traffic_bytes_per_launch"]
    assert bench.traffic_for(key, "per-tensor") is None
    assert bench.traffic_for("llama7b_attn_last4:unknown", "flat") is None
    monkeypatch.setattr(bench, "kernel_digest", lambda: "0" * 64)
    assert bench.traffic_for(key, "flat") is None
