"""The counter record bench.py reads for `roofline.traffic`
(profiles/adamw_counters.json): every entry's algorithmic bytes follow from
its workload's shapes, its bytes follow from the recorded counters and the
copy kernel's scale factors, and bench.py hands out an entry only for the
kernel sources and state layout it was measured on.  bench.py
--fold-counters, which writes the entries, is checked on made-up counter
files."""
from __future__ import annotations

import csv
import json

import pytest

import bench
import synth

REC = json.load(open(bench.COUNTERS))
COPY_KIB = 2 * (1 << 30) / 1024        # lema_measure_copy: 2 GiB read, 2 GiB written


def algorithmic(key: str) -> int:
    """Bytes per launch from the shapes: the fp32 step reads g (2 B), master,
    m, v (12 B) and writes master, m, v (12 B) and the bf16 weight (2 B),
    plus orig (2 B) in and delta (4 B) out; int8 moments replace 8 B of
    moments each way by 2 B of codes and 16 B of scales per row; merge reads
    a bf16 base and an fp32 delta and writes bf16."""
    wl, *mode = key.split(":")
    w = synth.WORKLOADS[wl]
    if mode == ["merge"]:
        return 8 * w.params
    if mode[0] == "q8":
        delta = mode[1] == "delta"
        return sum(n * (16 + (6 if delta else 0)) + 16 * -(-n // sh[-1])
                   for n, (_, sh) in zip(w.numels, w.segments))
    return w.params * (34 if mode[0] == "delta" else 28)


@pytest.mark.parametrize("key", sorted(REC["workloads"]))
def test_entry_is_consistent(key):
    e = REC["workloads"][key]
    assert e["algorithmic_bytes_per_launch"] == algorithmic(key)
    assert e["kernel"] == bench.counter_key_bytes(key)[0]
    assert e["fetch_factor"] == pytest.approx(e["copy_fetch_kib"] / COPY_KIB)
    assert e["write_factor"] == pytest.approx(e["copy_write_kib"] / COPY_KIB)
    assert e["read_bytes"] == pytest.approx(e["fetch_kib"] * 1024 / e["fetch_factor"])
    assert e["written_bytes"] == pytest.approx(e["write_kib"] * 1024 / e["write_factor"])
    total = e["read_bytes"] + e["written_bytes"]
    assert e["traffic_bytes_per_launch"] == pytest.approx(total)
    assert e["traffic_over_algorithmic"] == pytest.approx(total / algorithmic(key))
    # a streaming kernel moves each byte once: within 1% of the algorithmic bytes
    assert 0.99 < e["traffic_over_algorithmic"] < 1.01


@pytest.mark.parametrize("key", sorted(REC["workloads"]))
def test_lookup_checks_layout_and_sources(monkeypatch, key):
    e = REC["workloads"][key]
    if e.get("kernel_digest") != bench.kernel_digest(e["kernel"]):
        assert bench.traffic_for(key, "flat") is None
        return
    assert bench.traffic_for(key, e["layout"]) == e["traffic_bytes_per_launch"]
    other = "per-tensor" if e["layout"] == "flat" else "flat"
    assert bench.traffic_for(key, other) is None
    assert bench.traffic_for(key + ":unknown", e["layout"]) is None
    monkeypatch.setattr(bench, "kernel_digest", lambda kernel: "0" * 64)
    assert bench.traffic_for(key, e["layout"]) is None


COPY_GRID = 2 * (1 << 30) // 16        # work-items of the 2 GiB reference copy


def _counter_csv(path, counter, rows):
    """A rocprofv3 counter_collection CSV with the columns fold_counters
    reads; rows are (dispatch, kernel, value[, grid])."""
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size",
                                           "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for d, k, v, *g in rows:
            wr.writerow({"Dispatch_Id": d, "Kernel_Name": k,
                         "Grid_Size": g[0] if g else COPY_GRID, "Counter_Name": counter,
                         "Counter_Value": v})


def test_fold_counters(tmp_path, monkeypatch):
    rec_path = tmp_path / "counters.json"
    rec_path.write_text(json.dumps({"workloads": {"stale:delta": {"kernel": "adamw_tile_kernel",
                                                                  "kernel_digest": "x"}}}))
    monkeypatch.setattr(bench, "COUNTERS", str(rec_path))
    key = "llama7b_attn_last4:delta"
    alg = algorithmic(key)
    # FETCH_SIZE counts half the bytes read; each dispatch's value is split
    # over two counter instances; WRITE_SIZE counts the bytes written
    read, written = 16 * alg // 34, 18 * alg // 34
    fetch = [(1, "copy_kernel", COPY_KIB / 2 / 2), (1, "copy_kernel", COPY_KIB / 2 / 2)]
    write = [(1, "copy_kernel", COPY_KIB)]
    # a smaller copy of the same kernel (bench.py's same_bytes_copy) is not
    # the reference
    fetch += [(9, "copy_kernel", 1000.0, 4096)]
    write += [(9, "copy_kernel", 2000.0, 4096)]
    for d in (2, 3):
        fetch += [(d, "adamw_tile_kernel", read / 1024 / 2 / 2)] * 2
        write += [(d, "adamw_tile_kernel", written / 1024)]
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.fold_counters(key, str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    rec = json.loads(rec_path.read_text())
    assert list(rec["workloads"]) == [key]          # the stale entry is dropped
    e = rec["workloads"][key]
    assert e["dispatches"] == 2
    assert e["fetch_factor"] == pytest.approx(0.5)
    assert e["write_factor"] == pytest.approx(1.0)
    assert e["read_bytes"] == pytest.approx(read)
    assert e["written_bytes"] == pytest.approx(written)
    assert e["traffic_over_algorithmic"] == pytest.approx(1.0)
    assert e["kernel_digest"] == bench.kernel_digest("adamw_tile_kernel")
    assert bench.traffic_for(key, "flat") == pytest.approx(alg)
    with pytest.raises(SystemExit):
        bench.counter_key_bytes("llama7b_layer:delta")   # a multi-launch step has no entry


def test_fold_counters_two_launches_per_step(tmp_path, monkeypatch):
    """A step of two launches of different grid sizes (the int8 step over
    rows of 4096 and rows of 11,008): the entry holds the bytes of a whole
    step, the sum over its launches, not the mean of one dispatch."""
    rec_path = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS", str(rec_path))
    key = "llama7b_full:q8:delta"
    alg = algorithmic(key)
    parts = [(0.7, 1000), (0.3, 4000)]                 # share of the bytes, grid size
    fetch = [(1, "copy_kernel", COPY_KIB / 2)]
    write = [(1, "copy_kernel", COPY_KIB)]
    d = 2
    for _ in range(3):                                 # three steps
        for share, grid in parts:
            fetch.append((d, "adamw_q8_kernel", share * alg * 10 / 22 / 1024 / 2, grid))
            write.append((d, "adamw_q8_kernel", share * alg * 12 / 22 / 1024, grid))
            d += 1
    _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.fold_counters(key, str(tmp_path / "f.csv"), str(tmp_path / "w.csv"))
    e = json.loads(rec_path.read_text())["workloads"][key]
    assert e["dispatches"] == 6 and e["steps"] == 3 and e["launches_per_step"] == 2
    assert e["traffic_over_algorithmic"] == pytest.approx(1.0)
