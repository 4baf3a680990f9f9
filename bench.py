#!/usr/bin/env python3
"""Benchmark of the mixed-precision AdamW hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-delta]
    python bench.py --slot-stream [--layers L]

A step is one pass of the hot path over the whole workload on inputs already
resident in HBM: for one micro-batch, one lema_adamw_step call (constants,
segment walk, AdamW, bf16 write-back and, by default, the fp32 delta); for
the one-layer workload, 8 lema_grad_accum calls then the step on the fp32
accumulator.  The default workload is the whole Llama-2-7B shape resident in
HBM (291 tensors, 6,738,415,616 parameters, bf16 gradient, t = 10, delta on:
229 GB of HBM traffic per step), the largest selection of the LEMA README's
"Selective Full Fine-Tuning" section ("the entire model") that fits one GPU.
`--workload llama7b_attn_last4` is its example selection (q, k, v, o of the
last 4 layers, 268,435,456 parameters, t = 100).

--fold-counters KEY FETCH_CSV WRITE_CSV folds two rocprofv3 --pmc passes
(FETCH_SIZE, then WRITE_SIZE, of the same bench command) into the counter
record bench.py reads for roofline.traffic; it needs no GPU.

--slot-stream streams the whole Llama-2-7B shape from page-locked host
memory through two HBM slots (README "TensorStore", "Features") and reports
copy GB/s next to kernel time.

Prints one JSON line: parameters updated per second (value), HBM GB/s and
fraction of the 8 TB/s peak, the roofline of the AdamW kernel (per-launch
time from HIP events on its stream), the plain-copy ceiling of the same GPU,
and the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import statistics
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
METRIC = "AdamW params updated/sec + achieved HBM GB/s (% of MI355X peak), 1 GPU"
COUNTERS = os.path.join(ROOT, "profiles", "adamw_counters.json")
# the traffic counters of a kernel stand for it as built from these sources
# with the build's compiler flags (optimizer_step_lema_amd.build.FLAGS)
_CSRC = "optimizer_step_lema_amd/csrc/"
KERNEL_SOURCES = {
    "adamw_tile_kernel": [_CSRC + "lema_kernels.hip", _CSRC + "lema_device.h",
                          _CSRC + "lema_internal.h"],
    "merge_tile_kernel": [_CSRC + "lema_kernels.hip", _CSRC + "lema_device.h",
                          _CSRC + "lema_internal.h"],
    "adamw_q8_kernel": [_CSRC + "lema_q8.hip", _CSRC + "lema_device.h",
                        _CSRC + "lema_internal.h"],
}


def kernel_digest(kernel: str) -> str:
    from optimizer_step_lema_amd import build
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    h.update(" ".join(build.FLAGS).encode())
    return h.hexdigest()


def adamw_bytes_per_param(grad_f32: bool, delta: bool) -> int:
    # reads: grad, master, m, v (+ orig); writes: master, m, v, weight (+ delta)
    read = (4 if grad_f32 else 2) + 12 + (2 if delta else 0)
    write = 12 + 2 + (4 if delta else 0)
    return read + write


ACCUM_BYTES_OVERWRITE = 6      # read bf16 g, write fp32 acc
ACCUM_BYTES = 10               # read bf16 g and fp32 acc, write fp32 acc


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b_full")
    ap.add_argument("--no-delta", action="store_true", help="time the step without the delta")
    ap.add_argument("--fused-last", action="store_true",
                    help="multi-micro-batch workloads: fold the last micro-batch into the step "
                         "(lema_adamw_step_accum) instead of a separate accumulation pass")
    ap.add_argument("--resident-microbatches", action="store_true",
                    help="multi-micro-batch workloads: all K bf16 gradients stay resident and the "
                         "step sums them in fp32 (lema_adamw_step_microbatches), no accumulator")
    ap.add_argument("--layout", choices=("flat", "per-tensor"), default="flat",
                    help="flat: one buffer per array kind, tensors as views (flat optimizer "
                         "state); per-tensor: every array of every tensor allocated on its own")
    ap.add_argument("--stagger", type=int, default=4096,
                    help="flat layout: the k-th array kind's buffer starts k * STAGGER bytes "
                         "into its allocation (a multiple of 256; 0 = no offsets)")
    ap.add_argument("--state-sets", type=int, default=0,
                    help="resident and int8 benches: rotate over N copies of the workload's "
                         "state, one per timed launch in turn (0 = enough copies for 1 GiB of "
                         "traffic per rotation, at least 1)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-gib", type=float, default=4.0, help="size of the copy-ceiling test")
    ap.add_argument("--merge", action="store_true",
                    help="time lema_merge_delta (base + delta -> servable bf16) on the workload")
    ap.add_argument("--checkpoint", metavar="DIR", default=None,
                    help="time lema_checkpoint_save and lema_checkpoint_load of the "
                         "workload's master, m, v and delta to a file in DIR")
    ap.add_argument("--q8", action="store_true",
                    help="int8 moments with per-row scales (and int8 accumulators for "
                         "multi-micro-batch workloads), README 'Quantization'")
    ap.add_argument("--slot-stream", action="store_true",
                    help="stream the whole 7B shape from pinned host memory through 2 HBM slots")
    ap.add_argument("--layers", type=int, default=0,
                    help="with --slot-stream: stream only the first L loads (0 = all 34)")
    ap.add_argument("--duplex", action="store_true",
                    help="with --slot-stream: slot -> host copies on a stream of their own")
    ap.add_argument("--slots", type=int, default=2,
                    help="with --slot-stream: HBM slots in the pool (default 2)")
    ap.add_argument("--host-gib", type=float, default=0.0,
                    help="with --slot-stream: host state to stage at most (default: 56 GiB "
                         "page-locked, 120 GiB with --staged)")
    ap.add_argument("--staged", action="store_true",
                    help="with --slot-stream: host state in ordinary (pageable) memory, moved "
                         "through the pool's page-locked staging buffers")
    ap.add_argument("--host-threads", type=int, default=0,
                    help="with --staged: host copy threads (0 = library default)")
    ap.add_argument("--fold-counters", nargs=3, metavar=("KEY", "FETCH_CSV", "WRITE_CSV"),
                    default=None,
                    help="fold rocprofv3 FETCH_SIZE and WRITE_SIZE passes (counter_collection "
                         "CSVs) into the counter record under KEY, e.g. llama7b_full:delta, "
                         "llama7b_attn_last4:q8:delta or gpt2_cattn_first2:merge")
    return ap.parse_args()


def progress(msg):
    print(f"bench.py: {msg}", file=sys.stderr, flush=True)


def timed_events(torch, stream, fn, n):
    """Run fn(k) n times, each bracketed by its own event pair; returns ms list."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for k in range(n):
        evs[k][0].record(stream)
        fn(k)
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def copy_ceiling(torch, L, gib):
    """Read+write GB/s of the library's plain copy kernel (nbytes each way)."""
    nbytes = int(gib * (1 << 30)) // 2 // 4096 * 4096
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    for _ in range(3):
        L.measure_copy(src, dst, nbytes)
    torch.cuda.synchronize()
    ms = timed_events(torch, torch.cuda.current_stream(),
                      lambda k: L.measure_copy(src, dst, nbytes), 10)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (sum(ms) / len(ms) * 1e-3) / 1e9


def traffic_for(key, layout):
    """Counter-measured HBM bytes per launch, if recorded for this kernel
    source and state layout."""
    if not os.path.exists(COUNTERS):
        return None
    rec = json.load(open(COUNTERS))
    entry = rec.get("workloads", {}).get(key)
    if entry and entry.get("kernel_digest") == kernel_digest(entry["kernel"]) and \
            entry.get("layout", "per-tensor") == layout:
        return entry["traffic_bytes_per_launch"]
    return None


def counter_key_bytes(key):
    """(kernel name, algorithmic bytes per launch) of a counter-record key
    "<workload>:delta", ":nodelta", ":q8:delta", ":q8:nodelta" or ":merge"."""
    import synth
    wl, *mode = key.split(":")
    w = synth.WORKLOADS[wl]
    if mode == ["merge"]:
        return "merge_tile_kernel", 8 * w.params
    if mode and mode[0] == "q8" and len(mode) == 2 and mode[1] in ("delta", "nodelta"):
        return "adamw_q8_kernel", sum(
            q8_step_bytes(n, -(-n // sh[-1]), "bf16", mode[1] == "delta")
            for n, (_, sh) in zip(w.numels, w.segments))
    if mode in (["delta"], ["nodelta"]) and w.microbatches == 1:
        return "adamw_tile_kernel", w.params * adamw_bytes_per_param(False, mode[0] == "delta")
    raise SystemExit(f"bench.py: --fold-counters: unknown key {key!r}")


COPY_KIB = 2 * (1 << 30) / 1024          # lema_measure_copy in copy_ceiling: 2 GiB each way


def fold_counters(key, fetch_csv, write_csv):
    """FETCH_SIZE and WRITE_SIZE per step (KiB, summed over the counter's
    instances and over the step's launches of the key's kernel), each scaled
    by what the same counter read for the copy kernel's known 2 GiB read +
    2 GiB write in the same run, into the record's entry for `key`, stamped
    with the digest of the kernel's current sources (entries whose kernel
    has changed since are dropped).  A step's launches are told apart by
    their grid sizes: each appears once per step, so the number of steps is
    the smallest count of dispatches of one grid size (steps whose launches
    share a grid size are counted as one launch per step)."""
    import csv

    def per_step(path, kernel, counter, grid=None):
        vals, grids = {}, {}
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Kernel_Name"].strip('"') != kernel or row["Counter_Name"] != counter:
                    continue
                if grid is not None and int(row["Grid_Size"]) != grid:
                    continue
                d = row["Dispatch_Id"]
                vals[d] = vals.get(d, 0.0) + float(row["Counter_Value"])
                grids[d] = int(row["Grid_Size"])
        if not vals:
            raise SystemExit(f"bench.py: no {counter} rows for {kernel} in {path}")
        per_grid = {}
        for d, g in grids.items():
            per_grid[g] = per_grid.get(g, 0) + 1
        steps = min(per_grid.values())
        return sum(vals.values()) / steps, steps, len(vals) / steps

    kernel, alg = counter_key_bytes(key)
    layout = "flat"
    fk, nd, launches = per_step(fetch_csv, kernel, "FETCH_SIZE")
    wk, _, _ = per_step(write_csv, kernel, "WRITE_SIZE")
    # the reference is copy_ceiling's copy of 2 GiB each way (one 16-byte
    # vector per work-item); small workloads also run same_bytes_copy
    ref_grid = int(COPY_KIB * 1024) // 16
    cf, _, _ = per_step(fetch_csv, "copy_kernel", "FETCH_SIZE", ref_grid)
    cw, _, _ = per_step(write_csv, "copy_kernel", "WRITE_SIZE", ref_grid)
    ff, wf = cf / COPY_KIB, cw / COPY_KIB
    read, written = fk * 1024 / ff, wk * 1024 / wf
    rec = json.load(open(COUNTERS)) if os.path.exists(COUNTERS) else {}
    # entries measured on kernels built from other sources no longer count
    rec["workloads"] = {k: e for k, e in rec.get("workloads", {}).items()
                        if e.get("kernel_digest") == kernel_digest(e["kernel"])}
    rec.pop("kernel_digest", None)
    rec["note"] = ("HBM bytes per dispatch from two rocprofv3 --pmc passes (FETCH_SIZE, then "
                   "WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads "
                   "for lema_measure_copy of 2 GiB read + 2 GiB write in the same run")
    rec["commands"] = [
        "rocprofv3 --pmc FETCH_SIZE -T -f csv -d <out>/pmc_fetch -o fetch -- python3 "
        "<repo>/bench.py --steps 5 --warmup 1 --no-cpu-baseline --copy-gib 4 "
        "[--workload W] [--no-delta | --q8 | --merge]",
        "rocprofv3 --pmc WRITE_SIZE -T -f csv -d <out>/pmc_write -o write -- python3 "
        "<repo>/bench.py --steps 5 --warmup 1 --no-cpu-baseline --copy-gib 4 "
        "[--workload W] [--no-delta | --q8 | --merge]",
        "python3 <repo>/bench.py --fold-counters KEY <out>/pmc_fetch/fetch_counter_collection.csv "
        "<out>/pmc_write/write_counter_collection.csv"]
    rec["kernel_sources"] = {k: v + ["compiler flags: optimizer_step_lema_amd.build.FLAGS"]
                             for k, v in KERNEL_SOURCES.items()}
    rec["workloads"][key] = {
        "kernel": kernel, "kernel_digest": kernel_digest(kernel), "layout": layout,
        "dispatches": round(nd * launches), "steps": nd, "launches_per_step": launches,
        "fetch_kib": fk, "write_kib": wk,
        "copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_factor": ff, "write_factor": wf,
        "read_bytes": read, "written_bytes": written,
        "traffic_bytes_per_launch": read + written,
        "algorithmic_bytes_per_launch": alg,
        "traffic_over_algorithmic": (read + written) / alg}
    rec["workloads"] = dict(sorted(rec["workloads"].items()))
    with open(COUNTERS, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps({key: rec["workloads"][key]}))


def main():
    a = parse()
    if a.fold_counters:
        fold_counters(*a.fold_counters)
        return
    if a.gpus != 1:
        print(f"bench.py: --gpus {a.gpus}: only one GPU is supported; the data-parallel "
              "(sharded) layout is measured on one rank's share instead "
              "(--workload llama7b_full_shard8)", file=sys.stderr)
        sys.exit(2)
    if a.stagger < 0 or a.stagger % 256:
        print(f"bench.py: --stagger {a.stagger}: a non-negative multiple of 256 bytes is needed",
              file=sys.stderr)
        sys.exit(2)
    if a.slots < 2:
        print(f"bench.py: --slots {a.slots}: a slot pool needs at least 2 slots", file=sys.stderr)
        sys.exit(2)
    if a.state_sets < 0:
        print(f"bench.py: --state-sets {a.state_sets}: 0 (automatic) or a positive count is "
              "needed", file=sys.stderr)
        sys.exit(2)

    import torch
    import optimizer_step_lema_amd as L
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)
    if a.slot_stream:
        line = slot_stream_bench(torch, L, synth, a)
    elif a.checkpoint:
        line = checkpoint_bench(torch, L, synth, a)
    elif a.merge:
        line = merge_bench(torch, L, synth, a)
    elif a.q8:
        line = q8_bench(torch, L, synth, a)
    else:
        line = resident_bench(torch, L, synth, a)
    print(json.dumps(line), flush=True)


# ------------------------------------------------------------- resident

def resident_bench(torch, L, synth, a):
    dev = "cuda"
    w = synth.WORKLOADS[a.workload]
    delta = not a.no_delta
    hp = synth.HPARAMS
    P = w.params
    K = w.microbatches
    resident_mb = a.resident_microbatches and K > 1
    grad_f32 = K > 1 and not resident_mb
    fused = a.fused_last and K > 1 and not resident_mb
    step_bytes = adamw_bytes_per_param(grad_f32, delta) + (2 if fused else 0)
    if resident_mb:
        step_bytes += 2 * (K - 1)          # K bf16 gradients instead of one
    accum_launches = K - 1 if fused else K
    accum_bytes = (ACCUM_BYTES_OVERWRITE + (accum_launches - 1) * ACCUM_BYTES) \
        if K > 1 and not resident_mb else 0
    per_step = P * (step_bytes + accum_bytes)

    # state resident in HBM; small workloads get rotated copies so that the
    # working set exceeds the 256 MB last-level cache between launches
    nsets = a.state_sets or (max(1, -(-(1 << 30) // per_step)) if per_step < (1 << 30) else 1)
    t_setup = time.perf_counter()
    sets = [resident_state(torch, L, synth, w, a.layout, delta, grad_f32, resident_mb,
                           a.stagger)
            for _ in range(nsets)]
    torch.cuda.synchronize()
    progress(f"{a.workload}: {nsets} state set(s) of {P} params resident "
             f"({time.perf_counter() - t_setup:.1f} s)")
    stream = torch.cuda.current_stream()
    copy_gbps = copy_ceiling(torch, L, a.copy_gib)
    progress(f"copy ceiling {copy_gbps:.0f} GB/s")

    accum_plans = [[L.AccumPlan([L.AccumSegment(acc, g[j]) for acc, g in accs])
                    for j in range(accum_launches)] for _, accs, _ in sets] if grad_f32 else []

    def accumulate(k):
        for j, plan in enumerate(accum_plans[k % nsets]):
            plan.run(overwrite=(j == 0))

    # the step's arguments are marshalled once (a training loop's usage), so
    # the timed region holds the library call, not Python argument packing
    plans = [L.AdamwPlan(segs, last_grads=[g[K - 1] for _, g in accs] if fused else None,
                         microbatch_grads=[g for _, g in accs] if resident_mb else None)
             for segs, accs, _ in sets]

    def step(k):
        plans[k % nsets].step(step=w.step, **hp)

    def whole(k):
        if grad_f32:
            accumulate(k)
        step(k)

    # Each step is bracketed by its own pair of HIP events on the launch
    # stream, so steps do not overlap one another (the isolation the kernel
    # trace sees); the back-to-back rate, where one launch's tail overlaps the
    # next launch's start, is reported beside it as "pipelined".
    for k in range(a.warmup):
        whole(k)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    step_ms = timed_events(torch, stream, whole, a.steps)
    wall = time.perf_counter() - t_wall0
    ms = sum(step_ms) / len(step_ms)

    # the AdamW kernel alone, one launch per event pair
    if grad_f32:
        adamw_ms_list = timed_events(torch, stream, step, a.steps)
        accum_ms_list = timed_events(torch, stream, accumulate, a.steps)
    else:
        adamw_ms_list, accum_ms_list = step_ms, []
    adamw_ms = sum(adamw_ms_list) / len(adamw_ms_list)
    adamw_gbps = P * step_bytes / (adamw_ms * 1e-3) / 1e9

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for k in range(a.steps):
        whole(k)
    stop.record(stream)
    torch.cuda.synchronize()
    pipelined_ms = start.elapsed_time(stop) / a.steps
    progress(f"timed {a.steps} steps: {ms:.4f} ms per step")

    gbps = per_step / (ms * 1e-3) / 1e9
    key = f"{a.workload}:{'delta' if delta else 'nodelta'}" + (":fused" if fused else "") + \
        (":resident_mb" if resident_mb else "")
    info = L.device_info()
    line = {
        "metric": METRIC,
        "value": P / (ms * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": a.workload,
            "description": w.description,
            "params": P,
            "segments": len(w.segments),
            "grad": (f"{K} resident bf16 micro-batches summed in fp32 inside the step"
                     if resident_mb else ("fp32 accumulator of 8 bf16 micro-batches" +
                                          (", last one folded into the step" if fused else "")))
            if K > 1 else "bf16",
            "delta": delta,
            "step_t": w.step,
            "bytes_per_param": step_bytes + accum_bytes,
            "bytes_per_step": per_step,
            "rotated_state_sets": nsets,
            "layout": a.layout,
            "kind_offset_bytes": a.stagger if a.layout == "flat" else None,
        },
        "hbm_gbps": gbps,
        "pct_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
        "copy_ceiling_gbps": copy_gbps,
        "pct_copy_ceiling": 100.0 * gbps / copy_gbps,
        "roofline": {"bound": "hbm", "achieved": adamw_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": adamw_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic_for(key, a.layout), "kernel": "adamw_tile_kernel",
                     "algorithmic_bytes_per_launch": P * step_bytes,
                     "avg_launch_ms": adamw_ms, "min_launch_ms": min(adamw_ms_list),
                     "median_launch_ms": statistics.median(adamw_ms_list),
                     "max_launch_ms": max(adamw_ms_list)},
        "pipelined": {"ms_per_step": pipelined_ms,
                      "hbm_gbps": per_step / (pipelined_ms * 1e-3) / 1e9,
                      "params_per_s": P / (pipelined_ms * 1e-3)},
        "device": info,
        "host_wall_s_timed_region": wall,
    }
    if nsets > 1 or P * step_bytes < SMALL_STEP_BYTES:
        line["same_bytes_copy"] = same_bytes_copy(torch, L, stream, P * step_bytes, nsets, a.steps)
    if accum_ms_list:
        acc_ms = sum(accum_ms_list) / len(accum_ms_list)
        acc_gbps = P * accum_bytes / (acc_ms * 1e-3) / 1e9
        line["accumulation"] = {"kernel": "accum_tile_kernel", "launches_per_step": accum_launches,
                                "ms_per_step": acc_ms, "hbm_gbps": acc_gbps,
                                "frac": acc_gbps / HBM_PEAK_GBPS,
                                "algorithmic_bytes_per_step": P * accum_bytes}
    if not a.no_cpu_baseline:
        progress("timing the oracle on the host")
        line["cpu_baseline"] = cpu_baseline(sets[0][0], w, hp, delta, a.cpu_seconds,
                                            sets[0][1][0][1] if resident_mb else None,
                                            bytes_per_param=step_bytes + accum_bytes)
    return line


# steps that move less than this also time a plain copy of their bytes: the
# ramp and drain of such a launch are a visible part of it
SMALL_STEP_BYTES = 2 << 30


def same_bytes_copy(torch, L, stream, nbytes, nsets, steps):
    """The plain copy kernel moving the step's bytes (half read, half
    written) per launch, rotated over `nsets` buffer pairs like the step's
    state sets: the floor a launch of this size has, ramp and drain
    included, when every byte moves once."""
    half = nbytes // 2 // 4096 * 4096
    pairs = [(torch.empty(half, dtype=torch.uint8, device="cuda"),
              torch.empty(half, dtype=torch.uint8, device="cuda")) for _ in range(nsets)]
    for src, _ in pairs:
        src.fill_(1)
    run = lambda k: L.measure_copy(pairs[k % nsets][0], pairs[k % nsets][1], half)
    for k in range(5):
        run(k)
    torch.cuda.synchronize()
    ms = timed_events(torch, stream, run, steps)
    avg = sum(ms) / len(ms)
    return {"kernel": "copy_kernel", "bytes_per_launch": 2 * half, "rotated_buffer_pairs": nsets,
            "avg_launch_ms": avg, "median_launch_ms": statistics.median(ms),
            "min_launch_ms": min(ms), "gbps": 2 * half / (avg * 1e-3) / 1e9}


def resident_state(torch, L, synth, w, layout, delta, grad_f32, resident_mb, stagger=4096):
    """One state set of the workload on the GPU: (segments, [(accumulator or
    None, [bf16 micro-batch gradients])]) plus the buffers that back them.

    The values are the seeded synthetic draws either way; `layout` only
    decides where they live: "flat" puts each array kind of all tensors in
    one buffer, "per-tensor" allocates every array of every tensor alone."""
    dev = "cuda"
    K = w.microbatches
    accs = []
    if layout == "flat":
        nmb = K if (grad_f32 or resident_mb) else 0
        fs, segs = L.flat_adamw_state(
            w.numels, grad=None if resident_mb else (torch.float32 if grad_f32 else torch.bfloat16),
            delta=delta, microbatches=nmb, device=dev, stagger=stagger)
        for i in range(len(w.segments)):
            st = synth.make_segment_state(w, i, dev, with_orig=delta)
            s = segs[i]
            s.master.copy_(st["master"])
            s.exp_avg.copy_(st["m"])
            s.exp_avg_sq.copy_(st["v"])
            if delta:
                s.orig.copy_(st["orig"])
            if nmb:
                mbs = [fs.view(f"mb{k}", i) for k in range(K)]
                for dst, src in zip(mbs, st["grads"]):
                    dst.copy_(src)
                accs.append((s.grad if grad_f32 else None, mbs))
            else:
                s.grad.copy_(st["grads"][0])
            del st
        return segs, accs, fs
    segs = []
    for i in range(len(w.segments)):
        st = synth.make_segment_state(w, i, dev, with_orig=delta)
        n = w.numels[i]
        grad = torch.empty(n, device=dev) if grad_f32 else st["grads"][0]
        if grad_f32 or resident_mb:
            accs.append((grad, st["grads"]))
        if resident_mb:
            grad = None
        segs.append(L.AdamwSegment(st["master"], st["m"], st["v"], grad,
                                   torch.empty(n, dtype=torch.bfloat16, device=dev),
                                   st.get("orig"),
                                   torch.empty(n, device=dev) if delta else None))
    return segs, accs, None


def cpu_baseline(segs, w, hp, delta, seconds, microbatches=None, bytes_per_param=None):
    """Time the oracle (as it stands) on the first tensor of the workload;
    with `microbatches` (its resident bf16 gradients) each timed step is the
    oracle's accumulation of them followed by the step.  `bytes_per_param`,
    the GPU line's algorithmic bytes, turns params/s into GB/s."""
    import numpy as np
    import oracle
    import torch

    def host_copy(t):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view("uint16").copy()
        return t.numpy().copy()

    s = segs[0]
    master, m, v = host_copy(s.master), host_copy(s.exp_avg), host_copy(s.exp_avg_sq)
    orig = host_copy(s.orig) if delta else None
    n = master.shape[0]
    c = oracle.adamw_constants(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                               hp["weight_decay"], w.step)
    if microbatches is None:
        grad = host_copy(s.grad)
        one_step = lambda: oracle.adamw_step(master, m, v, grad, c, orig=orig)
    else:
        gs = [host_copy(g) for g in microbatches]
        acc = np.empty(n, np.float32)

        def one_step():
            for k, g in enumerate(gs):
                oracle.grad_accum(acc, g, overwrite=(k == 0))
            oracle.adamw_step(master, m, v, acc, c, orig=orig)
    one_step()                                                 # warm-up pass
    reps, el = timed_loop(one_step, seconds)
    cores = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        reps1, el1 = timed_loop(one_step, seconds / 4)
    finally:
        oracle.set_num_threads(cores)
    rate, rate1 = n * reps / el, n * reps1 / el1
    gbps = (lambda r: r * bytes_per_param / 1e9) if bytes_per_param else (lambda r: None)
    return {"value": rate, "unit": "params/s", "cores": cores, "gbps": gbps(rate),
            "kind": "oracle", "host": host_info(),
            "sample": f"{w.segments[0][0]} ({n} params), {reps} oracle steps in {el:.1f} s, "
                      f"delta {'on' if delta else 'off'}"
                      + (f", each with {len(microbatches)} accumulations" if microbatches else "")
                      + "; C oracle, OpenMP",
            "single_thread": {"value": rate1, "unit": "params/s", "cores": 1,
                              "gbps": gbps(rate1),
                              "sample": f"the same step, {reps1} times in {el1:.1f} s"}}


def host_info():
    """CPU model, logical CPUs and RAM of the host the oracle ran on."""
    info = {"logical_cpus": os.cpu_count()}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu"] = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    info["ram_gib"] = round(int(line.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:
        pass
    return info


def timed_loop(fn, seconds):
    """Runs fn until `seconds` have passed; returns (calls, elapsed s)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return reps, el


# ------------------------------------------------------------- int8

def q8_step_bytes(numel, rows, grad, delta):
    """Algorithmic bytes of one int8-moment step over one tensor: master
    read+write, m and v codes read+write, their row scales read+write, the
    gradient (bf16, or int8 codes plus row scales), bf16 weight, orig+delta."""
    per = 8 + 2 + 2 + 2 + (6 if delta else 0) + (2 if grad == "bf16" else 1)
    return numel * per + rows * (16 + (4 if grad == "q8" else 0))


def q8_accum_bytes(numel, rows, overwrite):
    """int8 accumulation of one bf16 micro-batch: read g, (read codes and
    scales,) write codes and scales."""
    return numel * (3 if overwrite else 4) + rows * (4 if overwrite else 8)


def q8_bench(torch, L, synth, a):
    """The step with int8 moments (README "Quantization", opt_state_bits = 8);
    multi-micro-batch workloads also accumulate into int8 (grad_acc_bits = 8)."""
    dev = "cuda"
    w = synth.WORKLOADS[a.workload]
    delta = not a.no_delta
    hp = synth.HPARAMS
    P = w.params
    K = w.microbatches
    grad = "q8" if K > 1 else "bf16"
    row_lens = [shape[-1] for _, shape in w.segments]
    from optimizer_step_lema_amd._native import LEMA_Q8_MAX_ROW
    if max(row_lens) > LEMA_Q8_MAX_ROW:
        # e.g. the rank-share workload: its segments are element ranges of the
        # flattened tensors, while int8 state is sharded on whole rows (a rank
        # owns complete rows and their scales)
        print(f"bench.py: --q8 --workload {a.workload}: its segments are 1-D element "
              f"ranges (rows of up to {max(row_lens)} elements, the limit is "
              f"{LEMA_Q8_MAX_ROW}); int8 state shards on whole rows", file=sys.stderr)
        sys.exit(2)
    rows = [-(-n // rl) for n, rl in zip(w.numels, row_lens)]
    step_bytes = sum(q8_step_bytes(n, r, grad, delta) for n, r in zip(w.numels, rows))
    accum_bytes = 0
    if K > 1:
        accum_bytes = sum(q8_accum_bytes(n, r, True) + (K - 1) * q8_accum_bytes(n, r, False)
                          for n, r in zip(w.numels, rows))
    per_step = step_bytes + accum_bytes

    nsets = a.state_sets or (max(1, -(-(1 << 30) // per_step)) if per_step < (1 << 30) else 1)
    t_setup = time.perf_counter()
    sets = [q8_state(torch, L, synth, w, row_lens, a.layout, delta, a.stagger)
            for _ in range(nsets)]
    torch.cuda.synchronize()
    progress(f"{a.workload}: {nsets} int8 state set(s) of {P} params resident "
             f"({time.perf_counter() - t_setup:.1f} s)")
    stream = torch.cuda.current_stream()
    copy_gbps = copy_ceiling(torch, L, a.copy_gib)
    progress(f"copy ceiling {copy_gbps:.0f} GB/s")

    accum_plans = [[L.AccumQ8Plan([L.AccumQ8Segment(acc, g[j]) for acc, g in accs])
                    for j in range(K)] for _, accs, _ in sets] if K > 1 else []
    plans = [L.AdamwQ8Plan(segs) for segs, _, _ in sets]

    def accumulate(k):
        for j, plan in enumerate(accum_plans[k % nsets]):
            plan.run(overwrite=(j == 0))

    def step(k):
        plans[k % nsets].step(step=w.step, **hp)

    def whole(k):
        if K > 1:
            accumulate(k)
        step(k)

    for k in range(a.warmup):
        whole(k)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    step_ms = timed_events(torch, stream, whole, a.steps)
    wall = time.perf_counter() - t_wall0
    ms = sum(step_ms) / len(step_ms)
    if K > 1:
        adamw_ms_list = timed_events(torch, stream, step, a.steps)
        accum_ms_list = timed_events(torch, stream, accumulate, a.steps)
    else:
        adamw_ms_list, accum_ms_list = step_ms, []
    adamw_ms = sum(adamw_ms_list) / len(adamw_ms_list)
    adamw_gbps = step_bytes / (adamw_ms * 1e-3) / 1e9

    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for k in range(a.steps):
        whole(k)
    stop.record(stream)
    torch.cuda.synchronize()
    pipelined_ms = start.elapsed_time(stop) / a.steps
    progress(f"timed {a.steps} int8 steps: {ms:.4f} ms per step")
    gbps = per_step / (ms * 1e-3) / 1e9
    key = f"{a.workload}:q8:{'delta' if delta else 'nodelta'}"
    line = {
        "metric": METRIC,
        "value": P / (ms * 1e-3),
        "unit": "params/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32 arithmetic; int8 moments" + (" and accumulators" if K > 1 else ""),
        "data": "synthetic",
        "config": {
            "workload": a.workload, "description": w.description, "params": P,
            "segments": len(w.segments),
            "moments": "int8 codes + fp32 scale per row (row = last dimension)",
            "grad": ("int8 accumulator of 8 bf16 micro-batches" if K > 1 else "bf16"),
            "delta": delta, "step_t": w.step,
            "bytes_per_param": per_step / P, "bytes_per_step": per_step,
            "rotated_state_sets": nsets,
            "layout": a.layout,
            "kind_offset_bytes": a.stagger if a.layout == "flat" else None,
        },
        "hbm_gbps": gbps,
        "pct_hbm_peak": 100.0 * gbps / HBM_PEAK_GBPS,
        "copy_ceiling_gbps": copy_gbps,
        "pct_copy_ceiling": 100.0 * gbps / copy_gbps,
        "roofline": {"bound": "hbm", "achieved": adamw_gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": adamw_gbps / HBM_PEAK_GBPS,
                     "traffic": traffic_for(key, a.layout), "kernel": "adamw_q8_kernel",
                     "algorithmic_bytes_per_launch": step_bytes,
                     "avg_launch_ms": adamw_ms, "min_launch_ms": min(adamw_ms_list),
                     "median_launch_ms": statistics.median(adamw_ms_list),
                     "max_launch_ms": max(adamw_ms_list)},
        "pipelined": {"ms_per_step": pipelined_ms,
                      "hbm_gbps": per_step / (pipelined_ms * 1e-3) / 1e9,
                      "params_per_s": P / (pipelined_ms * 1e-3)},
        "host_wall_s_timed_region": wall,
    }
    if nsets > 1 or step_bytes < SMALL_STEP_BYTES:
        line["same_bytes_copy"] = same_bytes_copy(torch, L, stream, step_bytes, nsets, a.steps)
    if accum_ms_list:
        acc_ms = sum(accum_ms_list) / len(accum_ms_list)
        acc_gbps = accum_bytes / (acc_ms * 1e-3) / 1e9
        line["accumulation"] = {"kernel": "code_rows_kernel", "launches_per_step": K,
                                "ms_per_step": acc_ms, "hbm_gbps": acc_gbps,
                                "frac": acc_gbps / HBM_PEAK_GBPS,
                                "algorithmic_bytes_per_step": accum_bytes}
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = q8_cpu_baseline(sets[0][0][0], w, row_lens[0], hp, delta,
                                               a.cpu_seconds, step_bytes / P)
    return line


def q8_state(torch, L, synth, w, row_lens, layout, delta, stagger=4096):
    """One int8-moment state set on the GPU: (segments, [(int8 accumulator,
    [bf16 micro-batch gradients])], buffers).  The moments are the seeded fp32
    draws quantized by lema_quantize_rows; `layout` as for resident_state."""
    dev = "cuda"
    K = w.microbatches
    accs = []
    if layout == "flat":
        el, rw, segs = L.flat_q8_state(w.numels, row_lens, grad="q8" if K > 1 else "bf16",
                                       delta=delta, device=dev, stagger=stagger)
        mbs = [L.FlatState(w.numels, {"g": torch.bfloat16}, device=dev) for _ in range(K)] \
            if K > 1 else []
        for i in range(len(w.segments)):
            st = synth.make_segment_state(w, i, dev, with_orig=delta)
            s = segs[i]
            s.master.copy_(st["master"])
            L.quantize_rows([(st["m"], s.exp_avg), (st["v"], s.exp_avg_sq)])
            if delta:
                s.orig.copy_(st["orig"])
            if K > 1:
                gs = [fs.view("g", i) for fs in mbs]
                for dst, src in zip(gs, st["grads"]):
                    dst.copy_(src)
                accs.append((s.grad, gs))
            else:
                s.grad.copy_(st["grads"][0])
            del st
        return segs, accs, (el, rw, mbs)
    segs = []
    for i in range(len(w.segments)):
        st = synth.make_segment_state(w, i, dev, with_orig=delta)
        n, rl = w.numels[i], row_lens[i]
        m, v = L.Q8.empty(n, rl), L.Q8.empty(n, rl)
        L.quantize_rows([(st["m"], m), (st["v"], v)])
        if K > 1:
            g = L.Q8.empty(n, rl)
            accs.append((g, st["grads"]))
        else:
            g = st["grads"][0]
        segs.append(L.AdamwQ8Segment(st["master"], m, v, g,
                                     torch.empty(n, dtype=torch.bfloat16, device=dev),
                                     st.get("orig"),
                                     torch.empty(n, device=dev) if delta else None))
        del st["m"], st["v"]
    return segs, accs, None


def q8_cpu_baseline(seg, w, row_len, hp, delta, seconds, bytes_per_param):
    """The oracle's int8 step (dequantize, fp32 step, quantize) on the first
    tensor of the workload; GB/s with the GPU line's algorithmic bytes."""
    import oracle
    import torch

    def host(t):
        t = t.detach().cpu()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view("uint16").copy()
        return t.numpy().copy()

    master = host(seg.master)
    m = (host(seg.exp_avg.codes), host(seg.exp_avg.scale))
    v = (host(seg.exp_avg_sq.codes), host(seg.exp_avg_sq.scale))
    grad = host(seg.grad)
    orig = host(seg.orig) if delta else None
    n = master.shape[0]
    c = oracle.adamw_constants(hp["lr"], hp["beta1"], hp["beta2"], hp["eps"],
                               hp["weight_decay"], w.step)
    oracle.adamw_step_q8(master, m, v, grad, c, row_len, orig=orig)
    reps, el = timed_loop(lambda: oracle.adamw_step_q8(master, m, v, grad, c, row_len, orig=orig),
                          seconds)
    return {"value": n * reps / el, "unit": "params/s", "cores": oracle.num_threads(),
            "gbps": n * reps / el * bytes_per_param / 1e9,
            "kind": "oracle", "host": host_info(),
            "sample": f"{w.segments[0][0]} ({n} params, rows of {row_len}), {reps} oracle "
                      f"int8 steps in {el:.1f} s, delta {'on' if delta else 'off'}; C oracle, "
                      "OpenMP, numpy glue"}


# ------------------------------------------------------------ merge

def merge_bench(torch, L, synth, a):
    """merge_delta over the workload's tensors: read bf16 base + fp32 delta,
    write the bf16 merged weight (8 B per parameter)."""
    w = synth.WORKLOADS[a.workload]
    P = w.params
    segs = []
    fs = L.FlatState(w.numels, {"base": torch.bfloat16, "delta": torch.float32,
                                "merged": torch.bfloat16},
                     stagger=a.stagger) if a.layout == "flat" else None
    for i in range(len(w.segments)):
        n = w.numels[i]
        base = synth.bf16_normal(n, 0.02, synth.seed_of(w.wid, 0, i), "cuda")
        delta = synth.normal(n, 1e-4, synth.seed_of(w.wid, 5, i), "cuda")
        if fs is not None:
            fs.view("base", i).copy_(base)
            fs.view("delta", i).copy_(delta)
            base, delta = fs.view("base", i), fs.view("delta", i)
            segs.append(L.MergeSegment(base, delta, fs.view("merged", i)))
        else:
            segs.append(L.MergeSegment(base, delta, torch.empty_like(base)))
    per = 8 * P
    nsets = 1
    torch.cuda.synchronize()
    progress(f"{a.workload}: base and delta of {P} params resident")
    stream = torch.cuda.current_stream()
    copy_gbps = copy_ceiling(torch, L, a.copy_gib)
    progress(f"copy ceiling {copy_gbps:.0f} GB/s")
    for _ in range(a.warmup):
        L.merge_delta(segs)
    torch.cuda.synchronize()
    ms_list = timed_events(torch, stream, lambda k: L.merge_delta(segs), a.steps)
    ms = sum(ms_list) / len(ms_list)
    gbps = per / (ms * 1e-3) / 1e9
    return {
        "metric": "merge_delta params/sec + achieved HBM GB/s, 1 GPU",
        "value": P / (ms * 1e-3), "unit": "params/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": a.workload, "params": P, "segments": len(w.segments),
                   "bytes_per_param": 8, "rotated_state_sets": nsets, "layout": a.layout,
                   "kind_offset_bytes": a.stagger if a.layout == "flat" else None},
        "hbm_gbps": gbps, "pct_hbm_peak": 100 * gbps / HBM_PEAK_GBPS,
        "copy_ceiling_gbps": copy_gbps,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS,
                     "traffic": traffic_for(f"{a.workload}:merge", a.layout),
                     "kernel": "merge_tile_kernel",
                     "algorithmic_bytes_per_launch": per, "avg_launch_ms": ms},
    }


# ------------------------------------------------------------ checkpoint

def checkpoint_bench(torch, L, synth, a):
    """lema_checkpoint_save and lema_checkpoint_load of the workload's fp32
    master, m, v and delta (README "Features": checkpoints of the delta with
    the optimizer states) to a safetensors file in --checkpoint DIR: the
    rate of each whole call, device to file and back, through the page cache
    of the file system DIR is on."""
    w = synth.WORKLOADS[a.workload]
    fs, segs = L.flat_adamw_state(w.numels, delta=True)
    for i, s in enumerate(segs):
        st = synth.make_segment_state(w, i, "cuda")
        s.master.copy_(st["master"])
        s.exp_avg.copy_(st["m"])
        s.exp_avg_sq.copy_(st["v"])
        s.delta.copy_(st["master"])
        del st
    tensors = L.checkpoint_tensors(segs, delta=True)
    nbytes = sum(t.numel() * t.element_size() for t in tensors.values())
    path = os.path.join(a.checkpoint, f"bench_{w.name}.safetensors")
    torch.cuda.synchronize()
    save_s, load_s = [], []
    file_bytes = None
    try:
        for _ in range(max(1, a.steps)):
            t0 = time.perf_counter()
            L.save_checkpoint(path, tensors, step=w.step)
            save_s.append(time.perf_counter() - t0)
            file_bytes = os.path.getsize(path)
            t0 = time.perf_counter()
            L.load_checkpoint(path, tensors)
            load_s.append(time.perf_counter() - t0)
    finally:
        if os.path.exists(path):
            os.remove(path)
    sv, ld = sorted(save_s)[len(save_s) // 2], sorted(load_s)[len(load_s) // 2]
    return {
        "metric": "checkpoint save GB/s (load GB/s beside it), 1 GPU",
        "value": nbytes / sv / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": len(save_s),
        "warmup": 0, "ms_per_step": 1e3 * sv, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": a.workload, "params": w.params, "segments": len(w.segments),
                   "tensors": len(tensors), "file_bytes": file_bytes, "data_bytes": nbytes,
                   "contents": "fp32 master, m, v and delta of every tensor"},
        "save_s": save_s, "load_s": load_s, "load_gbps": nbytes / ld / 1e9,
    }


# ------------------------------------------------------------ streamed

def slot_stream_bench(torch, L, synth, a):
    """The whole 7B shape in host memory, streamed per layer: fp32 master, m
    and v, or with --q8 int8 moments with row scales, kept as codes in host
    memory (README "Quantization")."""
    w = synth.WORKLOADS["llama7b_full"]
    hp = synth.HPARAMS
    q8 = a.q8
    row_len = lambda i: w.segments[i][1][-1]
    rows = lambda i: -(-w.numels[i] // row_len(i))
    # the 34 loads: embedding, 32 decoder layers, final norm + LM head
    loads = [[0]] + [list(range(1 + 9 * l, 10 + 9 * l)) for l in range(32)] + [[289, 290]]
    requested = len(loads)
    if a.layers:
        loads = loads[:a.layers]
    align = lambda x: (x + 255) // 256 * 256
    if q8:
        slot_bytes = max(sum(align(4 * w.numels[i]) + 2 * (align(w.numels[i]) + align(4 * rows(i)))
                             + align(2 * w.numels[i]) * 2 for i in ld) for ld in loads)
    else:
        slot_bytes = max(sum(align(4 * w.numels[i]) * 3 + align(2 * w.numels[i]) * 2 for i in ld)
                         for ld in loads)
    host_bpp = 10 if q8 else 16

    # device side first: the pool's slots, then the standalone pinned copy
    # ceilings (half a slot each way); host staging comes last because the
    # GPU-mappable page-locked memory of a host is bounded
    pool = L.SlotPool(slot_bytes, nslots=a.slots, duplex=a.duplex)
    stream = torch.cuda.current_stream()
    hbuf = L.pinned_empty(slot_bytes // 2, torch.uint8)
    dbuf = torch.empty(slot_bytes // 2, dtype=torch.uint8, device="cuda")
    h2d = timed_events(torch, stream, lambda k: dbuf.copy_(hbuf, non_blocking=True), 3)
    d2h = timed_events(torch, stream, lambda k: hbuf.copy_(dbuf, non_blocking=True), 3)
    h2d_gbps = hbuf.numel() / (min(h2d) * 1e-3) / 1e9
    d2h_gbps = hbuf.numel() / (min(d2h) * 1e-3) / 1e9
    del hbuf, dbuf

    t0 = time.perf_counter()
    layers, staged_bytes = [], 0
    host_gib = a.host_gib or (120.0 if a.staged else 56.0)
    budget = host_gib * (1 << 30)
    alloc = (lambda n, dt: torch.empty(n, dtype=dt)) if a.staged else L.pinned_empty
    for li, ld in enumerate(loads):
        need = host_bpp * sum(w.numels[i] for i in ld)
        if staged_bytes + need > budget:
            print(f"bench.py: host budget {host_gib} GiB reached after {len(layers)} loads",
                  file=sys.stderr, flush=True)
            break
        segs = []
        try:
            for i in ld:
                st = synth.make_segment_state(w, i, "cuda")
                n = w.numels[i]
                if q8:
                    dm, dv = L.Q8.empty(n, row_len(i)), L.Q8.empty(n, row_len(i))
                    L.quantize_rows([(st["m"], dm), (st["v"], dv)])
                    tensors = (("master", st["master"]), ("mc", dm.codes), ("ms", dm.scale),
                               ("vc", dv.codes), ("vs", dv.scale), ("g", st["grads"][0]))
                else:
                    tensors = (("master", st["master"]), ("m", st["m"]), ("v", st["v"]),
                               ("g", st["grads"][0]))
                host = {}
                for k, t in tensors:
                    host[k] = alloc(t.numel(), t.dtype)
                    host[k].copy_(t)
                if q8:
                    segs.append(L.AdamwQ8Segment(
                        host["master"], L.Q8(host["mc"], host["ms"], row_len(i)),
                        L.Q8(host["vc"], host["vs"], row_len(i)), host["g"],
                        alloc(n, torch.bfloat16)))
                else:
                    segs.append(L.AdamwSegment(host["master"], host["m"], host["v"], host["g"],
                                               alloc(n, torch.bfloat16)))
                del st
        except (L.LemaError, RuntimeError) as e:
            del segs
            print(f"bench.py: page-locked allocation failed at load {li + 1} ({e}); "
                  f"streaming {len(layers)} of {requested} loads", file=sys.stderr, flush=True)
            break
        layers.append(segs)
        staged_bytes += need
        print(f"bench.py: staged load {li + 1}/{len(loads)} in host memory "
              f"({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)
    loads = loads[:len(layers)]
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t0
    P = sum(w.numels[i] for ld in loads for i in ld)

    R = sum(rows(i) for ld in loads for i in ld)

    steps = max(1, min(a.steps, 3))
    stats = []
    kw = dict(staged=a.staged, host_threads=a.host_threads)
    run = pool.stream_q8 if q8 else pool.stream
    run(layers, step=w.step, **kw, **hp)                     # warm-up step
    print("bench.py: warm-up streamed step done", file=sys.stderr, flush=True)
    for k in range(steps):
        stats.append(run(layers, step=w.step + 1 + k, **kw, **hp))
        print(f"bench.py: streamed step {k + 1}/{steps}: {stats[-1]['call_ms']:.0f} ms",
              file=sys.stderr, flush=True)
    pool.close()
    # the whole call on the host clock: for the staged path this includes the
    # first host copy in and the last host copy out
    wall = sum(s["call_ms"] for s in stats) / steps
    s0 = stats[-1]
    full_params = w.params
    line = {
        "metric": METRIC,
        "value": P / (wall * 1e-3),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": 1,
        "ms_per_step": wall,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 arithmetic; int8 moments" if q8 else "f32",
        "data": "synthetic",
        "config": {"workload": "llama7b_full_streamed", "loads": len(loads),
                   "loads_requested": requested, "params": P, "slots": a.slots,
                   "slot_bytes": slot_bytes, "grad": "bf16", "delta": False,
                   "copy_streams": 2 if a.duplex else 1, "step_t": w.step,
                   "host_memory": "pageable, staged" if a.staged else "page-locked",
                   "moments": "int8 codes + fp32 scale per row" if q8 else "fp32",
                   "host_state_bytes": host_bpp * P + (8 * R if q8 else 0),
                   "pcie_bytes_per_param_each_way": (8 + 8 * R / P) if q8 else 14,
                   "setup_s": setup_s},
        "stream": {"h2d_gbps": s0["h2d_bytes"] / (s0["h2d_ms"] * 1e-3) / 1e9,
                   "d2h_gbps": s0["d2h_bytes"] / (s0["d2h_ms"] * 1e-3) / 1e9,
                   "standalone_h2d_gbps": h2d_gbps, "standalone_d2h_gbps": d2h_gbps,
                   "kernel_ms": s0["kernel_ms"], "copy_busy_ms": s0["copy_busy_ms"],
                   "wall_ms": s0["wall_ms"], "call_ms": s0["call_ms"],
                   "host_in_ms": s0["host_in_ms"], "host_out_ms": s0["host_out_ms"],
                   "last_kernel_ms": s0["last_kernel_ms"],
                   "exposed_ms": s0["wall_ms"] - s0["copy_busy_ms"],
                   "kernel_hbm_gbps": ((16 * P + 16 * R) if q8 else 28 * P)
                   / (s0["kernel_ms"] * 1e-3) / 1e9,
                   "ms_per_param_billion": wall / (P / 1e9),
                   "projected_full_7b_ms": wall * full_params / P},
    }
    st = line["stream"]
    # "fully hidden": only the pipeline's tail is exposed, and the copies
    # run at (nearly) their standalone rate while overlapped
    st["hidden"] = {
        "exposed_over_last_kernel": st["exposed_ms"] / st["last_kernel_ms"]
        if st["last_kernel_ms"] > 0 else None,
        "h2d_over_standalone": st["h2d_gbps"] / h2d_gbps if h2d_gbps else None,
        "d2h_over_standalone": st["d2h_gbps"] / d2h_gbps if d2h_gbps else None,
    }
    return line


if __name__ == "__main__":
    main()
