"""Benchmark: evaluate one elementwise tensor Command per step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]
                    [--no-cpu-baseline]

A step is one launch of the whole Command (load, E_ operations, store) over
the workload's synthetic tensors, which are resident in HBM before timing
starts.  The headline is the int32 fused DAG z = (x + y) * w - s on 2^24
elements.  Prints one JSON line with effective HBM GB/s (algorithmic bytes read
+ written per second), the roofline of the kernel, and the CPU oracle's rate on
the same workload as a baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0        # MI355X HBM3E peak, 8 TB/s
METRIC = "effective HBM GB/s (bytes read+written / time) and % of peak, per Command"
DTYPE_OF = {"add_f32": "f32", "int_fused": "i32", "axpby_f32": "f32", "mixed_two_out": "f16/f32",
            "transposed_2d": "f32"}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "elementwise_tensor_commands_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def setup(wl, n=None):
    import numpy as np
    import torch

    import elementwise_tensor_commands_amd as ecmd
    import workloads as W
    spec = W.WORKLOADS[wl]["spec"]
    vals, extra = W.make_inputs(wl, n)
    dev = torch.device("cuda:0")
    gv = [torch.from_numpy(np.ascontiguousarray(v)).to(dev) if isinstance(v, np.ndarray) else v for v in vals]
    side = W.WORKLOADS[wl]["n"] if n is None else n
    if wl == "transposed_2d":
        gv[0] = torch.from_numpy(extra["X_storage"]).to(dev)[:, :side]
        gv[1] = torch.from_numpy(extra["Y"]).to(dev).t()
    shape = (side, side) if wl == "transposed_2d" else (side,)
    td = {"f16": torch.float16, "f32": torch.float32, "i32": torch.int32}
    out_dt = []
    dts = {}
    for name, st in spec:
        if st[0] in ("load", "scalar"):
            dts[name] = st[1]
        elif st[0] == "cvt":
            dts[name] = st[2]
        elif st[0] in ("add", "sub", "mul", "neg"):
            dts[name] = dts[st[1]]
        elif st[0] == "store":
            out_dt.append(dts[st[1]])
    outs = [torch.empty(shape, dtype=td[d], device=dev) for d in out_dt]
    cmd = ecmd.from_spec(spec)
    args = gv + outs
    plan = cmd.plan(*args)
    return cmd, args, plan, vals


def time_steps(cmd, args, steps, warmup, cold=False):
    """Launch the Command steps times back to back; HIP events around every
    launch on the launch stream.  Returns (total_ms, per-launch ms list)."""
    import torch
    stream = torch.cuda.current_stream()
    # Cold runs: read 1 GiB of unrelated data before each timed launch (outside
    # the events) so that none of the Command's data is left in the 256 MB
    # last-level cache; reading, not writing, leaves no dirty lines behind.
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0") if cold else None
    for _ in range(warmup):
        cmd.launch(*args, stream=stream)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        if cold:
            flush.sum()
        starts[i].record(stream)
        cmd.launch(*args, stream=stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    total = starts[0].elapsed_time(ends[-1])
    return total, per, wall_ms


def cpu_baseline(wl, budget_s=20.0):
    """The oracle as it stands, on the GPU machine's host cores, over a bounded
    prefix of the same workload's inputs."""
    import numpy as np

    import workloads as W
    from oracle import oracle
    spec = W.WORKLOADS[wl]["spec"]
    threads = max(1, min(16, os.cpu_count() or 1))
    full = W.WORKLOADS[wl]["n"]
    n = full if wl != "transposed_2d" else 2048
    if wl in ("axpby_f32", "mixed_two_out"):
        n = 1 << 24
    vals, extra = W.make_inputs(wl, n)
    cmd = oracle.from_spec(spec)
    res = {}
    for t in (1, threads):
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            cmd.run(*vals, nthreads=t)
            runs.append(time.perf_counter() - t0)
            if sum(runs) > budget_s:
                break
        res[t] = statistics.median(runs)
    elems = W.elements(wl, n)
    byts = W.algorithmic_bytes(wl, n)
    best_t = threads
    return {
        "value": round(byts / res[best_t] / 1e9, 3), "unit": "GB/s", "cores": best_t, "kind": "oracle",
        "sample": "%s, first %d elements (%s of the workload), same seeded inputs; median of up to 3 runs"
                  % (wl, elems, "all" if elems == W.elements(wl) else "part"),
        "gelem_per_s": round(elems / res[best_t] / 1e9, 4),
        "single_thread_gbps": round(byts / res[1] / 1e9, 3),
        "seconds": round(res[best_t], 4),
    }


def traffic_from_profiles(wl, kernel_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    the kernels have not changed since it was taken (else None)."""
    path = os.path.join(ROOT, "profiles", "counters_%s.json" % wl)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("kernel_source_hash") != kernel_hash:
        return None
    return c.get("hbm_bytes_per_launch")


def measure(wl, steps, warmup, cold_too=True):
    import workloads as W
    cmd, args, plan, _ = setup(wl)
    byts = W.algorithmic_bytes(wl)
    elems = W.elements(wl)
    total_ms, per, wall_ms = time_steps(cmd, args, steps, warmup)
    avg_ms = statistics.mean(per)
    r = {
        "kernel": plan["kernel"], "grid": plan["grid"], "block": plan["block"],
        "algorithmic_bytes": byts, "elements": elems,
        "whole_job_gbps": byts * steps / (total_ms * 1e-3) / 1e9,
        "kernel_avg_us": avg_ms * 1e3, "kernel_median_us": statistics.median(per) * 1e3,
        "kernel_p10_us": sorted(per)[len(per) // 10] * 1e3, "kernel_p90_us": sorted(per)[(9 * len(per)) // 10] * 1e3,
        "total_ms": total_ms, "wall_ms": wall_ms,
    }
    r["kernel_gbps"] = byts / (avg_ms * 1e-3) / 1e9
    if cold_too:
        _, per_c, _ = time_steps(cmd, args, min(steps, 20), 1, cold=True)
        r["cold_median_us"] = statistics.median(per_c) * 1e3
        r["cold_gbps"] = byts / (statistics.median(per_c) * 1e-3) / 1e9
    return r


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="int_fused")
    ap.add_argument("--all", action="store_true", help="also measure every other workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold (cache-flushed) launches, e.g. under a kernel-trace profiler")
    a = ap.parse_args()
    if a.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    khash = kernel_source_hash()
    log("workload %s: %s" % (a.workload, W.WORKLOADS[a.workload]["label"]))
    head = measure(a.workload, a.steps, a.warmup, cold_too=not a.no_cold)
    log("headline %s: %.1f GB/s whole-job, kernel avg %.2f us" % (head["kernel"], head["whole_job_gbps"], head["kernel_avg_us"]))
    traffic = traffic_from_profiles(a.workload, khash)
    line = {
        "metric": METRIC,
        "value": round(head["whole_job_gbps"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["total_ms"] / a.steps, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_OF[a.workload],
        "data": "synthetic (seeded NumPy PCG64, seed 1000 + config index), resident in HBM",
        "config": {"workload": W.WORKLOADS[a.workload]["label"], "elements": head["elements"],
                   "algorithmic_bytes_per_step": head["algorithmic_bytes"], "kernel": head["kernel"],
                   "grid": head["grid"], "block": head["block"]},
        "pct_of_peak": round(100 * head["whole_job_gbps"] / PEAK_GBPS, 2),
        "gelem_per_s": round(head["elements"] * a.steps / (head["total_ms"] * 1e-3) / 1e9, 3),
        "cold": ({"median_us": round(head["cold_median_us"], 3), "gbps": round(head["cold_gbps"], 2)}
                 if "cold_median_us" in head else None),
        "roofline": {
            "bound": "hbm", "achieved": round(head["kernel_gbps"], 2), "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": round(head["kernel_gbps"] / PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel_avg_us": round(head["kernel_avg_us"], 3),
        },
        "kernel_source_hash": khash,
    }
    if a.all:
        line["commands"] = {}
        for wl in W.WORKLOADS:
            if wl == a.workload:
                r = head
            else:
                log("measuring %s" % wl)
                r = measure(wl, min(a.steps, 100), a.warmup)
            line["commands"][wl] = {
                "kernel": r["kernel"], "gbps": round(r["kernel_gbps"], 1),
                "pct_of_peak": round(100 * r["kernel_gbps"] / PEAK_GBPS, 2),
                "median_us": round(r["kernel_median_us"], 3), "p10_us": round(r["kernel_p10_us"], 3),
                "p90_us": round(r["kernel_p90_us"], 3), "cold_median_us": round(r["cold_median_us"], 3),
                "cold_gbps": round(r["cold_gbps"], 1), "whole_job_gbps": round(r["whole_job_gbps"], 1),
                "gelem_per_s": round(r["elements"] / (r["kernel_median_us"] * 1e-6) / 1e9, 2),
            }
            log("%s: %s" % (wl, json.dumps(line["commands"][wl])))
    if not a.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(a.workload)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
