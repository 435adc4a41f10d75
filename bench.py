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
            "transposed_2d": "f32", "copy_f32": "f32", "classify_u32": "i32", "fill_f32": "f32",
            "batched_transpose": "f32", "bias_nchw": "f32", "axpby_f16": "f16", "axpby_bf16": "bf16",
            "bias_relu_f32": "f32", "transposed_relu": "f32", "odd_rows_f32": "f32", "narrow_rows_f32": "f32"}
# Measured besides the five configurations: the plain copy (the bandwidth and
# counter reference), the widened op set, the rank-3/4 views and native 16-bit
# arithmetic, and a Command with no ahead-of-time kernel run by the interpreter
# and by a kernel compiled at run time ("_jit").


def split_workload(name):
    """("bias_relu_f32", True) for "bias_relu_f32_jit": the workload measured
    with its kernel compiled at run time."""
    return (name[:-4], True) if name.endswith("_jit") else (name, False)
EXTRA = ["copy_f32", "classify_u32", "fill_f32", "batched_transpose", "bias_nchw", "axpby_f16", "axpby_bf16",
         "bias_relu_f32", "bias_relu_f32_jit", "transposed_relu", "transposed_relu_jit", "odd_rows_f32",
         "odd_rows_f32_jit", "narrow_rows_f32", "narrow_rows_f32_jit"]
PROFILES = os.path.join(ROOT, "profiles")


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


def setup(wl, n=None, jit=False):
    import numpy as np
    import torch

    import elementwise_tensor_commands_amd as ecmd
    import workloads as W
    spec = W.WORKLOADS[wl]["spec"]
    vals, extra = W.make_inputs(wl, n)
    dev = torch.device("cuda:0")
    gv = W.to_torch(vals, extra, dev)
    shape = W.shape_of(wl, n)
    td = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32, "i32": torch.int32}
    out_dt = []
    dts = {}
    for name, st in spec:
        if st[0] in ("load", "scalar"):
            dts[name] = st[1]
        elif st[0] == "cvt":
            dts[name] = st[2]
        elif st[0] in ("add", "sub", "mul", "neg", "abs", "min", "max"):
            dts[name] = dts[st[1]]
        elif st[0] == "select":
            dts[name] = dts[st[2]]
        elif st[0] in ("eq", "ne", "lt", "le", "gt", "ge", "ltu", "leu", "gtu", "geu"):
            dts[name] = "i32"
        elif st[0] == "store":
            out_dt.append(dts[st[1]])
    outs = [torch.empty(shape, dtype=td[d], device=dev) for d in out_dt]
    cmd = ecmd.from_spec(spec)
    if jit:
        cmd.jit()
    args = gv + outs
    plan = cmd.plan(*args)
    return cmd, args, plan, vals


def time_steps(cmd, args, steps, warmup):
    """Launch the Command steps times back to back on the current stream, with
    HIP events at both ends of the timed region.  Returns (total_ms, wall_ms)."""
    import torch
    stream = torch.cuda.current_stream()
    bound = cmd.bind(*args, stream=stream)
    for _ in range(warmup):
        bound.launch()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        bound.launch()
    end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    return start.elapsed_time(end), wall_ms


def measure_graph(wl, launches=100, replays=20):
    """Back-to-back launches captured in one HIP graph (torch.cuda.CUDAGraph)
    and replayed: the rate once the host's per-launch cost is gone (the
    launch-bound 65,536-element configuration).  Timed by HIP events around
    the replays."""
    import torch
    import workloads as W
    cmd, args, plan, _ = setup(wl)
    bound = cmd.bind(*args)
    bound.launch()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = cmd.bind(*args)              # the capture stream
        for _ in range(launches):
            cap.launch()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    per_us = start.elapsed_time(end) * 1e3 / (launches * replays)
    byts = W.algorithmic_bytes(wl)
    return {"kernel": plan["kernel"], "launches_per_graph": launches, "replays": replays,
            "per_launch_us": round(per_us, 3), "gbps": round(byts / (per_us * 1e-6) / 1e9, 1)}


def time_each(cmd, args, reps, cold=False):
    """Per-launch HIP event pairs, optionally reading 1 GiB of unrelated data
    before each launch (outside the events) so that none of the Command's data
    is left in the 256 MB last-level cache; reading leaves no dirty lines."""
    import torch
    stream = torch.cuda.current_stream()
    bound = cmd.bind(*args, stream=stream)
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0") if cold else None
    bound.launch()
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        if cold:
            flush.sum()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        bound.launch()
        e.record(stream)
        e.synchronize()
        per.append(s.elapsed_time(e))
    return per


def cpu_baseline(wl, budget_s=20.0):
    """The oracle as it stands, on the host's cores, over a bounded
    prefix of the same workload's inputs."""
    import numpy as np

    import workloads as W
    from oracle import oracle
    spec = W.WORKLOADS[wl]["spec"]
    threads = max(1, min(16, os.cpu_count() or 1))
    full = W.WORKLOADS[wl].get("n")
    n = full if wl != "transposed_2d" else 2048
    if wl in ("axpby_f32", "mixed_two_out", "axpby_f16", "axpby_bf16"):
        n = 1 << 24
    shape = {"batched_transpose": (4, 2048, 2048), "bias_nchw": (2, 256, 128, 256), "odd_rows_f32": (2048, 8191),
             "narrow_rows_f32": (1 << 21, 6)}.get(wl)
    vals, extra = W.make_inputs(wl, n, shape=shape)
    cmd = oracle.from_spec(spec)
    # Repeat each thread count for about half the time budget (at least 3
    # runs, at most 200) and take the median run.
    res, counts = {}, {}
    for t in (1, threads):
        runs = []
        while len(runs) < 3 or (sum(runs) < budget_s / 2 and len(runs) < 200):
            t0 = time.perf_counter()
            cmd.run(*vals, nthreads=t)
            runs.append(time.perf_counter() - t0)
        res[t] = statistics.median(runs)
        counts[t] = len(runs)
    elems = W.elements(wl, n, shape)
    byts = W.algorithmic_bytes(wl, n, shape)
    best_t = threads
    return {
        "value": round(byts / res[best_t] / 1e9, 3), "unit": "GB/s", "cores": best_t, "kind": "oracle",
        "sample": "%s, first %d elements (%s of the workload), same seeded inputs; median of %d runs "
                  "(%d on one thread)" % (wl, elems, "all" if elems == W.elements(wl) else "part",
                                          counts[best_t], counts[1]),
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


def measure(wl, steps, warmup, cold_too=True, jit=False):
    """Timed region: steps back-to-back launches between two HIP events on the
    launch stream.  The kernel's average duration is that time / steps (the
    host queues launches faster than they run, so the GPU never waits).
    Separately, per-launch event pairs give median / p10 / p90 and, with a
    cache flush before each launch, the cold rate."""
    import workloads as W
    cmd, args, plan, _ = setup(wl, jit=jit)
    if jit:
        log("%s: run-time compiled kernel from %s" % (wl, {0: "memory", 1: "disk", 2: "compiler"}.get(cmd.prepare(*args))))
    byts = W.algorithmic_bytes(wl)
    elems = W.elements(wl)
    total_ms, wall_ms = time_steps(cmd, args, steps, warmup)
    avg_ms = total_ms / steps
    per = sorted(time_each(cmd, args, min(steps, 50)))
    r = {
        "kernel": plan["kernel"], "grid": plan["grid"], "block": plan["block"],
        "algorithmic_bytes": byts, "elements": elems,
        "whole_job_gbps": byts * steps / (total_ms * 1e-3) / 1e9,
        "kernel_avg_us": avg_ms * 1e3, "kernel_median_us": statistics.median(per) * 1e3,
        "kernel_p10_us": per[len(per) // 10] * 1e3, "kernel_p90_us": per[(9 * len(per)) // 10] * 1e3,
        "total_ms": total_ms, "wall_ms": wall_ms,
    }
    r["kernel_gbps"] = byts / (avg_ms * 1e-3) / 1e9
    if cold_too:
        per_c = time_each(cmd, args, 20, cold=True)
        r["cold_median_us"] = statistics.median(per_c) * 1e3
        r["cold_gbps"] = byts / (statistics.median(per_c) * 1e-3) / 1e9
    return r


def read_write_bytes(wl):
    """Algorithmic bytes read and written by one launch of the workload."""
    import workloads as W
    return W.algorithmic_read_write(split_workload(wl)[0])


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    return rows


def summarize_counters(root, command):
    """Turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs (root/fetch_<wl>,
    root/write_<wl>, one per workload plus copy_f32) into profiles/.  Each
    counter is scaled by what it reads for the plain copy of known size (1 GiB
    read + 1 GiB written)."""
    import workloads as W

    def per_dispatch(kind, wl):
        rows = [r for r in _csv_rows(os.path.join(root, "%s_%s" % (kind, wl)), "counter_collection.csv")
                if "ecmd::k_" in r["Kernel_Name"]]
        assert rows, "no ecmd kernel rows for %s %s" % (kind, wl)
        names = sorted({r["Kernel_Name"] for r in rows})
        assert len(names) == 1, names
        vals = [float(r["Counter_Value"]) for r in rows]
        return names[0], statistics.mean(vals), len(vals)

    khash = kernel_source_hash()
    cr, cw = read_write_bytes("copy_f32")
    _, f_copy, _ = per_dispatch("fetch", "copy_f32")
    _, w_copy, _ = per_dispatch("write", "copy_f32")
    cal_f, cal_w = cr / (f_copy * 1024), cw / (w_copy * 1024)
    lines = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Command (one counter per run, one run per workload):", "", "    " + command, "",
             "Calibration: the plain copy `copy_f32` (2^28 fp32: 1 GiB read, 1 GiB written) reads "
             "FETCH_SIZE = %.0f KiB and WRITE_SIZE = %.0f KiB per dispatch, so FETCH_SIZE is scaled by "
             "%.4f and WRITE_SIZE by %.4f." % (f_copy, w_copy, cal_f, cal_w), "",
             "kernel source hash: %s" % khash, "",
             "| workload | kernel | dispatches | FETCH KiB | WRITE KiB | read B (scaled) | algorithmic read B | "
             "ratio | written B (scaled) | algorithmic write B | ratio |",
             "|---|---|---|---|---|---|---|---|---|---|---|"]
    for wl in W.CONFIGS + EXTRA:
        if not os.path.isdir(os.path.join(root, "fetch_" + wl)):
            continue
        name, f, nf = per_dispatch("fetch", wl)
        _, w, _ = per_dispatch("write", wl)
        rd, wr = read_write_bytes(wl)
        fb, wb = f * 1024 * cal_f, w * 1024 * cal_w
        rec = {"workload": wl, "kernel": name, "dispatches": nf, "fetch_kib_per_dispatch": f,
               "write_kib_per_dispatch": w, "fetch_scale": cal_f, "write_scale": cal_w,
               "read_bytes_per_launch": fb, "write_bytes_per_launch": wb,
               "hbm_bytes_per_launch": fb + wb, "algorithmic_read_bytes": rd,
               "algorithmic_write_bytes": wr, "read_ratio": fb / rd if rd else None,
               "write_ratio": wb / wr,
               "kernel_source_hash": khash, "command": command}
        with open(os.path.join(PROFILES, "counters_%s.json" % wl), "w") as out:
            json.dump(rec, out, indent=1)
        lines.append("| %s | `%s` | %d | %.0f | %.0f | %.0f | %d | %s | %.0f | %d | %.4f |" % (
            wl, name[:70], nf, f, w, fb, rd, "%.4f" % (fb / rd) if rd else "-", wb, wr, wb / wr))
    with open(os.path.join(PROFILES, "counters_summary.md"), "w") as out:
        out.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_trace(directory, wl, bench_json, command):
    """profiles/kernel_trace_<wl>.txt from a rocprofv3 --kernel-trace --stats
    run of bench.py and the JSON line that same run printed."""
    rows = [r for r in _csv_rows(directory, "kernel_stats.csv") if "ecmd::k_" in r["Name"]]
    assert len(rows) == 1, [r["Name"] for r in rows]
    r = rows[0]
    with open(bench_json) as f:
        line = json.loads([l for l in f.read().splitlines() if l.startswith("{")][-1])
    prof_us = float(r["AverageNs"]) / 1e3
    bench_us = line["roofline"]["kernel_avg_us"]
    text = ["kernel trace: %s" % wl, "", "command:", "    " + command, "",
            "rocprofv3 kernel stats (ecmd kernel row):"]
    text += ["    %s: %s" % (k, v) for k, v in r.items()]
    text += ["", "bench.py HIP-event average over the same run's timed launches: %.3f us" % bench_us,
             "rocprofv3 average over all dispatches (warm-up + timed): %.3f us" % prof_us,
             "difference: %.2f %%" % (100 * (prof_us - bench_us) / bench_us),
             "bench value: %s %s; roofline achieved %s GB/s = %.1f %% of %s GB/s" % (
                 line["value"], line["unit"], line["roofline"]["achieved"], 100 * line["roofline"]["frac"],
                 line["roofline"]["peak"]),
             "kernel source hash: %s" % kernel_source_hash()]
    with open(os.path.join(PROFILES, "kernel_trace_%s.txt" % wl), "w") as out:
        out.write("\n".join(text) + "\n")
    print("\n".join(text))


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
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write profiles/ counter summaries from rocprofv3 --pmc output in DIR and exit")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "BENCH_JSON"),
                    help="write profiles/kernel_trace_<workload>.txt from a kernel-trace run and exit")
    ap.add_argument("--command", default="", help="the profiling command, recorded in the summary")
    a = ap.parse_args()
    if a.summarize_counters:
        summarize_counters(a.summarize_counters, a.command)
        return
    if a.summarize_trace:
        summarize_trace(a.summarize_trace[0], a.workload, a.summarize_trace[1], a.command)
        return
    if a.gpus != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    khash = kernel_source_hash()
    base, jit = split_workload(a.workload)
    label = W.WORKLOADS[base]["label"] + (" (kernel compiled at run time)" if jit else "")
    log("workload %s: %s" % (a.workload, label))
    head = measure(base, a.steps, a.warmup, cold_too=not a.no_cold, jit=jit)
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
        "dtype": DTYPE_OF[base],
        "data": "synthetic (seeded NumPy PCG64, seed 1000 + config index), resident in HBM",
        "config": {"workload": label, "elements": head["elements"],
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
        for wl in W.CONFIGS + EXTRA:
            if wl == a.workload:
                r = head
            else:
                log("measuring %s" % wl)
                wl_base, wl_jit = split_workload(wl)
                r = measure(wl_base, min(a.steps, 100), a.warmup, jit=wl_jit)
            line["commands"][wl] = {
                "kernel": r["kernel"], "gbps": round(r["kernel_gbps"], 1),
                "pct_of_peak": round(100 * r["kernel_gbps"] / PEAK_GBPS, 2),
                "avg_us": round(r["kernel_avg_us"], 3),
                "median_us": round(r["kernel_median_us"], 3), "p10_us": round(r["kernel_p10_us"], 3),
                "p90_us": round(r["kernel_p90_us"], 3), "cold_median_us": round(r["cold_median_us"], 3),
                "cold_gbps": round(r["cold_gbps"], 1), "whole_job_gbps": round(r["whole_job_gbps"], 1),
                "gelem_per_s": round(r["elements"] / (r["kernel_avg_us"] * 1e-6) / 1e9, 2),
            }
            log("%s: %s" % (wl, json.dumps(line["commands"][wl])))
        line["commands"]["add_f32_graph"] = measure_graph("add_f32")
        log("add_f32_graph: %s" % json.dumps(line["commands"]["add_f32_graph"]))
    if not a.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(base)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
