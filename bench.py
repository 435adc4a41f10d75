"""Benchmark: evaluate elementwise tensor Commands on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--all]
                    [--no-cpu-baseline] [--no-commands]

A step is one launch of the whole Command (load, E_ operations, store) over
the workload's synthetic tensors, resident in HBM before timing starts.  The
headline workload is the largest configuration on the linear path,
out = 1.5 x - 0.25 y in binary32 over 2^28 elements (3 GiB moved per step),
timed cold: before every step a 1 GiB read evicts the Command's data from the
256 MB last-level cache, so each step reads its operands from HBM.  Each
step's kernel time comes from HIP events that the launch's dispatch records at
its start and end (cmd_launch_timed: what a kernel-trace profiler measures);
`value` is algorithmic bytes x K / the K steps' summed kernel time.  After the
timed region the same cold steps are timed again by ordinary events recorded on
the stream around each launch (the command processor's dispatch latency
included, a few microseconds per launch) and reported beside it.  Then the
same K steps run once more over copies of the operands placed 4 KiB apart
modulo 32 KiB (ecmd.empty_staggered) instead of where torch's allocator puts
them; that rate goes to "placement", beside the value, not into it.

The same JSON line carries, under "commands", the five configurations (and a
plain copy, the reference for "% of copy", plus three programs with no
ahead-of-time kernel: compiled at run time), each with warm (back-to-back) and
cold per-launch median / p10 / p90, % of peak and of copy, the host's cost per
launch and a full-size parity check against the oracle; the roofline of the
headline kernel; the oracle's own rate on the host's cores; and a snapshot of
the machine.  Workload names take a suffix: "@noaot" runs a program on the
ahead-of-time list through a kernel compiled at run time instead,
"@interp" through the interpreter.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_GBPS = 8000.0        # MI355X HBM3E peak, 8 TB/s
METRIC = "effective HBM GB/s (bytes read+written / time) and % of peak, per Command"
HEADLINE = "axpby_f32"
DTYPE_OF = {"add_f32": "f32", "int_fused": "i32", "axpby_f32": "f32", "mixed_two_out": "f16/f32",
            "transposed_2d": "f32", "copy_f32": "f32", "classify_u32": "i32", "fill_f32": "f32",
            "batched_transpose": "f32", "bias_nchw": "f32", "axpby_f16": "f16", "axpby_bf16": "bf16",
            "bias_relu_f32": "f32", "transposed_relu": "f32", "odd_rows_f32": "f32", "narrow_rows_f32": "f32",
            "bias_nchw_f16": "f16", "transposed_2d_f16": "f16"}
CONFIGS = ["add_f32", "int_fused", "axpby_f32", "mixed_two_out", "transposed_2d"]
# Measured in every run besides the five configurations: the plain copy (the
# reference for "% of copy") and three programs with no ahead-of-time kernel.
LINE_EXTRA = ["copy_f32", "bias_relu_f32", "transposed_relu", "mixed_two_out@noaot"]
# --all adds the widened op set, rank-3/4 views, native 16-bit arithmetic, the
# gather path and the interpreters.
ALL_EXTRA = ["classify_u32", "fill_f32", "batched_transpose", "transposed_2d_f16", "bias_nchw", "bias_nchw_f16",
             "axpby_f16", "axpby_bf16",
             "odd_rows_f32", "narrow_rows_f32", "int_fused_wide", "bias_relu_f32@interp",
             "transposed_relu@interp", "mixed_two_out@interp", "odd_rows_f32@interp", "narrow_rows_f32@interp"]
PROFILES = os.path.join(ROOT, "profiles")
REPS = 50                 # per-launch event pairs, warm and cold
REPS_SMALL = 200          # the same for the 65,536-element configuration
BACK_TO_BACK_SMALL = 1000  # its back-to-back launches


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


def split_workload(name):
    """("bias_relu_f32", "interp") for "bias_relu_f32@interp"; "int_fused_wide"
    is the int32 fused Command (int_fused) on full-range int32 inputs."""
    base, _, variant = name.partition("@")
    return base, variant


def _out_dtypes(spec):
    dts, outs = {}, []
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
            outs.append(dts[st[1]])
    return outs


def make_host_inputs(name):
    import numpy as np

    import workloads as W
    base, _ = split_workload(name)
    if base == "int_fused_wide":
        # the int32 fused Command on full-range int32 inputs (wraparound in
        # nearly every element); int_fused's seed plus 100
        rng = np.random.default_rng(W.seed_of("int_fused") + 100)
        vals = [rng.integers(-2**31, 2**31, 1 << 24, dtype=np.int64).astype(np.int32) for _ in range(3)]
        vals.append(W.SCALARS["int_fused"]["s"])
        return "int_fused", vals, {"storage": [vals[0], vals[1], vals[2], None]}
    vals, extra = W.make_inputs(base)
    return base, vals, extra


class Setup:
    """One workload on the GPU: inputs, outputs, the Command and its plan."""

    def __init__(self, name):
        import torch

        import elementwise_tensor_commands_amd as ecmd
        import workloads as W
        self.name = name
        wl, variant = split_workload(name)
        self.wl, self.variant = wl, variant
        spec_wl, vals, extra = make_host_inputs(name)
        self.spec_wl = spec_wl
        self.spec = W.WORKLOADS[spec_wl]["spec"]
        self.vals = vals
        dev = torch.device("cuda:0")
        gv = W.to_torch(vals, extra, dev)
        shape = W.shape_of(spec_wl)
        td = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32, "i32": torch.int32}
        self.outs = [torch.empty(shape, dtype=td[d], device=dev) for d in _out_dtypes(self.spec)]
        cmd = ecmd.from_spec(self.spec)
        if variant == "noaot":
            cmd.aot(False).jit(ecmd.JIT_SYNC)
        elif variant == "interp":
            cmd.aot(False).jit(ecmd.JIT_OFF)
        elif variant:
            raise ValueError("unknown variant %r" % variant)
        self.cmd = cmd
        self.args = gv + self.outs
        # Kernels compiled at run time are built (or read from disk) here, off
        # the clock, as a deployment would with cmd_prepare.
        self.compiled_from = {-1: None, 0: "memory", 1: "disk", 2: "compiler"}[cmd.prepare(*self.args)]
        self.plan = cmd.plan(*self.args)
        self.bytes = W.algorithmic_bytes(spec_wl)
        self.elements = W.elements(spec_wl)
        self.read_write = W.algorithmic_read_write(spec_wl)


def _pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, int(q * len(xs)))]


def _stats_us(ms_list):
    us = [m * 1e3 for m in ms_list]
    return {"median_us": round(statistics.median(us), 3), "p10_us": round(_pct(us, 0.1), 3),
            "p90_us": round(_pct(us, 0.9), 3)}


class Flusher:
    """Reads 1 GiB of unrelated data: afterwards none of a Command's data is
    left in the 256 MB last-level cache (the read leaves no dirty lines)."""

    def __init__(self):
        import torch
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")

    def __call__(self):
        self.buf.sum()


def time_back_to_back(bound, steps):
    """steps launches back to back between two HIP events on the launch
    stream: (total ms, host wall ms)."""
    import torch
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        bound.launch()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end), (time.perf_counter() - t0) * 1e3


def _events(stream, n=2):
    """n timing events, each recorded once (torch creates events lazily)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for ev in evs:
        ev.record(stream)
    return evs


def time_each(bound, reps, flush=None, dispatch=False):
    """Per-launch kernel durations: the launch's dispatches record a pair of
    HIP events at their start and end (cmd_launch_timed), as a kernel-trace
    profiler times a kernel.  With flush, the cache is flushed before each
    launch.  With dispatch, ordinary events recorded on the stream around an
    ordinary launch instead (the command processor's dispatch latency
    included).  Returns ms per launch."""
    import torch
    stream = torch.cuda.current_stream()
    s, e = _events(stream, 2)
    per = []
    torch.cuda.synchronize()
    for _ in range(reps):
        if flush is not None:
            flush()
        if dispatch:
            s.record(stream)
            bound.launch()
            e.record(stream)
        else:
            bound.launch_timed(s, e)
        e.synchronize()
        per.append(s.elapsed_time(e))
    return per


def settle(bound, seconds=0.3, min_launches=20):
    """Launch back to back for about `seconds` (at least min_launches) so the
    GPU has left its idle power states before anything is timed: after the
    seconds of host work that building a workload's inputs takes, the first
    launches of a run measured up to 1% slower than the same kernel later in
    the process."""
    import torch
    t0 = time.perf_counter()
    k = 0
    while k < min_launches or time.perf_counter() - t0 < seconds:
        for _ in range(10):
            bound.launch()
        k += 10
        torch.cuda.synchronize()
    return k


def host_launch_us(bound, n=20):
    """Host wall time per launch call (argument marshalling done once,
    launches enqueued without waiting), averaged over n calls."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n):
        bound.launch()
    t = (time.perf_counter() - t0) / n
    torch.cuda.synchronize()
    return t * 1e6


def ctypes_call_us(n=20000):
    """Cost of one ctypes call into the library (cmd_version), to separate
    Python's share of the host launch cost from the library's and HIP's."""
    import elementwise_tensor_commands_amd as ecmd
    t0 = time.perf_counter()
    for _ in range(n):
        ecmd.cmd_version()
    return (time.perf_counter() - t0) / n * 1e6


def oracle_threads():
    """Threads for the oracle: the CPUs this process may run on, within the
    cgroup's CPU quota and OMP_NUM_THREADS (the share of the host the job is
    given), at least 1."""
    t = len(os.sched_getaffinity(0))
    q = cgroup_cpus()
    if q:
        t = min(t, max(1, int(q)))
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        t = min(t, int(omp))
    return max(1, t)


def cgroup_cpus():
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota, period = f.read().split()
        return None if quota == "max" else float(quota) / float(period)
    except (OSError, ValueError):
        return None


def host_snapshot():
    """CPU model, sockets, cores and SMT from /proc/cpuinfo (read only)."""
    model, phys, cores, siblings = "", set(), None, None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and not model:
                    model = v
                elif k == "physical id":
                    phys.add(v)
                elif k == "cpu cores" and cores is None:
                    cores = int(v)
                elif k == "siblings" and siblings is None:
                    siblings = int(v)
    except OSError:
        pass
    return {"cpu_model": model or platform.processor(), "sockets": len(phys) or None,
            "cores_per_socket": cores, "threads_per_socket": siblings,
            "smt": (siblings // cores) if cores and siblings else None,
            "nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "cgroup_cpu_quota": cgroup_cpus(), "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def env_snapshot():
    """Read-only snapshot of the machine the line was measured on."""
    import numpy as np
    import torch
    p = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    return {"gpu": p.name, "gfx": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "hbm_bytes": p.total_memory, "rocm": rocm, "torch_hip": torch.version.hip,
            "torch": torch.__version__, "numpy": np.__version__, "python": platform.python_version(),
            "host": host_snapshot()}


def ulp_report(got, ref):
    """Per-element ulp distance in the output's own type (+0 and -0 both 0,
    NaN against NaN 0): max and histogram {0, 1, 2, >2}."""
    import numpy as np
    width = got.itemsize * 8
    ut = {2: np.uint16, 4: np.uint32}[got.itemsize]
    gb = np.ascontiguousarray(got).view(ut).ravel().astype(np.int64)
    rb = np.ascontiguousarray(ref).view(ut).ravel().astype(np.int64)
    sign = 1 << (width - 1)

    def ordered(b):
        return np.where(b & sign, -(b & (sign - 1)), b)

    d = np.abs(ordered(gb) - ordered(rb))
    if got.dtype.kind == "f":
        ng, nr = np.isnan(got).ravel(), np.isnan(ref).ravel()
        d = np.where(ng & nr, 0, np.where(ng ^ nr, 1 << 40, d))
    return {"max_ulp": int(d.max()) if d.size else 0,
            "hist": {"0": int((d == 0).sum()), "1": int((d == 1).sum()), "2": int((d == 2).sum()),
                     ">2": int((d > 2).sum())}}


def parity(st, threads):
    """The GPU's outputs of the last launch against the oracle on the same
    host inputs, every element: mismatches (bitwise; NaN equals NaN), and for
    outputs of the mixed-precision Command the ulp report."""
    import numpy as np

    import torch
    from oracle import oracle
    # A Command without tensor inputs (the fill) takes its shape from the
    # outputs: the oracle writes into host arrays of the outputs' shape.
    outs = None
    if not any(isinstance(v, np.ndarray) for v in st.vals):
        npd = {torch.float32: np.float32, torch.float16: np.float16, torch.int32: np.int32, torch.bfloat16: np.uint16}
        outs = [np.empty(tuple(o.shape), dtype=npd[o.dtype]) for o in st.outs]
    t0 = time.perf_counter()
    ref = oracle.from_spec(st.spec).run(*st.vals, outputs=outs, nthreads=threads)
    oracle_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    res = {"compared": 0, "mismatches": 0, "oracle_threads": threads, "oracle_s": round(oracle_s, 3)}
    for k, (o, r) in enumerate(zip(st.outs, ref)):
        g = o.view(torch.int16).cpu().numpy().view(np.uint16) if o.dtype == torch.bfloat16 else o.cpu().numpy()
        ut = {2: np.uint16, 4: np.uint32}[r.itemsize]
        gb, rb = g.view(ut).ravel(), np.ascontiguousarray(r).view(ut).ravel()
        bad = gb != rb
        if r.dtype.kind == "f":
            bad &= ~(np.isnan(g).ravel() & np.isnan(r).ravel())
        res["compared"] += int(gb.size)
        res["mismatches"] += int(bad.sum())
        if st.spec_wl == "mixed_two_out":
            res["out%d_ulp" % k] = ulp_report(g, r)
    return res, ref, oracle_s


def measure(name, steps, warmup, flush, threads, check=True, reps=REPS):
    """Warm (back-to-back, and per-launch pairs) and cold (flushed before
    each launch) timings of one workload, its host launch cost and parity."""
    st = Setup(name)
    bound = st.cmd.bind(*st.args)
    small = st.bytes < (64 << 20)
    settled = settle(bound)
    for _ in range(warmup):
        bound.launch()
    b2b = BACK_TO_BACK_SMALL if small else steps
    total_ms, wall_ms = time_back_to_back(bound, b2b)
    reps = max(reps, REPS_SMALL) if small else reps
    each = time_each(bound, reps)
    cold = time_each(bound, reps, flush)
    host_us = host_launch_us(bound)
    avg_us = total_ms * 1e3 / b2b
    cold_med = statistics.median(cold) * 1e3
    r = {
        "kernel": st.plan["kernel"], "path": st.plan["path"], "grid": st.plan["grid"], "block": st.plan["block"],
        "elements": st.elements, "algorithmic_bytes": st.bytes,
        "warm": dict(avg_us=round(avg_us, 3), gbps=round(st.bytes / (avg_us * 1e-6) / 1e9, 1),
                     launches=b2b, **_stats_us(each)),
        "cold": dict(gbps=round(st.bytes / (cold_med * 1e-6) / 1e9, 1), launches=reps, **_stats_us(cold)),
        "gelem_per_s": round(st.elements / (cold_med * 1e-6) / 1e9, 2),
        "pct_of_peak": round(100 * st.bytes / (cold_med * 1e-6) / 1e9 / PEAK_GBPS, 2),
        # the slower of the cold rate and the back-to-back one: a kernel whose
        # stores stay in the caches leaves their write-back to the cache flush
        # of a cold launch, and pays it in back-to-back launches instead
        "sustained_gbps": round(min(st.bytes / (cold_med * 1e-6), st.bytes / (avg_us * 1e-6)) / 1e9, 1),
        "host_launch_us": round(host_us, 2),
        "launch_sequence": [settled + warmup, b2b, reps, reps, 20],
    }
    if st.compiled_from:
        r["compiled_from"] = st.compiled_from
    if small:
        r["warm"]["host_bound"] = True
    if check:
        r["parity"], _, _ = parity(st, threads)
    return r, st


def measure_graph(name, launches=100, replays=20):
    """Back-to-back launches captured in one HIP graph (torch.cuda.CUDAGraph)
    and replayed: the rate once the host's per-launch cost is gone (the
    launch-bound 65,536-element configuration).  Timed by HIP events around
    the replays."""
    import torch
    st = Setup(name)
    bound = st.cmd.bind(*st.args)
    bound.launch()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = st.cmd.bind(*st.args)              # the capture stream
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
    return {"kernel": st.plan["kernel"], "launches_per_graph": launches, "replays": replays,
            "per_launch_us": round(per_us, 3), "gbps": round(st.bytes / (per_us * 1e-6) / 1e9, 1),
            "launch_sequence": [1, launches * 3 + launches * replays]}


def torch_copy_gbps(flush, reps=REPS):
    """A plain device-to-device copy of 1 GiB (torch's copy_, not this
    library's code), cold: 2 GiB moved per copy."""
    import torch
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    stream = torch.cuda.current_stream()
    per = []
    for _ in range(reps):
        flush()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        dst.copy_(src)
        e.record(stream)
        e.synchronize()
        per.append(s.elapsed_time(e))
    med = statistics.median(per)
    return {"bytes": 2 << 30, "cold_median_us": round(med * 1e3, 3), "gbps": round((2 << 30) / (med * 1e-3) / 1e9, 1)}


def cpu_baseline(st, threads, gpu_gbps, budget_s=20.0):
    """The oracle as it stands, over the headline workload's own inputs (all
    of them), on `threads` threads and on one: median run of each."""
    from oracle import oracle
    cmd = oracle.from_spec(st.spec)
    res, counts = {}, {}
    for t in (threads, 1):
        runs = []
        while len(runs) < 3 or (sum(runs) < budget_s / 2 and len(runs) < 50):
            t0 = time.perf_counter()
            cmd.run(*st.vals, nthreads=t)
            runs.append(time.perf_counter() - t0)
        res[t] = statistics.median(runs)
        counts[t] = len(runs)
    byts, elems = st.bytes, st.elements
    v = byts / res[threads] / 1e9
    return {
        "value": round(v, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": "%s, all %d elements, the same seeded inputs; median of %d runs on %d threads, %d on one"
                  % (st.name, elems, counts[threads], threads, counts[1]),
        "seconds": round(res[threads], 4), "gelem_per_s": round(elems / res[threads] / 1e9, 4),
        "single_thread": {"gbps": round(byts / res[1] / 1e9, 3), "seconds": round(res[1], 3)},
        "gpu_over_oracle": round(gpu_gbps / v, 1),
        "gpu_over_oracle_single_thread": round(gpu_gbps / (byts / res[1] / 1e9), 1),
        "threads_rule": "CPUs in this process's affinity mask, within the cgroup CPU quota and OMP_NUM_THREADS",
        "host": host_snapshot(),
    }


def counters_record(wl, kernel_hash):
    """The committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary for the
    workload, if the kernels have not changed since it was taken (else None)."""
    path = os.path.join(PROFILES, "counters_%s.json" % wl.replace("@", "_"))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    return c if c.get("kernel_source_hash") == kernel_hash else None


def headline(a, flush, threads, khash):
    """The K steps of the headline workload, cold: the timed region is K
    steps, each a flush and one launch whose dispatch records a pair of HIP
    events at its start and end (one process, so no barrier; synchronised on
    both sides)."""
    import torch
    st = Setup(a.workload)
    bound = st.cmd.bind(*st.args)
    settled = settle(bound)
    for _ in range(a.warmup):
        bound.launch()
    torch.cuda.synchronize()
    per = time_each(bound, a.steps, flush)
    torch.cuda.synchronize()
    kernel_ms = sum(per)
    mean_us = kernel_ms * 1e3 / a.steps
    gbps = st.bytes * a.steps / (kernel_ms * 1e-3) / 1e9
    # after the timed region: the same cold steps between ordinary events
    pairs = time_each(bound, a.steps, flush, dispatch=True)
    return st, per, pairs, mean_us, gbps, settled


def headline_staggered(a, st, flush):
    """The headline's K cold steps again over copies of its operands placed
    by ecmd.empty_staggered (operand k starting k * 4 KiB past a 32 KiB
    boundary) instead of torch's 2 MiB-aligned tensors: the same kernel, bytes
    and values, another placement in HBM.  Reported beside the headline, not
    as its value; the outputs must equal the headline's bit for bit."""
    import torch

    import elementwise_tensor_commands_amd as ecmd
    tensors = [v for v in st.args if isinstance(v, torch.Tensor)]
    if not all(t.is_contiguous() for t in tensors):
        # a copy would change the views' layout, hence the path and the kernel
        return {"skipped": "the headline's operands are not all contiguous"}, None
    placed = iter(ecmd.empty_staggered([(t.shape, t.dtype) for t in tensors]))
    args = []
    for v in st.args:
        if isinstance(v, torch.Tensor):
            t = next(placed)
            t.copy_(v)
            args.append(t)
        else:
            args.append(v)
    n_out = len(st.outs)
    for t in args[-n_out:]:
        t.zero_()
    ptrs = [t.data_ptr() for t in args if isinstance(t, torch.Tensor)]
    bound = st.cmd.bind(*args)
    settled = settle(bound)
    for _ in range(a.warmup):
        bound.launch()
    torch.cuda.synchronize()
    per = time_each(bound, a.steps, flush)
    torch.cuda.synchronize()
    same = all(bool(torch.equal(x.view(torch.uint8), y.view(torch.uint8)))
               for x, y in zip(args[-n_out:], st.outs))
    gbps = st.bytes * a.steps / (sum(per) * 1e-3) / 1e9
    r = {"what": "the headline's kernel over the same values in operands placed 4 KiB apart modulo 32 KiB "
                 "(ecmd.empty_staggered) instead of torch's 2 MiB-aligned tensors; not the headline value",
         "offsets_mod_32k": [(p - ptrs[0]) % ecmd.STAGGER_PERIOD for p in ptrs],
         "step_us": _stats_us(per), "gbps": round(gbps, 2), "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
         "outputs_equal_headline": same}
    return r, [settled + a.warmup, a.steps]


# ---------------------------------------------------------------------------
# rocprofv3 summaries for profiles/.  A profiled run of this script launches
# the ecmd kernels in the order its JSON line's launch_sequence lists (per
# workload: warm-up, back-to-back, warm per-launch, cold per-launch, host-cost
# launches); the summaries split the profiler's ecmd dispatches by that order.


def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    return rows


def _bench_line(path):
    with open(path) as f:
        return json.loads([l for l in f.read().splitlines() if l.startswith("{")][-1])


def _split(rows, sequence):
    """rows: the ecmd dispatches in launch order; sequence: [[workload, [count
    per phase]], ...].  Returns {workload: [rows of each phase]} for the
    workloads fully covered."""
    out, i = {}, 0
    for name, counts in sequence:
        if i + sum(counts) > len(rows):
            break
        phases = []
        for c in counts:
            phases.append(rows[i:i + c])
            i += c
        out[name] = phases
    return out


def _order(r):
    return (int(r.get("Dispatch_Id") or 0), int(r.get("Start_Timestamp") or 0))


def summarize_trace(directory, bench_json, command, plain_json=None):
    """profiles/kernel_trace_<workload>.txt and kernel_trace_summary.md from a
    rocprofv3 --kernel-trace --stats run of this script and the JSON line that
    run printed: per workload, the kernel's own durations per phase beside the
    HIP-event figures of the line.  plain_json: the line of the same command
    run without the profiler on the same box just before (under the profiler
    the dispatch-recorded events read about 4 us longer per launch), compared
    the same way."""
    line = _bench_line(bench_json)
    plain = _bench_line(plain_json) if plain_json else None
    khash = line["kernel_source_hash"]
    disp = sorted((r for r in _csv_rows(directory, "kernel_trace.csv") if "ecmd::" in r["Kernel_Name"]), key=_order)
    stats = {r["Name"]: r for r in _csv_rows(directory, "kernel_stats.csv")}
    split = _split(disp, line["launch_sequence"])
    table = ["# Kernel durations: rocprofv3 kernel trace against bench.py's HIP events", "",
             "Command:", "", "    " + command, "",
             "kernel source hash: %s" % khash, "",
             "Per workload: the kernel trace's median over the cold per-launch phase (for the headline: its "
             "cold steps) and mean over the back-to-back phase, against the same figures of the bench line "
             "printed by the profiled run and by the same command run without the profiler on the same box "
             "just before (\"plain\").", "",
             "| workload | kernel | trace cold us | profiled bench cold us | diff | plain bench cold us | diff | "
             "trace back-to-back us | profiled bench us | diff | plain bench us | diff |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|"]

    def dur_us(rs):
        return [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]

    def pct(a, b):
        return "%.2f %%" % (100 * (b - a) / a) if a and b else "-"

    def figures(ln, name):
        """(cold median us, back-to-back us) of a workload in a bench line."""
        if ln is None:
            return None, None
        if name.startswith("headline:"):
            src = ln.get("placement", {}) if name.endswith("@staggered") else ln
            return (src["step_us"]["median_us"], None) if "step_us" in src else (None, None)
        c = ln.get("commands", {}).get(name)
        if not c or "cold" not in c:
            return None, None
        return c["cold"]["median_us"], c["warm"]["avg_us"]

    fmt = lambda v: "%.3f" % v if v else "-"
    for name, phases in split.items():
        if name.endswith("@graph"):
            continue
        names = sorted({r["Kernel_Name"] for ph in phases for r in ph})
        headline_row = name.startswith("headline:")
        cold = dur_us(phases[1] if headline_row else phases[3])
        b2b = None if headline_row else statistics.mean(dur_us(phases[1]))
        tr_cold = statistics.median(cold)
        pc, pb = figures(line, name)
        qc, qb = figures(plain, name)
        text = ["kernel trace: %s" % name, "", "command:", "    " + command, "", "kernels: " + "; ".join(names), "",
                "trace, cold %s median: %.3f us over %d launches" % ("step" if headline_row else "per-launch",
                                                                      tr_cold, len(cold)),
                "bench line of the profiled run: %s us (%s)" % (fmt(pc), pct(tr_cold, pc)),
                "bench line of the plain run:    %s us (%s)" % (fmt(qc), pct(tr_cold, qc))]
        if b2b:
            text += ["trace, back-to-back mean: %.3f us" % b2b,
                     "bench line of the profiled run: %s us (%s)" % (fmt(pb), pct(b2b, pb)),
                     "bench line of the plain run:    %s us (%s)" % (fmt(qb), pct(b2b, qb))]
        table.append("| %s | `%s` | %.3f | %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            name, names[0][:60], tr_cold, fmt(pc), pct(tr_cold, pc), fmt(qc), pct(tr_cold, qc),
            fmt(b2b), fmt(pb), pct(b2b, pb), fmt(qb), pct(b2b, qb)))
        for n in names:
            if n in stats:
                text += ["", "rocprofv3 kernel stats row (all dispatches of this kernel name in the run):"]
                text += ["    %s: %s" % (k, v) for k, v in stats[n].items()]
        text.append("kernel source hash: %s" % khash)
        fname = name.replace("headline:", "headline_").replace("@", "_")
        with open(os.path.join(PROFILES, "kernel_trace_%s.txt" % fname), "w") as out:
            out.write("\n".join(text) + "\n")
    with open(os.path.join(PROFILES, "kernel_trace_summary.md"), "w") as out:
        out.write("\n".join(table) + "\n")
    print("\n".join(table))


def summarize_counters(fetch_dir, fetch_json, write_dir, write_json, command):
    """profiles/counters_<workload>.json and counters_summary.md from two
    rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) and the JSON lines they printed.  Each counter is scaled by what
    it reads for the plain copy copy_f32 (1 GiB read, 1 GiB written); as an
    independent check of the FETCH_SIZE scale, the cache flush (torch's sum
    over 1 GiB, a read of known size by code outside this library) is scaled
    the same way."""
    import workloads as W
    khash = kernel_source_hash()

    def per_workload(directory, bench_json):
        rows = [r for r in _csv_rows(directory, "counter_collection.csv")]
        ecmd_rows = sorted((r for r in rows if "ecmd::" in r["Kernel_Name"]), key=_order)
        flush = [float(r["Counter_Value"]) for r in rows
                 if "ecmd::" not in r["Kernel_Name"] and float(r["Counter_Value"]) > 256 * 1024]
        line = _bench_line(bench_json)
        split = _split(ecmd_rows, line["launch_sequence"])
        res = {}
        for name, phases in split.items():
            rs = [r for ph in phases for r in ph]
            res[name] = (sorted({r["Kernel_Name"] for r in rs}), statistics.mean(float(r["Counter_Value"]) for r in rs),
                         len(rs))
        return res, flush

    fetch, flush_f = per_workload(fetch_dir, fetch_json)
    write, _ = per_workload(write_dir, write_json)
    assert "copy_f32" in fetch and "copy_f32" in write, "the copy must be measured for the calibration"
    cr, cw = W.algorithmic_read_write("copy_f32")
    cal_f, cal_w = cr / (fetch["copy_f32"][1] * 1024), cw / (write["copy_f32"][1] * 1024)
    flush_kib = statistics.median(flush_f) if flush_f else None
    lines = ["# L2-to-fabric traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
             "Commands (one counter per run):", "", "    " + command, "",
             "These counters count the bytes the L2 caches move to and from the fabric (the last-level "
             "cache and HBM behind it); they do not tell last-level cache hits from HBM accesses.", "",
             "Calibration: the plain copy `copy_f32` (2^28 fp32: 1 GiB read, 1 GiB written) reads "
             "FETCH_SIZE = %.0f KiB and WRITE_SIZE = %.0f KiB per dispatch, so FETCH_SIZE is scaled by "
             "%.4f and WRITE_SIZE by %.4f." % (fetch["copy_f32"][1], write["copy_f32"][1], cal_f, cal_w), ""]
    if flush_kib:
        lines += ["Independent check of the FETCH_SIZE scale: the cache flush (torch's sum over 2^28 fp32, "
                  "1 GiB read) reads FETCH_SIZE = %.0f KiB per dispatch: scale %.4f from it alone." % (
                      flush_kib, (1 << 30) / (flush_kib * 1024)), ""]
    lines += ["kernel source hash: %s" % khash, "",
              "| workload | kernel | dispatches | FETCH KiB | WRITE KiB | read B (scaled) | algorithmic read B | "
              "ratio | written B (scaled) | algorithmic write B | ratio |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    for name in fetch:
        if name not in write or name.startswith("headline:") or name.endswith("@graph"):
            continue
        base = split_workload(name)[0]
        spec_wl = "int_fused" if base == "int_fused_wide" else base
        names, f, nf = fetch[name]
        _, w, _ = write[name]
        rd, wr = W.algorithmic_read_write(spec_wl)
        fb, wb = f * 1024 * cal_f, w * 1024 * cal_w
        rec = {"workload": name, "kernel": names, "dispatches": nf, "fetch_kib_per_dispatch": f,
               "write_kib_per_dispatch": w, "fetch_scale": cal_f, "write_scale": cal_w,
               "fetch_scale_from_flush": (1 << 30) / (flush_kib * 1024) if flush_kib else None,
               "read_bytes_per_launch": fb, "write_bytes_per_launch": wb,
               "hbm_bytes_per_launch": fb + wb, "algorithmic_read_bytes": rd,
               "algorithmic_write_bytes": wr, "read_ratio": fb / rd if rd else None,
               "write_ratio": wb / wr, "kernel_source_hash": khash, "command": command}
        with open(os.path.join(PROFILES, "counters_%s.json" % name.replace("@", "_")), "w") as out:
            json.dump(rec, out, indent=1)
        lines.append("| %s | `%s` | %d | %.0f | %.0f | %.0f | %d | %s | %.0f | %d | %.4f |" % (
            name, names[0][:70], nf, f, w, fb, rd, "%.4f" % (fb / rd) if rd else "-", wb, wr, wb / wr))
    with open(os.path.join(PROFILES, "counters_summary.md"), "w") as out:
        out.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_lds(directory, bench_json, command):
    """profiles/lds_bank_conflicts.md from a rocprofv3 --pmc SQ_LDS_BANK_CONFLICT
    SQ_LDS_IDX_ACTIVE SQ_INSTS_LDS run of this script and the JSON line it
    printed: per workload, the counters per dispatch of its kernel."""
    line = _bench_line(bench_json)
    per = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if "ecmd::" not in r["Kernel_Name"]:
            continue
        d = per.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"], "order": _order(r)})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    disp = sorted(per.values(), key=lambda d: d["order"])
    split = _split(disp, line["launch_sequence"])
    lines = ["# LDS bank conflicts (rocprofv3 SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE, SQ_INSTS_LDS)", "",
             "Command:", "", "    " + command, "",
             "kernel source hash: %s" % line["kernel_source_hash"], "",
             "Per dispatch, averaged over the workload's dispatches.  SQ_LDS_IDX_ACTIVE counts the cycles LDS "
             "instructions keep the LDS busy, SQ_LDS_BANK_CONFLICT the cycles of those lost to bank conflicts.", "",
             "| workload | kernel | dispatches | SQ_INSTS_LDS | SQ_LDS_IDX_ACTIVE | SQ_LDS_BANK_CONFLICT | "
             "conflict share |", "|---|---|---|---|---|---|---|"]
    for name, phases in split.items():
        ds = [d for ph in phases for d in ph]
        if not ds or name.startswith("headline:"):
            continue
        mean = {c: statistics.mean(d.get(c, 0.0) for d in ds)
                for c in ("SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT")}
        share = mean["SQ_LDS_BANK_CONFLICT"] / mean["SQ_LDS_IDX_ACTIVE"] if mean["SQ_LDS_IDX_ACTIVE"] else 0.0
        lines.append("| %s | `%s` | %d | %.0f | %.0f | %.0f | %.2f %% |" % (
            name, sorted({d["name"] for d in ds})[0][:80], len(ds), mean["SQ_INSTS_LDS"], mean["SQ_LDS_IDX_ACTIVE"],
            mean["SQ_LDS_BANK_CONFLICT"], 100 * share))
    with open(os.path.join(PROFILES, "lds_bank_conflicts.md"), "w") as out:
        out.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--all", action="store_true", help="also measure the further workloads")
    ap.add_argument("--only", default="", help="comma-separated workloads to measure under commands "
                                               "(instead of the default set)")
    ap.add_argument("--no-commands", action="store_true", help="the headline only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true", help="skip the full-size oracle comparisons")
    ap.add_argument("--reps", type=int, default=REPS, help="per-launch event pairs per workload, warm and cold")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_DIR", "FETCH_JSON", "WRITE_DIR", "WRITE_JSON"),
                    help="write profiles/ counter summaries from two rocprofv3 --pmc runs of this script and exit")
    ap.add_argument("--summarize-trace", nargs="+", metavar="DIR BENCH_JSON [PLAIN_JSON]",
                    help="write profiles/kernel_trace_*.txt from a kernel-trace run of this script (its directory "
                         "and JSON line, optionally the line of the same command run without the profiler) and exit")
    ap.add_argument("--summarize-lds", nargs=2, metavar=("DIR", "BENCH_JSON"),
                    help="write profiles/lds_bank_conflicts.md from an LDS-counter run of this script and exit")
    ap.add_argument("--command", default="", help="the profiling command, recorded in the summary")
    a = ap.parse_args()
    if a.summarize_counters:
        summarize_counters(*a.summarize_counters, a.command)
        return
    if a.summarize_lds:
        summarize_lds(*a.summarize_lds, a.command)
        return
    if a.summarize_trace:
        summarize_trace(a.summarize_trace[0], a.summarize_trace[1], a.command,
                        a.summarize_trace[2] if len(a.summarize_trace) > 2 else None)
        return
    if a.gpus != 1:
        print("bench.py runs on exactly one GPU: there is no multi-GPU path "
              "(--gpus %d requested)" % a.gpus, file=sys.stderr)
        sys.exit(2)
    import torch

    import workloads as W
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    khash = kernel_source_hash()
    threads = oracle_threads()
    flush = Flusher()
    base, variant = split_workload(a.workload)
    label = W.WORKLOADS[base]["label"] + (" (%s)" % variant if variant else "")
    log("headline %s: %s, %d cold steps" % (a.workload, label, a.steps))
    st, per, pairs, mean_us, gbps, settled = headline(a, flush, threads, khash)
    log("headline %s: %.1f GB/s cold, kernel mean %.2f us" % (st.plan["kernel"], gbps, mean_us))
    placement, placement_seq = headline_staggered(a, st, flush)
    log("headline, staggered operands: %s" % json.dumps(placement))
    if placement_seq and not placement["outputs_equal_headline"]:
        log("WARNING: the headline over staggered operands gave other outputs (recorded in the line)")
    cnt = counters_record(a.workload, khash)
    line = {
        "metric": METRIC,
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(mean_us / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_OF[base],
        "data": "synthetic (seeded NumPy PCG64, seed 1000 + config index), resident in HBM; "
                "each step cold (last-level cache flushed before it, outside its HIP events)",
        "config": {"workload": label, "elements": st.elements,
                   "algorithmic_bytes_per_step": st.bytes, "kernel": st.plan["kernel"],
                   "grid": st.plan["grid"], "block": st.plan["block"]},
        "pct_of_peak": round(100 * gbps / PEAK_GBPS, 2),
        "gelem_per_s": round(st.elements * a.steps / (sum(per) * 1e-3) / 1e9, 3),
        "step_us": _stats_us(per),
        "step_us_with_dispatch": dict(_stats_us(pairs), gbps=round(st.bytes * len(pairs) / (sum(pairs) * 1e-3) / 1e9, 2),
                                      what="the same K cold steps again after the timed region, between "
                                           "ordinary HIP events recorded on the stream around each launch: "
                                           "the command processor's dispatch latency included"),
        "roofline": {
            "bound": "hbm", "achieved": round(gbps, 2), "peak": PEAK_GBPS, "unit": "GB/s",
            "frac": round(gbps / PEAK_GBPS, 4),
            "traffic": cnt["hbm_bytes_per_launch"] if cnt else None,
            "kernel_avg_us": round(mean_us, 3),
        },
        "kernel_source_hash": khash,
    }
    if cnt:
        line["roofline"]["traffic_counters"] = {
            "what": "L2-to-fabric bytes per launch (rocprofv3 FETCH_SIZE, WRITE_SIZE), scaled by the plain "
                    "copy's reading; MALL hits are not told apart from HBM",
            "fetch_kib_raw": cnt["fetch_kib_per_dispatch"], "write_kib_raw": cnt["write_kib_per_dispatch"],
            "fetch_scale": cnt["fetch_scale"], "write_scale": cnt["write_scale"],
            "read_ratio": cnt["read_ratio"], "write_ratio": cnt["write_ratio"]}
    if not a.no_parity:
        log("oracle on %d threads: full-size parity of the headline" % threads)
        line["parity"], _, _ = parity(st, threads)
        log("headline parity: %s" % json.dumps(line["parity"]))
    line["placement"] = placement
    line["launch_sequence"] = [["headline:" + a.workload, [settled + a.warmup, a.steps, a.steps]]]
    if placement_seq:
        line["launch_sequence"].append(["headline:" + a.workload + "@staggered", placement_seq])
    line["settle_launches"] = settled
    if not a.no_commands:
        names = a.only.split(",") if a.only else CONFIGS + LINE_EXTRA + (ALL_EXTRA if a.all else [])
        line["commands"] = {}
        for name in names:
            log("measuring %s" % name)
            r, s2 = measure(name, max(a.steps, 50), a.warmup, flush, threads, check=not a.no_parity, reps=a.reps)
            line["launch_sequence"].append([name, r.pop("launch_sequence")])
            line["commands"][name] = r
            del s2
            torch.cuda.empty_cache()
            log("%s: %s" % (name, json.dumps(r)))
        if "add_f32" in names:
            g = measure_graph("add_f32")
            line["launch_sequence"].append(["add_f32@graph", g.pop("launch_sequence")])
            line["commands"]["add_f32@graph"] = g
            log("add_f32@graph: %s" % json.dumps(g))
        copies = {}
        if "copy_f32" in line["commands"]:
            copies["copy_f32"] = line["commands"]["copy_f32"]["cold"]["gbps"]
        tc = torch_copy_gbps(flush)
        line["torch_copy"] = tc
        copies["torch_copy"] = tc["gbps"]
        ref_name = max(copies, key=copies.get)
        line["copy_reference"] = {"workload": ref_name, "cold_gbps": copies[ref_name],
                                  "rule": "the faster plain 1 GiB copy of this run, cold"}
        for name, r in line["commands"].items():
            if "cold" in r:
                r["pct_of_copy"] = round(100 * r["cold"]["gbps"] / copies[ref_name], 2)
        line["pct_of_copy"] = round(100 * gbps / copies[ref_name], 2)
        line["ctypes_call_us"] = round(ctypes_call_us(), 3)
    if not a.no_cpu_baseline:
        log("timing the CPU oracle")
        line["cpu_baseline"] = cpu_baseline(st, threads, gbps)
    line["env"] = env_snapshot()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
