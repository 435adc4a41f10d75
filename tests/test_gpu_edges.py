"""Edge values through the vector bodies of every kernel family on the GPU.

The hand-worked cases of tests/golden/hand_worked.txt run packed side by side
(case i % m at element i) over thousands of elements, so that each edge value
reaches the ahead-of-time kernels' vector bodies, the interpreters' tape walks
(linear, rows, tiled and gather paths) and the run-time compiled kernels, not
only their per-element tails; each element is compared with its case's
hand-worked result.  Then every pair of binary32 / int32 edge values plus 2^20
random pairs runs through each operation on the linear path's three kernel
kinds, against the oracle; the int32 fused Command on full-range int32
inputs (wraparound in nearly every element) at full size on its ahead-of-time
kernel; and the mixed-precision two-output Command at full size with its
per-element ulp report.
"""
import os
from collections import defaultdict

import numpy as np
import pytest
import torch

import test_oracle_pins as P
import workloads as W
from edge_values import conditions, pairs32
from gpu_util import NPD, compare, dev, host, run_oracle, to_dev
from specs import SPECS, arg_dtypes, input_kinds

pytestmark = pytest.mark.gpu

N_PACKED = 4 * 1024 + 21          # two super-chunks of the largest interpreter plus a ragged tail
NPU = {"f16": np.uint16, "bf16": np.uint16, "f32": np.uint32, "i32": np.uint32}


def _groups():
    """Golden cases grouped by (spec, scalar inputs): one launch per group."""
    g = defaultdict(list)
    for ln, name, ins, expect in P.GOLDEN_CASES:
        kinds = input_kinds(SPECS[name])
        scal = tuple(b for k, b in zip(kinds, ins) if k == "scalar")
        g[(name, scal)].append((ln, ins, expect))
    return sorted(g.items())


GROUPS = _groups()
GROUP_IDS = ["%s-%s" % (k[0], "-".join("%x" % s for s in k[1])) if k[1] else k[0] for k, _ in GROUPS]


def _rank2(spec):
    return [(n, (st[0], st[1], 2) if st[0] == "load" else (st[0], st[1], 2) if st[0] == "store" else st)
            for n, st in spec]


def _scalar_value(b, dt):
    if dt == "bf16":
        return np.uint16(b)
    if dt == "i32":
        return int(np.array(b, dtype=np.uint32).view(np.int32))
    return float(np.array(b, dtype=NPU[dt]).view(NPD[dt]))


def _check_packed(got, cases, k, dt, total, what):
    """Element e of the logical order holds case e % m's result."""
    m = len(cases)
    exp = np.array([c[2][k] for c in cases], dtype=np.uint64)[np.arange(total) % m]
    gb = np.ascontiguousarray(got).reshape(-1).view(NPU[dt]).astype(np.uint64)
    nan_case = np.array([P.is_nan_bits(c[2][k], dt) for c in cases])[np.arange(total) % m]
    if dt in ("f16", "bf16", "f32"):
        isnan = np.array([P.is_nan_bits(int(v), dt) for v in np.unique(gb)])
        nan_vals = set(np.unique(gb)[isnan].tolist())
        got_nan = np.isin(gb, list(nan_vals)) if nan_vals else np.zeros(total, bool)
    else:
        got_nan = np.zeros(total, bool)
    bad = np.flatnonzero(np.where(nan_case, ~got_nan, gb != exp))
    if bad.size:
        i = bad[0]
        ln = cases[i % m][0]
        raise AssertionError("%s out%d: %d of %d elements wrong; first at %d (golden line %d): expected %#x, GPU %#x"
                             % (what, k, bad.size, total, i, ln, int(exp[i]), int(gb[i])))


def _launch(spec, gv, out_specs, jit=False, generic=False):
    import elementwise_tensor_commands_amd as ecmd
    old = os.environ.get("ECMD_FORCE_GENERIC")
    if generic:
        os.environ["ECMD_FORCE_GENERIC"] = "1"
    try:
        cmd = ecmd.from_spec(spec)
        if jit:
            cmd.aot(False).jit(ecmd.JIT_SYNC)
        outs = [torch.empty(s, dtype={"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32,
                                      "i32": torch.int32}[d], device=dev()) for s, d in out_specs]
        cmd.launch(*gv, *outs)
        torch.cuda.synchronize()
        plan = cmd.plan(*gv, *outs)
    finally:
        if generic:
            if old is None:
                os.environ.pop("ECMD_FORCE_GENERIC", None)
            else:
                os.environ["ECMD_FORCE_GENERIC"] = old
    return plan, outs


@pytest.mark.parametrize("path", ["linear", "linear_interp", "linear_jit", "rows", "tiled", "gather"])
@pytest.mark.parametrize("group", range(len(GROUPS)), ids=GROUP_IDS)
def test_hand_worked_packed(path, group):
    (name, scal), cases = GROUPS[group]
    spec = SPECS[name]
    in_dt, out_dt = arg_dtypes(spec)
    kinds = input_kinds(spec)
    m = len(cases)
    tensor_pos = [i for i, k in enumerate(kinds) if k == "load"]
    if path in ("rows", "tiled"):
        spec = _rank2(spec)
        R, C = (132, 108) if path == "tiled" else (63, 68)
    else:
        R, C = 1, N_PACKED
    total = R * C
    # per tensor input: the logical values, element e = case e % m
    logical = {}
    for i in tensor_pos:
        col = np.array([c[1][i] for c in cases], dtype=np.uint64)[np.arange(total) % m]
        logical[i] = col.astype(NPU[in_dt[i]]).view(NPD[in_dt[i]])
    gv = []
    si = iter(scal)
    for i, (k, dt) in enumerate(zip(kinds, in_dt)):
        if k == "scalar":
            gv.append(_scalar_value(next(si), dt))
            continue
        v = logical[i]
        if path in ("linear", "linear_interp", "linear_jit"):
            gv.append(to_dev(v))
        elif path == "gather":                     # every other element of a twice-as-long storage
            st = np.zeros(2 * total, dtype=v.dtype)
            st[::2] = v
            gv.append(to_dev(st)[::2])
        elif path == "rows":                       # rows padded to C + 4
            st = np.zeros((R, C + 4), dtype=v.dtype)
            st[:, :C] = v.reshape(R, C)
            gv.append(to_dev(st)[:, :C])
        else:                                      # tiled: the first input direct, the others transposed
            if i == tensor_pos[0] and len(tensor_pos) > 1:
                gv.append(to_dev(v.reshape(R, C)))
            else:
                gv.append(to_dev(np.ascontiguousarray(v.reshape(R, C).T)).t())
    shape = (R, C) if path in ("rows", "tiled") else (total,)
    plan, outs = _launch(spec, gv, [(shape, d) for d in out_dt], jit=path == "linear_jit",
                         generic=path == "linear_interp")
    want = {"linear": "linear", "linear_interp": "linear", "linear_jit": "linear", "rows": "rows",
            "tiled": "tiled", "gather": "gather"}[path]
    assert plan["path"] == want, plan
    if path == "linear_interp":
        assert plan["kernel"] == "linear_generic", plan
    if path == "linear_jit":
        assert plan["compiled"], plan
    for k, (o, dt) in enumerate(zip(outs, out_dt)):
        _check_packed(host(o), cases, k, dt, total, "%s %s %s" % (name, path, plan["kernel"]))


# ---------------------------------------------------------------------------
# Every pair of binary32 / int32 edge values, and random pairs.

F32_BINARY = ["add_f32", "sub_f32", "mul_f32", "min_f32", "max_f32"] + \
             ["cmp_%s_f32" % c for c in ("eq", "ne", "lt", "le", "gt", "ge")]
I32_BINARY = ["add_i32", "sub_i32", "mul_i32", "min_i32", "max_i32"] + \
             ["cmp_%s_i32" % c for c in ("eq", "ne", "lt", "le", "gt", "ge", "ltu", "leu", "gtu", "geu")]
F32_UNARY = ["neg_f32", "abs_f32", "cvt_f32_i32", "cvt_f32_f16", "cvt_f32_bf16"]
I32_UNARY = ["neg_i32", "abs_i32", "cvt_i32_f32", "cvt_i32_f16", "cvt_i32_bf16"]


def _pair_inputs(name):
    dt = "f32" if name in F32_BINARY + F32_UNARY + ["select_f32"] else "i32"
    a, b = pairs32(dt)
    npd = np.float32 if dt == "f32" else np.int32
    if name.startswith("select_"):
        return [conditions(a.size).view(np.int32), a.view(npd), b.view(npd)]
    if name in F32_UNARY or name in I32_UNARY:
        return [np.unique(np.concatenate([a, b])).view(npd)]
    return [a.view(npd), b.view(npd)]


@pytest.mark.parametrize("kind", ["default", "interp", "jit"])
@pytest.mark.parametrize("name", F32_BINARY + I32_BINARY + F32_UNARY + I32_UNARY + ["select_f32", "select_i32"])
def test_edge_pairs_32bit(name, kind):
    spec = SPECS[name]
    vals = _pair_inputs(name)
    ref = run_oracle(spec, vals)
    _, out_dt = arg_dtypes(spec)
    n = vals[0].size
    plan, outs = _launch(spec, [to_dev(v) for v in vals], [((n,), d) for d in out_dt], jit=kind == "jit",
                         generic=kind == "interp")
    assert plan["path"] == "linear", plan
    if kind == "interp":
        assert plan["kernel"] == "linear_generic", plan
    if kind == "jit":
        assert plan["compiled"], plan
    for k, (o, r) in enumerate(zip(outs, ref)):
        compare(host(o), r, 0, "%s %s n=%d out%d" % (name, plan["kernel"], n, k))


# ---------------------------------------------------------------------------
# Full-size runs of the configurations' own kernels on edge-rich data.

def test_int_fused_full_range_full_size():
    """Configuration 1's Command on full-range int32 inputs at its full size,
    on its ahead-of-time kernel: x + y and the product wrap in nearly every
    element (its own inputs, drawn from [-2^15, 2^15), wrap with probability
    2^-48 per element)."""
    n = 1 << 24
    rng = np.random.default_rng(W.seed_of("int_fused") + 100)
    x, y, w = (rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32) for _ in range(3))
    # plus the hand-worked wrap cases at the start, in the tail and mid-vector
    x[:3], y[:3], w[:3] = [2**31 - 1, -32768, -1], [1, -32768, -1], [2, -32768, -1]
    x[-5:], y[-5:], w[-5:] = -2**31, -2**31, -1
    vals = [x, y, w, np.int32(12345)]
    ref = run_oracle(W.INT_FUSED, vals)[0]
    wraps = int(np.count_nonzero((x.astype(np.int64) + y) != (x + y).astype(np.int64)))
    print("  int fused full range: %d of %d sums wrap" % (wraps, n), flush=True)
    assert wraps > n // 8
    plan, (o,) = _launch(W.INT_FUSED, [to_dev(x), to_dev(y), to_dev(w), 12345], [((n,), "i32")])
    assert plan["kernel"] == "linear_int_fused", plan
    compare(host(o), ref, 0, "int fused full range")
    assert int(host(o)[0]) == -12345 and int(host(o)[1]) == 2147471303


def _ulp_hist(got, ref):
    width = got.itemsize * 8
    ut = {2: np.uint16, 4: np.uint32}[got.itemsize]
    sign = 1 << (width - 1)

    def ordered(b):
        b = b.astype(np.int64)
        return np.where(b & sign, -(b & (sign - 1)), b)

    d = np.abs(ordered(got.view(ut).ravel()) - ordered(ref.view(ut).ravel()))
    return int(d.max()), [int((d == 0).sum()), int((d == 1).sum()), int((d == 2).sum()), int((d > 2).sum())]


def test_mixed_full_size_ulp_report():
    """Configuration 3 at full size: per-element ulp distance of each output in
    its own type, histogram {0, 1, 2, >2} printed.  The bar is 2 ulp; 0 is
    what the arithmetic gives (x*y of two binary16 values is exact in
    binary32, so every later rounding is unique), and 0 is asserted."""
    wl = "mixed_two_out"
    n = W.WORKLOADS[wl]["n"]
    vals, extra = W.make_inputs(wl, n)
    ref = run_oracle(W.MIXED_TWO_OUT, vals)
    gv = W.to_torch(vals, extra, dev())
    plan, outs = _launch(W.MIXED_TWO_OUT, gv, [((n,), "f16"), ((n,), "f32")])
    assert plan["kernel"] == "linear_mixed_two_out", plan
    for k, (o, r) in enumerate(zip(outs, ref)):
        g = host(o)
        assert not np.isnan(g).any() and not np.isnan(r).any()
        worst, hist = _ulp_hist(g, r)
        print("  mixed out%d: max %d ulp, histogram {0: %d, 1: %d, 2: %d, >2: %d}" % (k, worst, *hist), flush=True)
        assert worst <= 2, "out%d: %d ulp" % (k, worst)
        assert worst == 0, "out%d: %d ulp (bar 2; 0 expected), histogram %s" % (k, worst, hist)
