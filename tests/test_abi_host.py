"""The C ABI on the host: symbols, validation, lowering and path selection.
CPU only -- cmd_plan and cmd_dump make no HIP call, and every cmd_launch here
fails a check before its first HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import elementwise_tensor_commands_amd as E
import workloads as W
from specs import SPECS, arg_dtypes

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ecmd.h")


def test_library_exports_every_declared_function():
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:int|int32_t|int64_t|const char \*)\s*(cmd_\w+)\s*\(", text, re.M))
    assert declared >= {"cmd_create", "cmd_destroy", "cmd_load", "cmd_scalar", "cmd_op", "cmd_store",
                        "cmd_launch", "cmd_plan", "cmd_dump", "cmd_last_error", "cmd_version"}
    lib = ctypes.CDLL(E.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.cmd_version() == 100


def test_struct_layout_matches_header():
    assert ctypes.sizeof(E.cmd_arg) == 88
    assert E.cmd_arg.ptr.offset == 8 and E.cmd_arg.size.offset == 16 and E.cmd_arg.bits.offset == 80
    assert ctypes.sizeof(E.cmd_plan_info) == 136
    assert E.cmd_plan_info.size.offset == 40 and E.cmd_plan_info.kernel.offset == 72


def _t(*shape, dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def _err(fn, name):
    with pytest.raises(E.Error) as e:
        fn()
    assert e.value.name == name, str(e.value)
    return e.value


# ---------------------------------------------------------------------------
# Building.

def test_build_errors():
    c = E.Command()
    x = c.load("f32")
    i = c.load("i32")
    h = c.load("f16")
    _err(lambda: c.add(x, i), "CMD_E_DTYPE")
    _err(lambda: c.add(x, 17), "CMD_E_TAG")
    bh = c.load("bf16")
    _err(lambda: c.add(h, bh), "CMD_E_DTYPE")                       # binary16 and bfloat16 do not mix
    _err(lambda: c.op(E.E_NEG, x, -1, "i32"), "CMD_E_DTYPE")
    _err(lambda: c.op(E.E_NEG, x, x), "CMD_E_ARG")
    _err(lambda: c.op(99, x, x), "CMD_E_ARG")
    _err(lambda: c.op(E.E_SELECT, x, x), "CMD_E_ARG")                # ternary: cmd_select only
    _err(lambda: c.op(E.E_CMP["lt"], x, x, "f32"), "CMD_E_DTYPE")    # comparisons give int32
    _err(lambda: c.cmp("ltu", x, x), "CMD_E_DTYPE")                  # unsigned needs int32
    _err(lambda: c.cmp("geu", bh, bh), "CMD_E_DTYPE")                # unsigned needs int32
    assert c.add(h, h) >= 0 and c.mul(bh, bh) >= 0 and c.cmp("lt", h, h) >= 0   # 16-bit compute types
    _err(lambda: c.min(x, i), "CMD_E_DTYPE")
    _err(lambda: c.select(x, x, x), "CMD_E_DTYPE")                   # condition must be int32
    _err(lambda: c.select(i, x, h), "CMD_E_DTYPE")                   # values of one dtype
    _err(lambda: c.select(i, x, 77), "CMD_E_TAG")
    assert c.cmp("gtu", i, i) >= 0 and c.select(i, h, h) >= 0 and c.abs(h) >= 0 and c.max(x, x) >= 0
    _err(lambda: c.load(7), "CMD_E_DTYPE")
    _err(lambda: c.load("f32", 5), "CMD_E_LIMIT")
    _err(lambda: c.load("f32", 0), "CMD_E_LIMIT")
    assert c.load("f32", 3) >= 0 and c.load("f32", 4) >= 0
    _err(lambda: c.store(99), "CMD_E_TAG")
    assert c.neg(h) >= 0 and c.cvt(h, "i32") >= 0


def test_nostore_and_frozen():
    c = E.Command()
    x = c.load("f32")
    _err(lambda: c.plan(_t(4)), "CMD_E_NOSTORE")
    _err(lambda: c.store(x), "CMD_E_STATE")      # the first plan froze it
    c2 = E.from_spec(W.ADD_F32)
    c2.plan(_t(4), _t(4), _t(4))
    _err(lambda: c2.load("f32"), "CMD_E_STATE")


def test_argument_limits():
    c = E.Command()
    for _ in range(16):
        c.load("f32")
    _err(lambda: c.load("f32"), "CMD_E_LIMIT")
    c = E.Command()
    xs = [c.load("f32") for _ in range(9)]
    acc = xs[0]
    for v in xs[1:]:
        acc = c.add(acc, v)
    c.store(acc)
    _err(lambda: c.plan(*[_t(8)] * 10), "CMD_E_LIMIT")    # nine live loads


def test_too_many_live_temporaries():
    c = E.Command()
    x = c.load("f32")
    ts = [c.neg(x)]
    for _ in range(8):
        ts.append(c.neg(ts[-1]))
    acc = ts[0]
    for t in ts[1:]:
        acc = c.add(acc, t)          # all nine negations alive until summed
    c.store(acc)
    _err(lambda: c.plan(_t(8), _t(8)), "CMD_E_LIMIT")


# ---------------------------------------------------------------------------
# Binding values.

def test_binding_errors():
    c = E.from_spec(W.ADD_F32)
    _err(lambda: c.plan(_t(4), _t(4)), "CMD_E_ARG")                       # count
    _err(lambda: c.plan(_t(4), _t(5), _t(4)), "CMD_E_SHAPE")
    _err(lambda: c.plan(_t(4), _t(4, dtype=torch.int32), _t(4)), "CMD_E_DTYPE")
    _err(lambda: c.plan(_t(4), _t(2, 2), _t(4)), "CMD_E_SHAPE")           # rank 2 for a rank-1 load
    b = _t(16)
    _err(lambda: c.plan(b[:8], b[4:12], b[6:14]), "CMD_E_ALIAS")          # output overlaps an input
    o = _t(8)
    c.plan(o, b[:8], o)                                                   # identical view: in place
    two = E.from_spec(W.MIXED_TWO_OUT)
    h = _t(8, dtype=torch.float16)
    buf = _t(8)
    _err(lambda: two.plan(h, h, h, 0.5, buf.view(torch.float16)[:8], buf), "CMD_E_ALIAS")   # outputs overlap


def _raw_args(c, views):
    arr = (E.cmd_arg * len(views))()
    for i, v in enumerate(views):
        for k, val in v.items():
            if k in ("size", "stride"):
                for d, x in enumerate(val):
                    getattr(arr[i], k)[d] = x
            else:
                setattr(arr[i], k, val)
    return arr


def test_raw_stride_and_null_errors():
    c = E.from_spec(W.ADD_F32)
    x = _t(64)
    good = dict(kind=E.ARG_TENSOR, dtype=E.F32, ptr=x.data_ptr(), size=(8, 0), stride=(1, 0))
    info = E.cmd_plan_info()
    args = _raw_args(c, [good, dict(good, stride=(-1, 0)), good])
    assert E.lib.cmd_plan(c._h, args, 3, ctypes.byref(info)) == -5
    args = _raw_args(c, [good, good, dict(good, ptr=None)])
    assert E.lib.cmd_plan(c._h, args, 3, ctypes.byref(info)) == -1
    out = _t(64)
    args = _raw_args(c, [good, good, dict(good, ptr=out.data_ptr(), stride=(0, 0))])
    assert E.lib.cmd_plan(c._h, args, 3, ctypes.byref(info)) == -5         # non-injective store
    args = _raw_args(c, [good, dict(good, stride=(0, 0)), dict(good, ptr=out.data_ptr())])
    assert E.lib.cmd_plan(c._h, args, 3, ctypes.byref(info)) == 0          # broadcast load is fine
    assert info.path == E.PATH_ROWS                                        # one row with a broadcast value
    args = _raw_args(c, [good, good, dict(good, ptr=out.data_ptr(), reserved=1)])
    assert E.lib.cmd_plan(c._h, args, 3, ctypes.byref(info)) == -1
    args = _raw_args(c, [good, good, dict(good, ptr=out.data_ptr() + 1)])
    assert E.lib.cmd_plan(c._h, args, 3, ctypes.byref(info)) == -1         # not element aligned
    assert b"aligned" in E.lib.cmd_last_error(c._h)


def test_launch_checks_precede_any_hip_call():
    """On this GPU-less host, a launch that fails a check returns that check's
    code (not CMD_E_LAUNCH): nothing reached the HIP runtime."""
    c = E.from_spec(W.ADD_F32)
    for bad, name in (((_t(4), _t(5), _t(4)), "CMD_E_SHAPE"),
                      ((_t(4), _t(4, dtype=torch.int32), _t(4)), "CMD_E_DTYPE"),
                      ((_t(4), _t(4)), "CMD_E_ARG")):
        with pytest.raises(E.Error) as e:
            c.launch(*bad, stream=0)
        assert e.value.name == name
    b = _t(16)
    with pytest.raises(E.Error) as e:
        c.launch(b[:8], b[:8], b[1:9], stream=0)
    assert e.value.name == "CMD_E_ALIAS"


def test_empty_launch_succeeds_without_gpu():
    c = E.from_spec(W.ADD_F32)
    c.launch(_t(0), _t(0), _t(0), stream=0)
    assert c.plan(_t(0), _t(0), _t(0))["path"] == "none"


# ---------------------------------------------------------------------------
# Lowering.

def test_shared_subexpression_evaluated_once():
    c = E.from_spec(W.MIXED_TWO_OUT)
    d = c.dump()
    ops = [l for l in d.splitlines() if re.match(r"s\d+ = ", l)]
    assert sum(1 for l in ops if "mul.f32" in l) == 2            # t = x*y once, and u*v
    assert sum(1 for l in ops if "cvt.f16.f32" in l) == 3
    assert len(ops) == 9


def test_select_and_compare_lowering():
    """A select's three operands stay alive until it runs; comparisons and
    min/max list the smaller reference first when they commute."""
    c = E.Command()
    x = c.load("f32")
    y = c.load("f32")
    lt = c.cmp("lt", y, x)
    eq = c.cmp("eq", y, x)
    m = c.min(y, x)
    s = c.select(lt, m, c.neg(x))
    c.store(s)
    c.store(eq)
    d = c.dump()
    assert "lt.f32 in1, in0" in d and "eq.f32 in0, in1" in d and "min.f32 in0, in1" in d
    assert re.search(r"s\d = select s\d, s\d, s\d", d), d


def test_fill_plan():
    c = E.Command()
    v = c.scalar("f32")
    c.store(v)
    p = c.plan(2.5, _t(1000))
    assert p["path"] == "linear" and p["kernel"] == "linear_fill_f32"


def test_dead_code_is_dropped():
    c = E.Command()
    x = c.load("f32")
    y = c.load("f32")
    c.mul(x, y)                      # never stored
    c.store(c.neg(x))
    d = c.dump()
    assert "mul" not in d and "in1" not in d
    plan = c.plan(_t(8), _t(8), _t(8))
    assert plan["path"] == "linear"


def test_same_type_cvt_is_an_alias():
    c = E.Command()
    x = c.load("f32")
    a = c.cvt(x, "f32")
    c.store(c.add(a, x))
    assert c.dump().count("add.f32 in0, in0") == 1


def test_commutative_operands_canonical():
    specs = [W.AXPBY_F32, [("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)),
                           ("alpha", ("scalar", "f32")), ("beta", ("scalar", "f32")),
                           ("ax", ("mul", "x", "alpha")), ("by", ("mul", "y", "beta")),
                           ("r", ("add", "by", "ax")), ("out", ("store", "r", 1))]]
    dumps = [E.from_spec(s).dump() for s in specs]
    assert dumps[0] == dumps[1]


@pytest.mark.parametrize("wl,kernel", [("add_f32", "linear_add_f32"), ("int_fused", "linear_int_fused"),
                                       ("axpby_f32", "linear_axpby_f32"),
                                       ("mixed_two_out", "linear_mixed_two_out"),
                                       ("transposed_2d", "tiled_add_scaled_f32"),
                                       ("batched_transpose", "tiled_add_scaled_f32"),
                                       ("bias_nchw", "rows_affine_f32"),
                                       ("odd_rows_f32", "gather_segments"),
                                       ("narrow_rows_f32", "gather_whole_rows")])
def test_workloads_select_their_kernels(wl, kernel):
    spec = W.WORKLOADS[wl]["spec"]
    n = 1 << 12 if wl != "transposed_2d" else 256
    small = {"batched_transpose": (3, 64, 96), "bias_nchw": (2, 8, 4, 16), "odd_rows_f32": (33, 1001),
             "narrow_rows_f32": (1000, 6)}
    vals, extra = W.make_inputs(wl, n, shape=small.get(wl))
    n = None if wl in small else n
    tv = W.to_torch(vals, extra, "cpu")
    _, outs = arg_dtypes(spec)
    shape = W.shape_of(wl, n, small.get(wl))
    o = [torch.empty(shape, dtype={"f16": torch.float16, "f32": torch.float32, "i32": torch.int32}[d]) for d in outs]
    plan = E.from_spec(spec).plan(*tv, *o)
    assert plan["kernel"] == kernel and bool(plan["specialised"] and plan["vector"]) == (plan["path"] != "gather")


def test_geometry_rules():
    """Work-group and grid obey the dispatch rules: grid >= 1, work-group size
    nonzero and at most 1024, LDS within 64 KiB."""
    c = E.from_spec(W.ADD_F32)
    for n in (1, 7, 8, 2048, 1 << 20, 1 << 26):
        p = c.plan(_t(n), _t(n), _t(n))
        assert p["grid"] >= 1 and 0 < p["block"] <= 1024 and p["lds_bytes"] <= 65536
    c2 = E.from_spec(W.TRANSPOSED_2D)
    for R, C in ((2, 2), (65, 129), (1000, 3)):
        X = _t(R, C)
        Y = _t(C, R)
        p = c2.plan(X, Y.t(), 2.0, _t(R, C))
        assert p["grid"] >= 1 and p["block"] in ((64,) if p["path"] == "gather" else (256, 512)), p


def test_unaligned_views_pick_slower_variants():
    c = E.from_spec(W.ADD_F32)
    b = _t(40)
    assert not c.plan(b[1:33], b[:32], _t(32))["vector"]
    c2 = E.from_spec(W.TRANSPOSED_2D)
    Xs = _t(64, 67)
    Y = _t(64, 64)
    assert c2.plan(Xs[:, :64], Y.t(), 2.0, _t(64, 64))["path"] == "gather"     # row stride 67: not 16B
    Xs = _t(64, 68)
    assert c2.plan(Xs[:, :64], Y.t(), 2.0, _t(64, 64))["path"] == "tiled"


# ---------------------------------------------------------------------------
# A test-only executor of the lowered listing (numpy arithmetic, no FMA) run
# against the oracle: it catches lowering mistakes (slot reuse, operand order,
# aliasing) without a GPU.

def _bf_vals(a):
    """bfloat16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _bf_round(x):
    """float32 values -> bfloat16 bit patterns, torch's round-to-nearest-even."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _i32_to_bf(a):
    """int32 -> bfloat16 rounded once from the exact integer (Python integers)."""
    out = []
    for i in np.asarray(a, dtype=np.int64).tolist():
        m = abs(i)
        if m < (1 << 24):
            out.append(int(_bf_round(np.array([np.float32(i)]))[0]))
            continue
        ulp = 1 << (m.bit_length() - 8)
        lo = (m // ulp) * ulp
        up = 2 * (m - lo) > ulp or (2 * (m - lo) == ulp and (lo // ulp) % 2 == 1)
        v = float(lo + ulp if up else lo) * (1 if i > 0 else -1)
        out.append(int(_bf_round(np.array([v], dtype=np.float32))[0]))   # exact in binary32
    return np.array(out, dtype=np.uint16)


def _minmax_zero_fix(A, B, r, is_min, zero):
    z = (A == 0) & (B == 0)
    neg = np.signbit(A) | np.signbit(B) if is_min else np.signbit(A) & np.signbit(B)
    return np.where(z, np.where(neg, -zero, zero), r)


def _emulate(listing, ins, uni, n, lds=False):
    """Runs the listing (or, with lds, its form over the interpreters' LDS
    entries: input k starts in entry k, results go where the host placed
    them) with NumPy arithmetic and returns the stored values."""
    regs = {}
    outs = []
    f16 = np.float16

    def f2i(a):
        a = a.astype(np.float64)
        r = np.where(np.isnan(a), 0, np.clip(np.trunc(np.nan_to_num(a)), -2**31, 2**31 - 1))
        return r.astype(np.int64).astype(np.int32)
    for k, v in enumerate(ins):
        regs[("e%d" if lds else "in%d") % k] = v
    for k, v in enumerate(uni):
        regs["u%d" % k] = np.full(n, v)
    for line in listing.splitlines():
        if line.startswith("lds ") != lds:
            continue
        line = line[4:] if lds else line
        m = re.match(r"([se]\d+) = (\S+) (\S+?)(?:, (\S+?))?(?:, (\S+))?$", line)
        if m:
            dst, op, a, b, c = m.groups()
            A = regs[a]
            B = regs[b] if b else None
            C = regs[c] if c else None
            with np.errstate(all="ignore"):
                if op.endswith(".bf16") and op.split(".")[0] in ("add", "sub", "mul"):
                    x, y = _bf_vals(A), _bf_vals(B)
                    # binary32 result rounded to bfloat16 = the exact result rounded once
                    r = _bf_round({"add": x + y, "sub": x - y, "mul": x * y}[op.split(".")[0]])
                elif op in ("min.bf16", "max.bf16"):
                    x, y = _bf_vals(A), _bf_vals(B)
                    r = _minmax_zero_fix(x, y, (np.fmin if op == "min.bf16" else np.fmax)(x, y),
                                         op == "min.bf16", np.float32(0.0))
                    r = _bf_round(r)
                elif op == "cvt.f16.bf16": r = _bf_round(A.astype(np.float32))
                elif op == "cvt.bf16.f16": r = _bf_vals(A).astype(f16)
                elif op == "cvt.bf16.f32": r = _bf_vals(A)
                elif op == "cvt.f32.bf16": r = _bf_round(A)
                elif op == "cvt.bf16.i32": r = f2i(_bf_vals(A))
                elif op == "cvt.i32.bf16": r = _i32_to_bf(A)
                elif op == "abs.bf16": r = (A & 0x7FFF).astype(np.uint16)
                elif op in ("add.f32", "add.i32", "add.f16"): r = A + B
                elif op in ("sub.f32", "sub.i32", "sub.f16"): r = A - B
                elif op in ("mul.f32", "mul.i32", "mul.f16"): r = A * B
                elif op.startswith("neg"): r = (A.view(np.uint32 if A.itemsize == 4 else np.uint16) ^ (0x80000000 if A.itemsize == 4 else 0x8000)).view(A.dtype) if op != "neg.i32" else (np.int32(0) - A)
                elif op == "cvt.f16.f32": r = A.astype(np.float32)
                elif op == "cvt.f32.f16": r = A.astype(f16)
                elif op == "cvt.i32.f32": r = A.astype(np.float32)
                elif op == "cvt.f32.i32": r = f2i(A)
                elif op == "cvt.i32.f16": r = A.astype(np.float64).astype(f16)
                elif op == "cvt.f16.i32": r = f2i(A.astype(np.float32))
                elif op.split(".")[0] in ("eq", "ne", "lt", "le", "gt", "ge"):
                    X, Y = (A.view(np.uint32), B.view(np.uint32)) if op.endswith(".u32") else \
                        ((_bf_vals(A), _bf_vals(B)) if op.endswith(".bf16") else (A, B))
                    r = getattr(np, {"eq": "equal", "ne": "not_equal", "lt": "less", "le": "less_equal",
                                     "gt": "greater", "ge": "greater_equal"}[op.split(".")[0]])(X, Y).astype(np.int32)
                elif op in ("min.i32", "max.i32"): r = (np.minimum if op == "min.i32" else np.maximum)(A, B)
                elif op in ("min.f32", "max.f32", "min.f16", "max.f16"):
                    r = (np.fmin if op.startswith("min") else np.fmax)(A, B)
                    # order -0 below +0 on ties
                    r = _minmax_zero_fix(A, B, r, op.startswith("min"), A.dtype.type(0.0))
                elif op.startswith("abs"):
                    r = (A.view(np.uint32) & 0x7FFFFFFF).view(A.dtype) if op == "abs.f32" else \
                        ((A.view(np.uint16) & 0x7FFF).view(A.dtype) if op == "abs.f16" else np.abs(A))
                elif op == "select": r = np.where(A != 0, B, C)
                else: raise AssertionError(op)
            regs[dst] = r
            continue
        m = re.match(r"store\.\S+ arg\d+ <- (\S+)", line)
        if m:
            outs.append(regs[m.group(1)])
    return outs


def _max_live(listing, n_in):
    """max(n_in, the largest number of values an operation needs at once: the
    values made earlier and read later, plus its result)."""
    slot, last, defs, ops = {}, {}, [], []
    for k in range(n_in):
        defs.append(("in%d" % k, -1))
    for line in listing.splitlines():
        m = re.match(r"(s\d+) = \S+ (.*)$", line)
        if m:
            i = len(ops)
            reads = []
            for r in m.group(2).split(", "):
                v = slot.get(r, r) if r.startswith("s") else r
                if not r.startswith("u"):
                    reads.append(v)
                    last[v] = i
            v = "v%d" % i
            slot[m.group(1)] = v
            defs.append((v, i))
            ops.append(reads)
        m = re.match(r"store\.\S+ arg\d+ <- (\S+)$", line)
        if m and not m.group(1).startswith("u"):
            r = m.group(1)
            last[slot.get(r, r) if r.startswith("s") else r] = len(ops) + 1   # read after the tape
    peak = 0
    for i in range(len(ops)):
        live = sum(1 for v, d in defs if d < i and last.get(v, -1) > i)
        peak = max(peak, live + 1)
    return max(n_in, peak)


@pytest.mark.parametrize("seed", range(40))
def test_lowered_listing_matches_oracle(oracle_mod, seed):
    import random_commands as G
    rng = np.random.default_rng(1000 + seed)
    spec = G._random_spec(rng, int(rng.integers(1, 5)), int(rng.integers(1, 14)), 1)
    n = 257
    vals = G._random_inputs(rng, spec, (n,))
    try:
        ref = oracle_mod.from_spec(spec).run(*vals)
    except oracle_mod.OracleError:
        pytest.skip("invalid random Command")
    c = E.from_spec(spec)
    try:
        listing = c.dump()
    except E.Error as e:
        assert e.name == "CMD_E_LIMIT"
        pytest.skip(str(e))
    # inputs / uniforms in the listing's numbering: live loads and scalars in order
    in_args = [int(a) for a in re.findall(r"in\d+ = load\.\S+ arg(\d+)", listing)]
    u_args = [int(a) for a in re.findall(r"u\d+ = scalar\.\S+ arg(\d+)", listing)]
    ins = [vals[a] for a in in_args]
    uni = [vals[a] for a in u_args]
    # the listing, then the same program over the interpreters' LDS entries
    for lds in (False, True):
        got = _emulate(listing, ins, uni, n, lds)
        assert len(got) == len(ref)
        for k, (g, r) in enumerate(zip(got, ref)):
            g = np.asarray(g).astype(r.dtype) if np.asarray(g).dtype != r.dtype else g
            gb = g.view(np.uint16 if r.itemsize == 2 else np.uint32)
            rb = r.view(np.uint16 if r.itemsize == 2 else np.uint32)
            if r.dtype.kind == "f":
                ok = (gb == rb) | (np.isnan(g) & np.isnan(r))
            elif r.dtype == np.uint16:          # bfloat16 bit patterns: any NaN equals any NaN
                ok = (gb == rb) | (np.isnan(_bf_vals(gb)) & np.isnan(_bf_vals(rb)))
            else:
                ok = gb == rb
            assert ok.all(), "seed %d out%d (lds %s)\n%s" % (seed, k, lds, listing)
    # entries in use: exactly max(inputs, the most values live at one operation)
    # -- the optimum for values live over intervals
    n_ent = int(re.search(r"^lds entries (\d+)$", listing, re.M).group(1))
    assert n_ent == _max_live(listing, len(ins)), listing


# Hand-counted LDS entries of the interpreters' register file: (spec, entries).
# Inputs keep entries 0 .. n_in - 1; a result takes a dying operand's entry
# (or the lowest free one); values a later operation or a store reads stay.
_ENTRY_CASES = [
    # no operations: a uniform value stored (no entry), an input passed through
    ([("s", ("scalar", "f32")), ("o", ("store", "s", 1))], 0),
    ([("x", ("load", "f32", 1)), ("o", ("store", "x", 1))], 1),
    # x + x: x dies at its only use, the sum takes its entry
    ([("x", ("load", "f32", 1)), ("t", ("add", "x", "x")), ("o", ("store", "t", 1))], 1),
    # x stored as well as used: it stays live to the end, the sum needs a second entry
    ([("x", ("load", "f32", 1)), ("t", ("add", "x", "x")), ("o0", ("store", "t", 1)),
      ("o1", ("store", "x", 1))], 2),
    # select over three inputs: all die at it
    ([("c", ("load", "i32", 1)), ("a", ("load", "f32", 1)), ("b", ("load", "f32", 1)),
      ("r", ("select", "c", "a", "b")), ("o", ("store", "r", 1))], 3),
    # a chain over one input and a uniform: everything in place
    ([("x", ("load", "f32", 1)), ("s", ("scalar", "f32")), ("t", ("mul", "x", "s")), ("u", ("add", "t", "s")),
      ("v", ("max", "u", "s")), ("o", ("store", "v", 1))], 1),
    # two values kept for two stores while a third is made
    ([("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)), ("t", ("add", "x", "y")), ("u", ("sub", "x", "y")),
      ("w", ("mul", "t", "u")), ("o0", ("store", "t", 1)), ("o1", ("store", "w", 1))], 3),
]


@pytest.mark.parametrize("case", range(len(_ENTRY_CASES)))
def test_interpreter_entries(oracle_mod, case):
    """The entry count of hand-worked programs, and the entry form of each
    run with NumPy against the oracle."""
    spec, want = _ENTRY_CASES[case]
    c = E.from_spec(spec)
    listing = c.dump()
    assert int(re.search(r"^lds entries (\d+)$", listing, re.M).group(1)) == want, listing
    n = 33
    rng = np.random.default_rng(case)
    vals = []
    for _, st in spec:
        if st[0] == "load":
            vals.append(rng.integers(0, 2, n, dtype=np.int32) if st[1] == "i32" else
                        rng.standard_normal(n).astype(np.float32))
        elif st[0] == "scalar":
            vals.append(np.float32(0.75))
    loads = any(st[0] == "load" for _, st in spec)
    # without loads the stores give the shape
    ref = oracle_mod.from_spec(spec).run(*vals, outputs=None if loads else [np.zeros(n, np.float32)])
    in_args = [int(a) for a in re.findall(r"in\d+ = load\.\S+ arg(\d+)", listing)]
    u_args = [int(a) for a in re.findall(r"u\d+ = scalar\.\S+ arg(\d+)", listing)]
    got = _emulate(listing, [vals[a] for a in in_args], [vals[a] for a in u_args], n, lds=True)
    assert len(got) == len(ref)
    for g, r in zip(got, ref):
        g = np.broadcast_to(np.asarray(g, dtype=r.dtype), r.shape)
        assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), listing
