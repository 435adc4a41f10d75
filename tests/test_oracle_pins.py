"""Pins for the oracle: hand-worked values, closed forms, invariants, library
special cases and brute force.  CPU only; nothing here touches a GPU.

The oracle must be right before it can judge the GPU path, so every part of it
is checked against something other than itself:
  * hand-worked bit patterns (tests/golden/hand_worked.txt);
  * NumPy's own float32/int32/float16 arithmetic and casts (NumPy never fuses
    multiply-add and wraps int32 silently);
  * binary64 evaluation: +, -, * done in binary64 and rounded once to binary32
    equal the correctly rounded binary32 result, because binary64 carries at
    least 2*24+2 significant bits (Figueroa, "When is double rounding
    innocuous?", 1995);
  * algebraic identities that hold bit for bit in two's-complement and IEEE
    arithmetic.
"""
import os

import numpy as np
import pytest
import torch

import workloads as W
from specs import SPECS, arg_dtypes, input_kinds

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.txt")
NPD = {"f16": np.float16, "bf16": np.uint16, "f32": np.float32, "i32": np.int32}
NPU = {"f16": np.uint16, "bf16": np.uint16, "f32": np.uint32, "i32": np.uint32}


def load_golden():
    cases = []
    with open(GOLDEN) as f:
        for ln, line in enumerate(f, 1):
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            spec, ins, outs = [p.strip() for p in line.split("|")]
            cases.append((ln, spec, [int(v, 16) for v in ins.split()],
                          [int(v, 16) for v in outs.split()]))
    return cases


def is_nan_bits(bits, dt):
    if dt == "f16":
        return (bits & 0x7C00) == 0x7C00 and (bits & 0x3FF) != 0
    if dt == "bf16":
        return (bits & 0x7F80) == 0x7F80 and (bits & 0x7F) != 0
    if dt == "f32":
        return (bits & 0x7F800000) == 0x7F800000 and (bits & 0x7FFFFF) != 0
    return False


def run_bits(oracle_mod, spec_name, in_bits, n=1):
    """Run a spec on length-n inputs filled with the given bit patterns."""
    spec = SPECS[spec_name]
    cmd = oracle_mod.from_spec(spec)
    in_dt, out_dt = arg_dtypes(spec)
    vals = []
    for kind, dt, b in zip(input_kinds(spec), in_dt, in_bits):
        if kind == "scalar":
            vals.append(np.array(b, dtype=NPU[dt]).view(NPD[dt]).reshape(()))
        else:
            vals.append(np.full(n, b, dtype=NPU[dt]).view(NPD[dt]))
    outs = cmd.run(*vals)
    return [o.view(NPU[dt]) for o, dt in zip(outs, out_dt)], out_dt


GOLDEN_CASES = load_golden()


@pytest.mark.parametrize("case", GOLDEN_CASES, ids=["L%d-%s" % (c[0], c[1]) for c in GOLDEN_CASES])
def test_hand_worked(oracle_mod, case):
    ln, spec, ins, expect = case
    outs, out_dt = run_bits(oracle_mod, spec, ins, n=3)
    for o, e, dt in zip(outs, expect, out_dt):
        for got in o:
            got = int(got)
            if is_nan_bits(e, dt):
                assert is_nan_bits(got, dt), "line %d: expected NaN, got %#x" % (ln, got)
            else:
                assert got == e, "line %d: expected %#x, got %#x" % (ln, e, got)


def test_golden_covers_every_spec_family():
    names = {c[1] for c in GOLDEN_CASES}
    for need in ("add_f32", "int_fused", "axpby_f32", "mixed_two_out", "neg_f32", "neg_i32",
                 "cvt_f32_f16", "cvt_f16_f32", "cvt_i32_f32", "cvt_f32_i32", "cvt_i32_f16",
                 "cvt_f16_i32", "mul_i32", "mul_f32", "sub_f32"):
        assert need in names


def test_fp_environment(oracle_mod):
    assert oracle_mod.lib().oracle_check_fpenv() == 0


# ---------------------------------------------------------------------------
# Workloads against NumPy's own arithmetic, at reduced sizes.

def test_add_f32_vs_numpy(oracle_mod):
    vals, _ = W.make_inputs("add_f32")
    (z,) = oracle_mod.from_spec(W.ADD_F32).run(*vals)
    assert np.array_equal(z.view(np.uint32), (vals[0] + vals[1]).view(np.uint32))


@pytest.mark.parametrize("wide", [False, True])
def test_int_fused_vs_numpy(oracle_mod, wide):
    n = 1 << 16
    if wide:   # full int32 range so that every step wraps often
        rng = np.random.default_rng(7)
        x, y, w = (rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32) for _ in range(3))
        vals = [x, y, w, np.int32(12345)]
    else:
        vals, _ = W.make_inputs("int_fused", n)
    (z,) = oracle_mod.from_spec(W.INT_FUSED).run(*vals)
    with np.errstate(over="ignore"):
        ref = (vals[0] + vals[1]) * vals[2] - np.int32(12345)
    assert ref.dtype == np.int32
    assert np.array_equal(z, ref)


def test_axpby_vs_numpy_and_binary64(oracle_mod):
    vals, _ = W.make_inputs("axpby_f32", 1 << 16)
    x, y, a, b = vals
    (o,) = oracle_mod.from_spec(W.AXPBY_F32).run(*vals)
    ref = a * x + b * y
    assert np.array_equal(o.view(np.uint32), ref.view(np.uint32))
    # each step rounded once from binary64
    ax = (np.float64(a) * x.astype(np.float64)).astype(np.float32)
    by = (np.float64(b) * y.astype(np.float64)).astype(np.float32)
    r64 = (ax.astype(np.float64) + by.astype(np.float64)).astype(np.float32)
    assert np.array_equal(o.view(np.uint32), r64.view(np.uint32))
    # and a contracted evaluation differs on this data (the data can see contraction)
    fused = (np.float64(a) * x.astype(np.float64) + by.astype(np.float64)).astype(np.float32)
    assert np.count_nonzero(fused.view(np.uint32) != o.view(np.uint32)) > 0


def _mixed_ref_numpy(x, y, z, s):
    x32, y32, z32 = (v.astype(np.float32) for v in (x, y, z))
    t = x32 * y32
    u = t + z32
    v = t - z32
    return (u * v).astype(np.float16), u + np.float32(s)


def test_mixed_vs_numpy(oracle_mod):
    vals, _ = W.make_inputs("mixed_two_out", 1 << 18)
    o0, o1 = oracle_mod.from_spec(W.MIXED_TWO_OUT).run(*vals)
    r0, r1 = _mixed_ref_numpy(*vals)
    assert np.array_equal(o0.view(np.uint16), r0.view(np.uint16))
    assert np.array_equal(o1.view(np.uint32), r1.view(np.uint32))


def test_mixed_within_one_f16_ulp_of_binary64(oracle_mod):
    """out0 against the DAG evaluated in binary64 and rounded once: the binary32
    pipeline's relative error (about 3 * 2^-24) is far below half an fp16 ulp,
    so the two differ by at most one fp16 ulp."""
    vals, _ = W.make_inputs("mixed_two_out", 1 << 18)
    o0, _ = oracle_mod.from_spec(W.MIXED_TWO_OUT).run(*vals)
    x, y, z = (v.astype(np.float64) for v in vals[:3])
    t = x * y
    exact = ((t + z) * (t - z)).astype(np.float16)
    def ordered(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    d = np.abs(ordered(o0.view(np.uint16)) - ordered(exact.view(np.uint16)))
    assert d.max() <= 1


def test_mixed_shared_t_fp16_subnormals_present():
    vals, _ = W.make_inputs("mixed_two_out", 1 << 20)
    x = vals[0].view(np.uint16)
    assert np.count_nonzero(((x & 0x7C00) == 0) & ((x & 0x3FF) != 0)) > 0
    x32 = vals[0].astype(np.float32)
    assert np.all((x32 >= -4) & (x32 < 4))


# ---------------------------------------------------------------------------
# Binary64 pins for single operations on wide-range data.

def _wide_f32(rng, n):
    bits = rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


@pytest.mark.parametrize("op", ["add", "sub", "mul"])
def test_f32_ops_equal_binary64_rounded_once(oracle_mod, op):
    rng = np.random.default_rng(11)
    x = _wide_f32(rng, 1 << 16)
    y = _wide_f32(rng, len(x))
    n = min(len(x), len(y))
    x, y = x[:n], y[:n]
    # also operands close in magnitude, where cancellation and ties happen
    e = rng.integers(-3, 4, n).astype(np.float32)
    x2 = (rng.random(n, dtype=np.float32) + 1) * np.exp2(e)
    y2 = (rng.random(n, dtype=np.float32) + 1) * np.exp2(e)
    x, y = np.concatenate([x, x2]), np.concatenate([y, y2])
    (r,) = oracle_mod.from_spec(SPECS[op + "_f32"]).run(x, y)
    fn = {"add": np.add, "sub": np.subtract, "mul": np.multiply}[op]
    with np.errstate(all="ignore"):
        ref = fn(x.astype(np.float64), y.astype(np.float64)).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(r), nan)
    assert np.array_equal(r.view(np.uint32)[~nan], ref.view(np.uint32)[~nan])


# ---------------------------------------------------------------------------
# Algebraic invariants, each side its own Command.

def _int_full(rng, n):
    v = rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32)
    v[:4] = [np.iinfo(np.int32).min, np.iinfo(np.int32).max, 0, -1]
    return v


def test_int32_invariants(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(5)
    n = 4096
    x, y, w = _int_full(rng, n), _int_full(rng, n), _int_full(rng, n)
    zero, one = np.zeros(n, np.int32), np.ones(n, np.int32)

    def run(steps, *vals):
        return O.from_spec(steps).run(*vals)[0]

    L = lambda nm: (nm, ("load", "i32", 1))
    add = [L("a"), L("b"), ("r", ("add", "a", "b")), ("o", ("store", "r", 1))]
    sub = [L("a"), L("b"), ("r", ("sub", "a", "b")), ("o", ("store", "r", 1))]
    mul = [L("a"), L("b"), ("r", ("mul", "a", "b")), ("o", ("store", "r", 1))]
    neg = [L("a"), ("r", ("neg", "a")), ("o", ("store", "r", 1))]
    assert np.array_equal(run(add, x, zero), x)
    assert np.array_equal(run(mul, x, one), x)
    assert np.array_equal(run(sub, x, x), zero)
    assert np.array_equal(run(add, x, y), run(add, y, x))
    assert np.array_equal(run(mul, x, y), run(mul, y, x))
    assoc_l = [L("a"), L("b"), L("c"), ("ab", ("add", "a", "b")), ("r", ("add", "ab", "c")), ("o", ("store", "r", 1))]
    assoc_r = [L("a"), L("b"), L("c"), ("bc", ("add", "b", "c")), ("r", ("add", "a", "bc")), ("o", ("store", "r", 1))]
    assert np.array_equal(run(assoc_l, x, y, w), run(assoc_r, x, y, w))
    dist_l = [L("a"), L("b"), L("c"), ("ab", ("add", "a", "b")), ("r", ("mul", "ab", "c")), ("o", ("store", "r", 1))]
    dist_r = [L("a"), L("b"), L("c"), ("ac", ("mul", "a", "c")), ("bc", ("mul", "b", "c")),
              ("r", ("add", "ac", "bc")), ("o", ("store", "r", 1))]
    assert np.array_equal(run(dist_l, x, y, w), run(dist_r, x, y, w))
    sub_as_neg = [L("a"), L("b"), ("nb", ("neg", "b")), ("r", ("add", "a", "nb")), ("o", ("store", "r", 1))]
    assert np.array_equal(run(sub, x, y), run(sub_as_neg, x, y))
    assert np.array_equal(run(neg, run(neg, x)), x)
    # and the wrap is real: INT_MIN + (-1) wraps to INT_MAX
    assert run(add, x[:1], np.array([-1], np.int32))[0] == np.iinfo(np.int32).max


def test_f32_invariants(oracle_mod):
    O = oracle_mod
    rng = np.random.default_rng(6)
    x = _wide_f32(rng, 8192)
    y = _wide_f32(rng, len(x))[: len(x)]
    x = x[: len(y)]
    n = len(x)
    bits = lambda a: a.view(np.uint32)
    L = lambda nm: (nm, ("load", "f32", 1))
    def run(op, *vals):
        if op == "neg":
            steps = [L("a"), ("r", ("neg", "a")), ("o", ("store", "r", 1))]
        else:
            steps = [L("a"), L("b"), ("r", (op, "a", "b")), ("o", ("store", "r", 1))]
        return O.from_spec(steps).run(*vals)[0]
    ok = ~np.isnan(run("add", x, y))
    assert np.array_equal(bits(run("add", x, y))[ok], bits(run("add", y, x))[ok])
    ok = ~np.isnan(run("mul", x, y))
    assert np.array_equal(bits(run("mul", x, y))[ok], bits(run("mul", y, x))[ok])
    zero, one = np.zeros(n, np.float32), np.ones(n, np.float32)
    # x + (+0) = x, except -0 + +0 = +0
    r = run("add", x, zero)
    expect = np.where(bits(x) == 0x80000000, np.uint32(0), bits(x))
    assert np.array_equal(bits(r), expect)
    assert np.array_equal(bits(run("mul", x, one)), bits(x))
    assert np.all(bits(run("sub", x, x)) == 0)              # finite x: +0
    r1, r2 = run("sub", x, y), run("add", x, run("neg", y))
    ok = ~np.isnan(r1)
    assert np.array_equal(bits(r1)[ok], bits(r2)[ok])
    assert np.array_equal(bits(run("neg", run("neg", x))), bits(x))
    assert np.array_equal(bits(run("neg", x)), bits(x) ^ np.uint32(0x80000000))


# ---------------------------------------------------------------------------
# Conversions against NumPy's casts.

def test_f16_to_f32_all_patterns(oracle_mod):
    got = oracle_mod.f16_to_f32_all()
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    ref = h.astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got.view(np.float32)), nan)
    assert np.array_equal(got[~nan], ref.view(np.uint32)[~nan])


def _check_f32_to_f16(oracle_mod, bits):
    bits = np.ascontiguousarray(bits, dtype=np.uint32)
    (got,) = oracle_mod.from_spec(SPECS["cvt_f32_f16"]).run(bits.view(np.float32))
    with np.errstate(over="ignore"):
        ref = bits.view(np.float32).astype(np.float16)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    bad = np.flatnonzero(got.view(np.uint16)[~nan] != ref.view(np.uint16)[~nan])
    assert bad.size == 0, [hex(int(b)) for b in bits[~nan][bad[:5]]]


def test_f32_to_f16_every_tie_and_neighbour(oracle_mod):
    """Every binary16 value, every midpoint between neighbouring binary16
    values, and the binary32 values on either side of each midpoint."""
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    up = np.append(h[1:], 65536.0)
    mids = ((h + up) / 2).astype(np.float32)      # exact: at most 12 significant bits
    vals = np.concatenate([h.astype(np.float32), mids,
                           np.nextafter(mids, np.float32(np.inf)),
                           np.nextafter(mids, np.float32(0))])
    vals = np.concatenate([vals, -vals])
    _check_f32_to_f16(oracle_mod, vals.view(np.uint32))


def test_f32_to_f16_structured_and_random(oracle_mod):
    hi = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x2001, 0x3FFF, 0x7FFF,
                     0x8000, 0x8001, 0xEFFF, 0xF000, 0xFFFF], dtype=np.uint32)
    _check_f32_to_f16(oracle_mod, (hi[:, None] | lows[None, :]).ravel())
    rng = np.random.default_rng(3)
    _check_f32_to_f16(oracle_mod, rng.integers(0, 2**32, 1 << 22, dtype=np.uint64).astype(np.uint32))


@pytest.mark.skipif(os.environ.get("ECMD_FULL_SWEEP") != "1",
                    reason="all 2^32 binary32 patterns take minutes; set ECMD_FULL_SWEEP=1")
def test_f32_to_f16_all_2pow32(oracle_mod):
    from concurrent.futures import ThreadPoolExecutor
    chunk = 1 << 24
    def one(k):
        first = k * chunk
        got = oracle_mod.f32_to_f16_range(first, chunk)
        x = np.arange(first, first + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
        with np.errstate(over="ignore"):
            ref = x.astype(np.float16)
        nan = np.isnan(ref)
        return int(np.count_nonzero(got[~nan] != ref.view(np.uint16)[~nan])) + \
            int(np.count_nonzero((got[nan] & 0x7C00) != 0x7C00))
    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as ex:
        assert sum(ex.map(one, range(256))) == 0


def test_f16_roundtrip_identity(oracle_mod):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = oracle_mod.f16_to_f32_all()
    back = np.array([oracle_mod.f32_to_f16_bits(int(v)) for v in f], dtype=np.uint16)
    nan = ((h & 0x7C00) == 0x7C00) & ((h & 0x3FF) != 0)
    assert np.array_equal(back[~nan], h[~nan])


def test_i32_conversions_vs_numpy(oracle_mod):
    rng = np.random.default_rng(9)
    i = _int_full(rng, 1 << 16)
    i = np.concatenate([i, np.arange(-70000, 70000, dtype=np.int32)])
    (f,) = oracle_mod.from_spec(SPECS["cvt_i32_f32"]).run(i)
    assert np.array_equal(f, i.astype(np.float32))
    (h,) = oracle_mod.from_spec(SPECS["cvt_i32_f16"]).run(i)
    with np.errstate(over="ignore"):
        ref = i.astype(np.float64).astype(np.float16)   # one rounding from the exact value
    assert np.array_equal(h.view(np.uint16), ref.view(np.uint16))
    x = np.concatenate([_wide_f32(rng, 1 << 16), np.float32([2.5, -2.5, 2**31 - 128, -2**31])])
    (r,) = oracle_mod.from_spec(SPECS["cvt_f32_i32"]).run(x)
    ok = np.abs(x) < 2**31
    assert np.array_equal(r[ok], np.trunc(x[ok]).astype(np.int32))
    assert np.all(r[(~ok) & (x > 0)] == np.iinfo(np.int32).max)
    assert np.all(r[(~ok) & (x < 0)] == np.iinfo(np.int32).min)


# ---------------------------------------------------------------------------
# 2-D views, tails and bases, brute force.

SHAPES = [(1, 1), (1, 7), (7, 1), (3, 5), (17, 33), (64, 64), (65, 63), (130, 70)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("pad", [0, 1, 64])
@pytest.mark.parametrize("base", [0, 3])
def test_transposed_brute_force(oracle_mod, shape, pad, base):
    R, C = shape
    rng = np.random.default_rng(R * 1000 + C)
    xs = np.full(base + R * (C + pad), np.nan, np.float32)
    X = np.lib.stride_tricks.as_strided(xs[base:], (R, C), ((C + pad) * 4, 4))
    X[...] = rng.random((R, C), dtype=np.float32) * 2 - 1
    Y = rng.random((C, R), dtype=np.float32) * 2 - 1
    (o,) = oracle_mod.from_spec(W.TRANSPOSED_2D).run(X, Y.T, np.float32(2))
    ref = np.empty((R, C), np.float32)
    for i in range(R):                 # element by element
        for j in range(C):
            ref[i, j] = X[i, j] + np.float32(2) * Y[j, i]
    assert np.array_equal(o.view(np.uint32), ref.view(np.uint32))
    assert not np.isnan(o).any()       # NaN padding of X never reaches out


def test_transposed_self_is_three_x(oracle_mod):
    rng = np.random.default_rng(1)
    X = rng.random((96, 80), dtype=np.float32) * 2 - 1
    Y = np.ascontiguousarray(X.T)      # Y^T == X
    (o,) = oracle_mod.from_spec(W.TRANSPOSED_2D).run(X, Y.T, np.float32(2))
    assert np.array_equal(o.view(np.uint32), (np.float32(3) * X).view(np.uint32))


def test_transposed_workload_small(oracle_mod):
    vals, extra = W.make_inputs("transposed_2d", 200)
    (o,) = oracle_mod.from_spec(W.TRANSPOSED_2D).run(*vals)
    ref = vals[0] + np.float32(2) * extra["Y"].T
    assert np.array_equal(o.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n", [0, 1, 2, 3, 5, 7, 8, 15, 17, 31, 33, 63, 65, 255, 257, 1023, 1025, 65537])
@pytest.mark.parametrize("off", [0, 1, 3])
def test_tails_and_offsets(oracle_mod, n, off):
    rng = np.random.default_rng(n + 100 * off)
    xs = rng.random(n + off, dtype=np.float32)
    ys = rng.random(n + off, dtype=np.float32)
    guard = np.full(n + 2 * 16 + off, 7.0, np.float32)
    out = guard[16 + off: 16 + off + n]
    oracle_mod.from_spec(W.ADD_F32).run(xs[off:], ys[off:], outputs=[out])
    assert np.array_equal(out, xs[off:] + ys[off:])
    assert np.all(guard[: 16 + off] == 7.0) and np.all(guard[16 + off + n:] == 7.0)


def test_strided_store_and_broadcast_load(oracle_mod):
    rng = np.random.default_rng(2)
    x = rng.random(10, dtype=np.float32)
    b = np.lib.stride_tricks.as_strided(np.float32([0.25]), (10,), (0,))   # stride-0 load
    out = np.zeros(30, np.float32)
    oracle_mod.from_spec(W.ADD_F32).run(x, b, outputs=[out[::3]])
    assert np.array_equal(out[::3], x + np.float32(0.25))
    assert np.all(out[1::3] == 0) and np.all(out[2::3] == 0)


def test_multithreaded_equals_single(oracle_mod):
    vals, _ = W.make_inputs("mixed_two_out", 100003)
    cmd = oracle_mod.from_spec(W.MIXED_TWO_OUT)
    a = cmd.run(*vals, nthreads=1)
    b = cmd.run(*vals, nthreads=7)
    for p, q in zip(a, b):
        assert np.array_equal(p.view(np.uint8), q.view(np.uint8))


# ---------------------------------------------------------------------------
# The oracle front end's own checks.

def test_front_end_rejects(oracle_mod):
    O = oracle_mod
    c = O.OracleCommand()
    x = c.load("f32")
    i = c.load("i32")
    h = c.load("f16")
    with pytest.raises(O.OracleError):
        c.add(x, i)                    # dtypes differ
    with pytest.raises(O.OracleError):
        c.add(x, 99)                   # unknown tag
    b = c.load("bf16")
    with pytest.raises(O.OracleError):
        c.add(h, b)                    # binary16 and bfloat16 do not mix
    with pytest.raises(O.OracleError):
        c.op("ltu", h, h)              # unsigned comparison needs int32
    with pytest.raises(O.OracleError):
        c.load("f32", 5)
    c3 = O.from_spec([("s", ("scalar", "bf16")), ("o", ("store", "s", 1))])
    with pytest.raises(O.OracleError):
        c3.run(1.5, outputs=[np.zeros(3, np.uint16)])   # bfloat16 scalars are bit patterns
    c2 = O.from_spec(W.ADD_F32)
    with pytest.raises(O.OracleError):
        c2.run(np.zeros(4, np.float32), np.zeros(5, np.float32))
    with pytest.raises(O.OracleError):
        c2.run(np.zeros(4, np.float32), np.zeros(4, np.int32))


# ---------------------------------------------------------------------------
# Comparisons, select, min / max, abs against NumPy on special-value-rich data.

def _special_f32(rng, n):
    x = rng.standard_normal(n).astype(np.float32)
    sp = np.float32([0.0, -0.0, np.inf, -np.inf, np.nan, 1.0, -1.0, 1e-45, -1e-45, 3.4e38])
    idx = rng.integers(0, n, n // 4)
    x[idx] = rng.choice(sp, idx.size)
    return x


def test_new_ops_vs_numpy(oracle_mod):
    from specs import COMPARES, UNSIGNED
    rng = np.random.default_rng(21)
    n = 1 << 14
    x, y = _special_f32(rng, n), _special_f32(rng, n)
    y[: n // 8] = x[: n // 8]                                  # many equal pairs
    npcmp = {"eq": np.equal, "ne": np.not_equal, "lt": np.less, "le": np.less_equal,
             "gt": np.greater, "ge": np.greater_equal}
    with np.errstate(invalid="ignore"):
        for c in COMPARES:
            (r,) = oracle_mod.from_spec(SPECS["cmp_%s_f32" % c]).run(x, y)
            assert np.array_equal(r, npcmp[c](x, y).astype(np.int32)), c
    xi = rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32)
    yi = rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32)
    yi[: n // 8] = xi[: n // 8]
    for c in COMPARES:
        (r,) = oracle_mod.from_spec(SPECS["cmp_%s_i32" % c]).run(xi, yi)
        assert np.array_equal(r, npcmp[c](xi, yi).astype(np.int32)), c
    for c in UNSIGNED:
        (r,) = oracle_mod.from_spec(SPECS["cmp_%s_i32" % c]).run(xi, yi)
        assert np.array_equal(r, npcmp[c[:2]](xi.view(np.uint32), yi.view(np.uint32)).astype(np.int32)), c
    # min / max: NumPy's fmin / fmax ignore a NaN; tied zeros of opposite sign are
    # pinned by the hand-worked cases instead (C's fmin may return either)
    tie = (x == y) & (x == 0)
    for name, fn in (("min", np.fmin), ("max", np.fmax)):
        (r,) = oracle_mod.from_spec(SPECS[name + "_f32"]).run(x, y)
        ref = fn(x, y)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(r), nan)
        ok = ~nan & ~tie
        assert np.array_equal(r.view(np.uint32)[ok], ref.view(np.uint32)[ok]), name
        (ri,) = oracle_mod.from_spec(SPECS[name + "_i32"]).run(xi, yi)
        assert np.array_equal(ri, (np.minimum if name == "min" else np.maximum)(xi, yi))
    (r,) = oracle_mod.from_spec(SPECS["abs_f32"]).run(x)
    assert np.array_equal(r.view(np.uint32), x.view(np.uint32) & np.uint32(0x7FFFFFFF))
    (r,) = oracle_mod.from_spec(SPECS["abs_i32"]).run(xi)
    with np.errstate(over="ignore"):
        assert np.array_equal(r, np.abs(xi))                  # NumPy's abs wraps at INT_MIN too
    cond = rng.integers(-2, 3, n).astype(np.int32)
    (r,) = oracle_mod.from_spec(SPECS["select_f32"]).run(cond, x, y)
    assert np.array_equal(r.view(np.uint32), np.where(cond != 0, x, y).view(np.uint32))


def test_fill_is_a_scalar_store(oracle_mod):
    spec = [("s", ("scalar", "f32")), ("o", ("store", "s", 1))]
    out = np.zeros(37, np.float32)
    oracle_mod.from_spec(spec).run(np.float32(-0.0), outputs=[out])
    assert np.all(out.view(np.uint32) == 0x80000000)


# ---------------------------------------------------------------------------
# Rank-3 and rank-4 views: permuted, broadcast (stride 0), strided; brute force.

def _brute(expr, shape, *arrs):
    """Element-by-element reference: expr applied to the i-th elements."""
    out = np.empty(shape, np.float32)
    for idx in np.ndindex(*shape):
        out[idx] = expr(*(a[idx] for a in arrs))
    return out


@pytest.mark.parametrize("case", range(6))
def test_rank_n_views_brute_force(oracle_mod, case):
    rng = np.random.default_rng(300 + case)
    shape = [(2, 3, 4), (3, 1, 5, 2), (4, 5, 6), (2, 3, 4, 5), (1, 7, 1, 3), (5, 4, 3, 2)][case]
    r = len(shape)
    base = rng.random(shape, dtype=np.float32)
    perm = rng.permutation(r)
    # X: the transpose of a contiguous array, viewed back in the logical order
    xs = np.ascontiguousarray(np.transpose(base, perm))
    X = np.transpose(xs, np.argsort(perm))
    # Y: broadcast along a random dimension (stride 0) of a smaller array
    bd = int(rng.integers(r))
    small = rng.random(tuple(1 if d == bd else s for d, s in enumerate(shape)), dtype=np.float32)
    Y = np.broadcast_to(small, shape)
    # out: every other element of a wider buffer along the last dimension
    wide = np.zeros(shape[:-1] + (2 * shape[-1],), np.float32)
    out = wide[..., ::2]
    spec = [("x", ("load", "f32", r)), ("y", ("load", "f32", r)), ("a", ("scalar", "f32")),
            ("ay", ("mul", "a", "y")), ("o", ("sub", "x", "ay")), ("out", ("store", "o", r))]
    oracle_mod.from_spec(spec).run(X, Y, np.float32(1.5), outputs=[out])
    ref = _brute(lambda x, y: np.float32(x - np.float32(1.5) * y), shape, X, Y)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    assert np.all(wide[..., 1::2] == 0)


def test_rank_mixing_right_aligned(oracle_mod):
    """A rank-1 view of n matches a rank-3 view of shape (1, 1, n)."""
    x = np.arange(7, dtype=np.float32)
    y = np.arange(7, dtype=np.float32).reshape(1, 1, 7) * 2
    spec = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 3)), ("r", ("add", "x", "y")),
            ("o", ("store", "r", 3))]
    (o,) = oracle_mod.from_spec(spec).run(x, y)
    assert o.shape == (1, 1, 7) and np.array_equal(o.ravel(), x * 3)
    with pytest.raises(oracle_mod.OracleError):
        oracle_mod.from_spec(spec).run(x, np.zeros((1, 2, 7), np.float32))


@pytest.mark.parametrize("shape", [(3, 20, 36), (1, 1, 1), (2, 7, 130)])
def test_batched_transpose_workload_matches_numpy(oracle_mod, shape):
    """out[b] = X[b] + 2 * Y[b]^T: numpy's float32 operations round each
    product and sum once, and 2*y is exact."""
    vals, extra = W.make_inputs("batched_transpose", shape=shape)
    (o,) = oracle_mod.from_spec(W.BATCHED_TRANSPOSE).run(*vals)
    Y = extra["storage"][1]
    ref = vals[0] + np.float32(2) * np.transpose(Y, (0, 2, 1))
    assert np.array_equal(o.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("shape", [(2, 5, 3, 7), (1, 1, 1, 1), (3, 16, 1, 9)])
def test_bias_nchw_workload_matches_numpy(oracle_mod, shape):
    """out = x * scale[c] + bias[c] through stride-0 views, against numpy's
    own broadcasting of the per-channel arrays."""
    vals, extra = W.make_inputs("bias_nchw", shape=shape)
    assert vals[1].strides[0] == 0 and vals[1].strides[2:] == (0, 0)
    (o,) = oracle_mod.from_spec(W.BIAS_NCHW).run(*vals)
    _, scale, bias = extra["storage"]
    ref = vals[0] * scale.reshape(1, -1, 1, 1) + bias.reshape(1, -1, 1, 1)
    assert np.array_equal(o.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("shape", [(2, 5, 3, 7), (1, 1, 1, 1), (3, 16, 1, 9)])
def test_bias_nchw_f16_workload_matches_numpy(oracle_mod, shape):
    """The binary16 per-channel map: each operation rounds to binary16, as
    NumPy's float16 multiply and add do (binary32 arithmetic, exact for one
    product or sum of two binary16 values, then one rounding)."""
    vals, extra = W.make_inputs("bias_nchw_f16", shape=shape)
    assert vals[0].dtype == np.float16 and vals[1].strides[0] == 0
    (o,) = oracle_mod.from_spec(W.BIAS_NCHW_F16).run(*vals)
    _, scale, bias = extra["storage"]
    ref = (vals[0] * scale.reshape(1, -1, 1, 1)).astype(np.float16) + bias.reshape(1, -1, 1, 1)
    assert ref.dtype == np.float16
    assert np.array_equal(o.view(np.uint16), ref.view(np.uint16))


def test_transposed_f16_workload_matches_numpy(oracle_mod):
    vals, extra = W.make_inputs("transposed_2d_f16", 96)
    (o,) = oracle_mod.from_spec(W.TRANSPOSED_2D_F16).run(*vals)
    ref = vals[0] + (np.float16(2) * extra["Y"].T).astype(np.float16)
    assert ref.dtype == np.float16
    assert np.array_equal(o.view(np.uint16), ref.view(np.uint16))


# ---------------------------------------------------------------------------
# Native binary16 / bfloat16 arithmetic and bfloat16 conversions.
#
# Library special cases: NumPy's float16 operations and torch's CPU bfloat16
# operations compute in binary32 and round the result to the 16-bit format
# (nearest even).  binary32 has 24 >= 2p + 2 bits for p = 11 and p = 8, so that
# double rounding equals rounding the exact result once (Figueroa 1995) -- the
# definition the oracle implements by a different route (binary64, then its
# own rounding).  torch keeps subnormals on the CPU unless told otherwise.

def _tbf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def _nbf(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _nan16(bits, dt):
    bits = np.asarray(bits, dtype=np.uint16)
    if dt == "bf16":
        return ((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0)
    return ((bits & 0x7C00) == 0x7C00) & ((bits & 0x3FF) != 0)


def _same16(got, ref, dt, what):
    got, ref = np.asarray(got, dtype=np.uint16), np.asarray(ref, dtype=np.uint16)
    ng, nr = _nan16(got, dt), _nan16(ref, dt)
    bad = (ng != nr) | (~ng & (got != ref))
    idx = np.flatnonzero(bad)
    assert idx.size == 0, "%s: %d differ, first %s" % (what, idx.size, [(int(i), hex(got[i]), hex(ref[i])) for i in idx[:5]])


def _special16(dt):
    """Every sign and exponent field with fractions at the edges: zeros,
    subnormals, the largest finite values, infinities, NaN."""
    fb = 10 if dt == "f16" else 7
    eb = 5 if dt == "f16" else 8
    fr = [0, 1, 2, 3, (1 << (fb - 1)) - 1, 1 << (fb - 1), (1 << (fb - 1)) + 1, (1 << fb) - 2, (1 << fb) - 1]
    out = [(s << 15) | (e << fb) | f for s in (0, 1) for e in range(1 << eb) for f in fr]
    return np.array(sorted(set(out)), dtype=np.uint16)


# Sizes of the 16-bit pair sweeps; the planted-mistake harness lowers them.
PAIRS_RANDOM = 1 << 20
PAIRS_SPECIAL_BF16 = 1000


def _pairs16(dt, n_random=None, seed=77):
    n_random = PAIRS_RANDOM if n_random is None else min(n_random, PAIRS_RANDOM)
    sp = _special16(dt)
    if dt == "bf16":                       # 4,600 specials: keep the pairs at ~1M
        rng0 = np.random.default_rng(seed + 1)
        sp = np.sort(rng0.choice(sp, PAIRS_SPECIAL_BF16, replace=False))
    a = np.repeat(sp, sp.size)
    b = np.tile(sp, sp.size)
    rng = np.random.default_rng(seed)
    ra = rng.integers(0, 1 << 16, n_random, dtype=np.uint32).astype(np.uint16)
    rb = rng.integers(0, 1 << 16, n_random, dtype=np.uint32).astype(np.uint16)
    return np.concatenate([a, ra]), np.concatenate([b, rb])


def _oracle16(oracle_mod, spec_name, dt, *ins):
    vals = [x.view(np.float16) if dt == "f16" else x for x in ins]
    (o,) = oracle_mod.from_spec(SPECS[spec_name]).run(*vals, nthreads=8)
    return o.view(np.uint16) if o.dtype != np.int32 else o


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("op", ["add", "sub", "mul"])
def test_16bit_arith_vs_libraries(oracle_mod, op, dt):
    a, b = _pairs16(dt)
    got = _oracle16(oracle_mod, "%s_%s" % (op, dt), dt, a, b)
    if dt == "f16":
        x, y = a.view(np.float16), b.view(np.float16)
        with np.errstate(all="ignore"):
            ref = {"add": x + y, "sub": x - y, "mul": x * y}[op].view(np.uint16)
    else:
        x, y = _tbf(a), _tbf(b)
        ref = _nbf({"add": x + y, "sub": x - y, "mul": x * y}[op])
    _same16(got, ref, dt, "%s %s" % (op, dt))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_16bit_min_max_compare_vs_libraries(oracle_mod, dt):
    """Min / max (NaN ignored: torch.fmin / fmax and NumPy fmin / fmax) and
    the six comparisons; equal zeros of opposite signs are checked by hand in
    the golden file, since the libraries do not fix which zero fmin returns."""
    a, b = _pairs16(dt, n_random=1 << 18)
    if dt == "f16":
        x, y = a.view(np.float16), b.view(np.float16)
    else:
        x, y = _tbf(a).float().numpy(), _tbf(b).float().numpy()   # exact
    zeros = ((a & 0x7FFF) == 0) & ((b & 0x7FFF) == 0)
    with np.errstate(all="ignore"):
        for op, fn in (("min", np.fmin), ("max", np.fmax)):
            got = _oracle16(oracle_mod, "%s_%s" % (op, dt), dt, a, b)
            ref = fn(x, y)
            ref = ref.view(np.uint16) if dt == "f16" else _nbf(torch.from_numpy(ref).to(torch.bfloat16))
            _same16(got[~zeros], ref[~zeros], dt, "%s %s" % (op, dt))
        for c, fn in (("eq", np.equal), ("ne", np.not_equal), ("lt", np.less), ("le", np.less_equal),
                      ("gt", np.greater), ("ge", np.greater_equal)):
            got = _oracle16(oracle_mod, "cmp_%s_%s" % (c, dt), dt, a, b)
            assert np.array_equal(got, fn(x, y).astype(np.int32)), (c, dt)


def test_bf16_conversions_vs_torch(oracle_mod):
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    # bfloat16 -> binary32: every pattern (exact)
    got = oracle_mod.from_spec(SPECS["cvt_bf16_f32"]).run(allb)[0].view(np.uint32)
    ref = _tbf(allb).float().numpy().view(np.uint32)
    nan = ((allb & 0x7F80) == 0x7F80) & ((allb & 0x7F) != 0)
    assert np.array_equal(got[~nan], ref[~nan]) and np.isnan(got[nan].view(np.float32)).all()
    # binary32 -> bfloat16: every bfloat16 value, each midpoint to the next one and the midpoint's
    # neighbours, plus random patterns
    v = allb.astype(np.uint32) << 16
    f = np.concatenate([v, v + 0x8000, v + 0x7FFF, v + 0x8001,
                        np.random.default_rng(5).integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)])
    got = oracle_mod.from_spec(SPECS["cvt_f32_bf16"]).run(f.view(np.float32))[0]
    ref = _nbf(torch.from_numpy(f.view(np.float32)).to(torch.bfloat16))
    _same16(got, ref, "bf16", "f32 -> bf16")
    # binary16 <-> bfloat16: every pattern (through the exact binary32 value in torch)
    got = oracle_mod.from_spec(SPECS["cvt_f16_bf16"]).run(allb.view(np.float16))[0]
    ref = _nbf(torch.from_numpy(allb.view(np.float16).astype(np.float32)).to(torch.bfloat16))
    _same16(got, ref, "bf16", "f16 -> bf16")
    got = oracle_mod.from_spec(SPECS["cvt_bf16_f16"]).run(allb)[0].view(np.uint16)
    ref = _tbf(allb).float().numpy().astype(np.float16).view(np.uint16)
    _same16(got, ref, "f16", "bf16 -> f16")
    # bfloat16 -> int32 equals the (pinned) binary32 -> int32 of the exact value
    got = oracle_mod.from_spec(SPECS["cvt_bf16_i32"]).run(allb)[0]
    ref = oracle_mod.from_spec(SPECS["cvt_f32_i32"]).run(_tbf(allb).float().numpy())[0]
    assert np.array_equal(got, ref)


def test_i32_to_bf16(oracle_mod):
    """Below 2^24 an int32 is exact in binary32, so torch's int -> binary32 ->
    bfloat16 is a single rounding; above it, each result is checked to be a
    nearest bfloat16 with an even fraction on ties, by exact integer
    arithmetic on its two neighbours (brute force per element)."""
    rng = np.random.default_rng(6)
    small = np.concatenate([np.arange(-70000, 70000, dtype=np.int32),
                            rng.integers(-(1 << 24), 1 << 24, 1 << 20, dtype=np.int64).astype(np.int32)])
    got = oracle_mod.from_spec(SPECS["cvt_i32_bf16"]).run(small)[0]
    ref = _nbf(torch.from_numpy(small.astype(np.float32)).to(torch.bfloat16))
    _same16(got, ref, "bf16", "small int32 -> bf16")
    big = rng.integers(-(1 << 31), 1 << 31, 20000, dtype=np.int64)
    big = big[np.abs(big) >= (1 << 24)]
    ties = np.array([(1 << 24) + (k << 16) for k in range(8)] + [(1 << 30) + (3 << 22), -(1 << 26) - (1 << 18)],
                    dtype=np.int64)
    big = np.concatenate([big, ties, ties + 1, ties - 1]).astype(np.int32)
    got = oracle_mod.from_spec(SPECS["cvt_i32_bf16"]).run(big)[0]
    vals = _tbf(got).double().numpy()
    for i, g, r in zip(big.tolist(), got.tolist(), vals.tolist()):
        m = abs(i)
        ulp = 1 << (m.bit_length() - 8)          # bfloat16 spacing in m's binade
        lo = (m // ulp) * ulp
        hi = lo + ulp
        if 2 * (m - lo) < ulp or (2 * (m - lo) == ulp and (lo // ulp) % 2 == 0):
            want = lo
        else:
            want = hi
        assert int(r) == (want if i > 0 else -want), (i, hex(g))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_16bit_invariants(oracle_mod, dt):
    """x*1 = x, x+(+0) = x (x != -0), x+y = y+x, x*y = y*x, x-y = x+Neg(y),
    Neg(Neg(x)) = x, x-x = +0 for finite x: bit for bit on every pattern
    (the second operands at random)."""
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    one = np.full_like(allb, 0x3C00 if dt == "f16" else 0x3F80)
    zero = np.zeros_like(allb)
    nan = _nan16(allb, dt)
    run = lambda name, *xs: _oracle16(oracle_mod, "%s_%s" % (name, dt), dt, *xs)
    _same16(run("mul", allb, one), allb, dt, "x*1")
    keep = allb != 0x8000
    _same16(run("add", allb, zero)[keep], allb[keep], dt, "x+0")
    y = np.random.default_rng(8).permutation(allb)
    _same16(run("add", allb, y), run("add", y, allb), dt, "x+y")
    _same16(run("mul", allb, y), run("mul", y, allb), dt, "x*y")
    neg_y = (y ^ 0x8000).astype(np.uint16)
    _same16(run("sub", allb, y), run("add", allb, neg_y), dt, "x-y")
    (nn,) = oracle_mod.from_spec([("x", ("load", dt, 1)), ("a", ("neg", "x")), ("b", ("neg", "a")),
                                   ("o", ("store", "b", 1))]).run(allb.view(np.float16) if dt == "f16" else allb)
    assert np.array_equal(nn.view(np.uint16), allb)
    inf = (allb & (0x7C00 if dt == "f16" else 0x7F80)) == (0x7C00 if dt == "f16" else 0x7F80)
    d = run("sub", allb, allb)
    assert np.all(d[~inf] == 0) and np.all(_nan16(d[inf], dt))


@pytest.mark.parametrize("wl", ["axpby_f16", "axpby_bf16"])
def test_16bit_axpby_workloads_vs_libraries(oracle_mod, wl):
    vals, _ = W.make_inputs(wl, 1 << 18)
    (o,) = oracle_mod.from_spec(W.WORKLOADS[wl]["spec"]).run(*vals, nthreads=8)
    if wl == "axpby_f16":
        x, y, al, be = vals
        ref = (al * x + be * y).view(np.uint16)
        _same16(o.view(np.uint16), ref, "f16", wl)
    else:
        x, y = _tbf(vals[0]), _tbf(vals[1])
        al, be = _tbf(np.array([vals[2]])), _tbf(np.array([vals[3]]))
        _same16(o, _nbf(al * x + be * y), "bf16", wl)
