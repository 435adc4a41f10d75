"""The oracle on every pair of binary32 / int32 edge values (and 2^20 random
pairs), against NumPy's and torch's own arithmetic: IEEE binary32 add, sub
and mul rounded to nearest even with subnormals kept, fmin / fmax (NaN
ignored), the comparisons, int32 arithmetic modulo 2^32 and unsigned
comparisons, sign operations, select and the conversions.  These are the
same inputs the GPU sweep uses, so the oracle the GPU is compared with is
pinned on exactly those values."""
import numpy as np
import pytest
import torch

from edge_values import conditions, pairs32
from specs import SPECS

N_RANDOM = 1 << 18


def _f(bits):
    return bits.view(np.float32)


def _i(bits):
    return bits.view(np.int32)


def _run(oracle_mod, name, *vals):
    return oracle_mod.from_spec(SPECS[name]).run(*vals, nthreads=8)[0]


def _same(got, ref, what):
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.dtype == ref.dtype, (got.dtype, ref.dtype)
    if got.dtype.kind == "f":
        ng, nr = np.isnan(got), np.isnan(ref)
        assert np.array_equal(ng, nr), "%s: NaN positions differ" % what
        ut = {2: np.uint16, 4: np.uint32}[got.itemsize]
        gb, rb = got.view(ut)[~ng], ref.view(ut)[~nr]
    else:
        gb, rb = got, ref
    bad = np.flatnonzero(gb != rb)
    assert bad.size == 0, "%s: %d differ, first at %s" % (what, bad.size, bad[:5])


@pytest.mark.parametrize("op", ["add", "sub", "mul"])
def test_f32_arith_pairs(oracle_mod, op):
    a, b = pairs32("f32", N_RANDOM)
    x, y = _f(a), _f(b)
    with np.errstate(all="ignore"):
        ref = {"add": x + y, "sub": x - y, "mul": x * y}[op]
    _same(_run(oracle_mod, "%s_f32" % op, x, y), ref, op)


def test_f32_min_max_pairs(oracle_mod):
    """minimumNumber / maximumNumber: NumPy's fmin / fmax, except that for two
    zeros NumPy does not fix which one is returned; there min is -0 unless
    both are +0, and max is +0 unless both are -0."""
    a, b = pairs32("f32", N_RANDOM)
    x, y = _f(a), _f(b)
    zz = (x == 0) & (y == 0)
    for op, lib in (("min", np.fmin), ("max", np.fmax)):
        got = _run(oracle_mod, "%s_f32" % op, x, y)
        _same(got[~zz], lib(x, y)[~zz], op)
        neg = np.signbit(got[zz])
        want = (np.signbit(x[zz]) | np.signbit(y[zz])) if op == "min" else (np.signbit(x[zz]) & np.signbit(y[zz]))
        assert np.array_equal(neg, want), "%s of two zeros" % op


@pytest.mark.parametrize("dt", ["f32", "i32"])
def test_compare_pairs(oracle_mod, dt):
    a, b = pairs32(dt, N_RANDOM)
    x, y = (_f(a), _f(b)) if dt == "f32" else (_i(a), _i(b))
    with np.errstate(all="ignore"):
        for c, fn in (("eq", np.equal), ("ne", np.not_equal), ("lt", np.less), ("le", np.less_equal),
                      ("gt", np.greater), ("ge", np.greater_equal)):
            _same(_run(oracle_mod, "cmp_%s_%s" % (c, dt), x, y), fn(x, y).astype(np.int32), "cmp %s %s" % (c, dt))
    if dt == "i32":
        for c, fn in (("ltu", np.less), ("leu", np.less_equal), ("gtu", np.greater), ("geu", np.greater_equal)):
            _same(_run(oracle_mod, "cmp_%s_i32" % c, x, y), fn(a, b).astype(np.int32), "cmp %s" % c)


def test_i32_arith_pairs(oracle_mod):
    a, b = pairs32("i32", N_RANDOM)
    x, y = _i(a), _i(b)
    m = np.uint64(0xFFFFFFFF)
    a64, b64 = a.astype(np.uint64), b.astype(np.uint64)
    for op, ref in (("add", (a64 + b64) & m), ("sub", (a64 - b64) & m), ("mul", (a64 * b64) & m)):
        _same(_run(oracle_mod, "%s_i32" % op, x, y), ref.astype(np.uint32).view(np.int32), op)
    _same(_run(oracle_mod, "min_i32", x, y), np.minimum(x, y), "min i32")
    _same(_run(oracle_mod, "max_i32", x, y), np.maximum(x, y), "max i32")


def test_sign_ops_and_select(oracle_mod):
    a, b = pairs32("f32", N_RANDOM)
    x, y = _f(a), _f(b)
    # neg flips the sign bit, abs clears it, NaNs included
    _same(_run(oracle_mod, "neg_f32", x).view(np.uint32), a ^ np.uint32(0x80000000), "neg f32")
    _same(_run(oracle_mod, "abs_f32", x).view(np.uint32), a & np.uint32(0x7FFFFFFF), "abs f32")
    ia, ib = pairs32("i32", N_RANDOM)
    xi = _i(ia)
    _same(_run(oracle_mod, "neg_i32", xi), ((np.uint64(1 << 32) - ia.astype(np.uint64)) & np.uint64(0xFFFFFFFF))
          .astype(np.uint32).view(np.int32), "neg i32")
    with np.errstate(all="ignore"):
        _same(_run(oracle_mod, "abs_i32", xi), np.abs(xi), "abs i32")      # |INT_MIN| wraps to INT_MIN
    c = _i(conditions(a.size))
    _same(_run(oracle_mod, "select_f32", c, x, y).view(np.uint32), np.where(c != 0, a, b), "select f32")
    _same(_run(oracle_mod, "select_i32", _i(conditions(ia.size)), xi, _i(ib)),
          np.where(_i(conditions(ia.size)) != 0, xi, _i(ib)), "select i32")


def test_conversions_of_edge_values(oracle_mod):
    a, _ = pairs32("f32", N_RANDOM)
    x = _f(np.unique(a))
    with np.errstate(all="ignore"):
        # binary32 -> int32: truncate toward zero, saturate, NaN -> 0
        t = np.trunc(x.astype(np.float64))
        ref = np.where(np.isnan(t), 0, np.clip(np.nan_to_num(t, nan=0.0), -2.0**31, 2.0**31 - 1)).astype(np.int32)
        _same(_run(oracle_mod, "cvt_f32_i32", x), ref, "f32 -> i32")
        _same(_run(oracle_mod, "cvt_f32_f16", x), x.astype(np.float16), "f32 -> f16")
    bf = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = _run(oracle_mod, "cvt_f32_bf16", x).view(np.uint16)
    nan = lambda b: ((b & 0x7F80) == 0x7F80) & ((b & 0x7F) != 0)
    assert np.array_equal(nan(got), nan(bf)), "f32 -> bf16: NaN positions differ"
    _same(got[~nan(got)], bf[~nan(bf)], "f32 -> bf16")
    ia, _ = pairs32("i32", N_RANDOM)
    xi = _i(np.unique(ia))
    _same(_run(oracle_mod, "cvt_i32_f32", xi), xi.astype(np.float32), "i32 -> f32")
    # int32 -> binary16 rounds the exact value once: binary64 holds it exactly
    _same(_run(oracle_mod, "cvt_i32_f16", xi), xi.astype(np.float64).astype(np.float16), "i32 -> f16")
