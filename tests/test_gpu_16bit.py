"""Native binary16 / bfloat16 arithmetic and bfloat16 conversions on the GPU,
compared with the oracle bit for bit (any NaN equals any NaN).

The oracle rounds each exact result once to the 16-bit format; the GPU adds
and multiplies binary16 with the packed 16-bit instructions and bfloat16
through binary32, then converts with gfx950's binary32 -> bfloat16
instruction."""
import os

import numpy as np
import pytest
import torch

import test_oracle_pins as P
import workloads as W
from gpu_util import compare, dev, host, run_gpu, run_oracle, to_dev
from specs import SPECS

pytestmark = pytest.mark.gpu


def _dev16(bits, dt):
    return to_dev(bits.view(np.float16) if dt == "f16" else bits)


def _run_pair(spec_name, dt, a, b, out_dt):
    ref = run_oracle(SPECS[spec_name], [a.view(np.float16) if dt == "f16" else a,
                                         b.view(np.float16) if dt == "f16" else b])[0]
    _, (o,) = run_gpu(SPECS[spec_name], [_dev16(a, dt), _dev16(b, dt)], [((a.size,), out_dt)])
    return host(o), ref


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("op", ["add", "sub", "mul"])
def test_16bit_arith_pairs(op, dt):
    """Every pair of edge values (zeros, subnormals, largest finite,
    infinities, NaN, each exponent with edge fractions) and 2^20 random pairs."""
    a, b = P._pairs16(dt)
    got, ref = _run_pair("%s_%s" % (op, dt), dt, a, b, dt)
    compare(got, ref, 0, "%s %s" % (op, dt))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_16bit_min_max_compare(dt):
    a, b = P._pairs16(dt, n_random=1 << 18)
    for op in ("min", "max"):
        got, ref = _run_pair("%s_%s" % (op, dt), dt, a, b, dt)
        compare(got, ref, 0, "%s %s" % (op, dt))
    for c in ("eq", "ne", "lt", "le", "gt", "ge"):
        got, ref = _run_pair("cmp_%s_%s" % (c, dt), dt, a, b, "i32")
        compare(got, ref, 0, "cmp %s %s" % (c, dt))


def _run_unary(spec_name, x, out_dt):
    ref = run_oracle(SPECS[spec_name], [x])[0]
    _, (o,) = run_gpu(SPECS[spec_name], [to_dev(x)], [((x.size,), out_dt)])
    return host(o), ref


def test_conversions_from_every_16bit_pattern():
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    for name, src, out_dt in (("cvt_bf16_f32", allb, "f32"), ("cvt_bf16_f16", allb, "f16"),
                              ("cvt_bf16_i32", allb, "i32"), ("cvt_f16_bf16", allb.view(np.float16), "bf16"),
                              ("neg_bf16", allb, "bf16"), ("abs_bf16", allb, "bf16")):
        got, ref = _run_unary(name, src, out_dt)
        compare(got, ref, 0, name)


def test_int32_to_bf16():
    rng = np.random.default_rng(12)
    ties = np.array([(1 << 24) + (k << 16) + d for k in range(16) for d in (-1, 0, 1)] +
                    [-(1 << 31), (1 << 31) - 1, 0, 1, -1, (1 << 30) + (3 << 22)], dtype=np.int64)
    x = np.concatenate([rng.integers(-(1 << 31), 1 << 31, 1 << 22, dtype=np.int64),
                        rng.integers(-(1 << 25), 1 << 25, 1 << 20, dtype=np.int64), ties]).astype(np.int32)
    got, ref = _run_unary("cvt_i32_bf16", x, "bf16")
    compare(got, ref, 0, "i32 -> bf16")


def test_f32_to_bf16_all_2pow32():
    """Every binary32 bit pattern through the GPU's conversion, 16 launches of
    2^28, each compared with the oracle."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle
    chunk = 1 << 28
    base = torch.arange(chunk, dtype=torch.int64, device=dev())
    out = torch.empty(chunk, dtype=torch.bfloat16, device=dev())
    sub = 1 << 24
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for k in range(16):
            first = k * chunk
            v = base + first
            x = torch.where(v >= 2**31, v - 2**32, v).to(torch.int32).view(torch.float32)
            run_gpu(SPECS["cvt_f32_bf16"], [x], None, outputs=[out])
            got = host(out)
            ref = np.concatenate(list(ex.map(lambda j: oracle.f32_to_bf16_range(first + j * sub, sub),
                                             range(chunk // sub))))
            compare(got, ref, 0, "f32 -> bf16 chunk %d" % k)
            print("  f32->bf16 chunk %d/16 ok" % (k + 1), flush=True)


@pytest.mark.parametrize("wl", ["axpby_f16", "axpby_bf16"])
@pytest.mark.parametrize("n", [1, 7, 1027, (1 << 20) + 3, 1 << 28])
def test_16bit_axpby_workloads(wl, n):
    """The two 16-bit workloads from a few elements to the full size the
    benchmark times, every element compared."""
    if n == 1 << 28:
        print("  full size %s" % wl, flush=True)
    spec = W.WORKLOADS[wl]["spec"]
    vals, extra = W.make_inputs(wl, n)
    ref = run_oracle(spec, vals)
    gv = W.to_torch(vals, extra, dev())
    dt = "f16" if wl == "axpby_f16" else "bf16"
    cmd, (o,) = run_gpu(spec, gv, [((n,), dt)])
    plan = cmd.plan(*gv, o)
    compare(host(o), ref[0], 0, "%s n=%d %s" % (wl, n, plan["kernel"]))
    assert plan["specialised"] and plan["kernel"] == "linear_" + wl


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_16bit_generic_and_strided(dt):
    """The interpreter and the gather path on 16-bit arithmetic: a 2-D
    transposed load through the tiled kernel and a strided one through the
    gather kernel."""
    rng = np.random.default_rng(3)
    R, C = 132, 264
    spec = [("x", ("load", dt, 2)), ("y", ("load", dt, 2)), ("s", ("scalar", dt)), ("p", ("mul", "x", "y")),
            ("q", ("sub", "p", "s")), ("m", ("min", "q", "x")), ("o", ("store", "m", 2))]
    raw = lambda shape: (rng.standard_normal(shape).astype(np.float32) * 3)
    if dt == "f16":
        x, ys = raw((R, C)).astype(np.float16), raw((C, R)).astype(np.float16)
        s = np.float16(0.375)
    else:
        x = (raw((R, C)).view(np.uint32) >> 16).astype(np.uint16)
        ys = (raw((C, R)).view(np.uint32) >> 16).astype(np.uint16)
        s = np.uint16(0x3EC0)                  # 0.375
    ref = run_oracle(spec, [x, ys.T, s])[0]
    xd, yd = to_dev(x), to_dev(ys)
    cmd, (o,) = run_gpu(spec, [xd, yd.t(), s], [((R, C), dt)])
    assert cmd.plan(xd, yd.t(), s, o)["path"] == "tiled"
    compare(host(o), ref, 0, "%s tiled" % dt)
    # every other column: no unit stride -> gather
    x2 = np.ascontiguousarray(np.repeat(x, 2, axis=1))
    ref2 = run_oracle(spec, [x2[:, ::2], ys.T, s])[0]
    x2d = to_dev(x2)[:, ::2]
    cmd, (o2,) = run_gpu(spec, [x2d, yd.t(), s], [((R, C), dt)])
    assert cmd.plan(x2d, yd.t(), s, o2)["path"] == "gather"
    compare(host(o2), ref2, 0, "%s gather" % dt)
