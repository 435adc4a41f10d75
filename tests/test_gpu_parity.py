"""GPU parity: the HIP path against the oracle (and against the hand-worked
pins), element by element, on the same seeded inputs.

Bar: bit-exact for int32 and for binary32 (the library builds with FMA
contraction off); at most 2 ulp per element for the mixed binary16/binary32
Command (expected: 0, since x*y of two binary16 values is exact in binary32).
"""
import os

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import NPD, TD, bits, compare, dev, host, run_gpu, run_oracle, to_dev
from specs import SPECS, arg_dtypes, input_kinds
import test_oracle_pins as P
from random_commands import _random_inputs, _random_spec

pytestmark = pytest.mark.gpu

LINEAR = ["add_f32", "int_fused", "axpby_f32", "mixed_two_out"]
ULP = {"mixed_two_out": 2}


def _gpu_values(wl, vals, extra, n):
    return W.to_torch(vals, extra, dev())


def _check_workload(wl, n, generic=False):
    spec = W.WORKLOADS[wl]["spec"]
    vals, extra = W.make_inputs(wl, n)
    _, outs = arg_dtypes(spec)
    shape = W.shape_of(wl, n)
    if any(isinstance(v, np.ndarray) for v in vals):
        ref = run_oracle(spec, vals)
    else:                                  # no tensor input: the outputs give the shape
        ref = run_oracle(spec, vals, outputs=[np.zeros(shape, NPD[d]) for d in outs])
    gv = _gpu_values(wl, vals, extra, n)
    old = os.environ.get("ECMD_FORCE_GENERIC")
    if generic:
        os.environ["ECMD_FORCE_GENERIC"] = "1"
    try:
        cmd, got = run_gpu(spec, gv, [(shape, d) for d in outs])
        plan = cmd.plan(*gv, *got)
    finally:
        if generic:
            if old is None:
                del os.environ["ECMD_FORCE_GENERIC"]
            else:
                os.environ["ECMD_FORCE_GENERIC"] = old
    for k, (g, r) in enumerate(zip(got, ref)):
        compare(host(g), r, ULP.get(wl, 0), "%s n=%d out%d %s" % (wl, n, k, plan["kernel"]))
    return plan


# ---------------------------------------------------------------------------
# Hand-worked pins straight on the GPU (no oracle in between).

@pytest.mark.parametrize("n", [3, 8, 21])
def test_hand_worked_on_gpu(n):
    for ln, spec_name, ins, expect in P.GOLDEN_CASES:
        spec = SPECS[spec_name]
        in_dt, out_dt = arg_dtypes(spec)
        vals = []
        for kind, dt, b in zip(input_kinds(spec), in_dt, ins):
            if kind == "scalar":
                if dt == "bf16":
                    vals.append(np.uint16(b))
                else:
                    vals.append(float(np.array(b, dtype=P.NPU[dt]).view(NPD[dt])) if dt != "i32"
                                else int(np.array(b, dtype=np.uint32).view(np.int32)))
            else:
                vals.append(to_dev(np.full(n, b, dtype=P.NPU[dt]).view(NPD[dt])))
        _, got = run_gpu(spec, vals, [((n,), d) for d in out_dt])
        for o, e, dt in zip(got, expect, out_dt):
            ob = bits(host(o))
            for g in ob:
                if P.is_nan_bits(e, dt):
                    assert P.is_nan_bits(int(g), dt), "golden line %d: NaN expected, GPU %#x" % (ln, g)
                else:
                    assert int(g) == e, "golden line %d (%s): expected %#x, GPU %#x" % (ln, spec_name, e, g)


# ---------------------------------------------------------------------------
# The workloads: small sizes spanning several steps and ragged tails, then full size.

@pytest.mark.parametrize("wl", LINEAR)
@pytest.mark.parametrize("n", [1, 7, 8, 9, 255, 2048 * 8 + 5, 65536, (1 << 20) + 3,
                               256 * 2, 256 * 5 + 3, 256 * 31 + 17, 256 * 4099 + 255])
def test_linear_small(wl, n):
    """Small sizes through the ahead-of-time linear kernels: tails only, whole
    chunks only, and a last work-group whose spare wavefronts idle (chunk
    counts not a multiple of 4) beside the tail."""
    plan = _check_workload(wl, n)
    assert plan["path"] == "linear" and plan["specialised"]


@pytest.mark.parametrize("wl", ["axpby_f16", "axpby_bf16"])
@pytest.mark.parametrize("n", [511, 512 * 3, 512 * 5 + 3, 512 * 31 + 509, (1 << 20) + 7])
def test_linear_small_16bit(wl, n):
    """The same for the 16-bit kernels (chunks of 512 elements)."""
    plan = _check_workload(wl, n)
    assert plan["path"] == "linear" and plan["specialised"] and plan["elems_per_thread"] == 8, plan


@pytest.mark.parametrize("wl", LINEAR)
@pytest.mark.parametrize("shape", ["8x4", "8x8", "4x4", "8x4/ld0", "8x4/st0", "8x8/ld0st0", "4x4/ld0st0",
                                   "8x4/xcd", "8x4/cap", "4x4/stream", "8x8/stream", "4x4/occ"])
def test_linear_shapes(wl, shape):
    """Every linear kernel instantiation (group size, nontemporal loads and
    stores on or off, XCD renumbering, capped grid with a grid-stride loop,
    streaming stores forced below the size that selects them, occupancy
    bounded through LDS) against the oracle, at a size with several chunks and
    a ragged tail."""
    g, _, opt = shape.partition("/")
    env = {"ECMD_LINEAR_SHAPE": g, "ECMD_NT_LOAD": "0" if "ld0" in opt else "1",
           "ECMD_NT_STORE": "0" if "st0" in opt else "1"}
    if opt == "xcd":
        env["ECMD_XCD_REMAP"] = "1"
    if opt == "cap":
        env["ECMD_BLOCKS_PER_CU"] = "1"
    env["ECMD_STREAM_STORE"] = "1" if opt == "stream" else "0"
    if opt == "occ":
        env["ECMD_OCC_LDS"] = "24576"
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        n = 256 * 8 * 16 * 9 + 77 if opt == "xcd" else (1 << 19) + 333
        _check_workload(wl, n)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.mark.parametrize("wl", ["int_fused", "mixed_two_out", "axpby_f32", "add_f32", "axpby_f16"])
@pytest.mark.parametrize("order", ["0", "1", "2", "lean0"])
@pytest.mark.parametrize("n", [(1 << 19) + 333, 256 * 31 + 17])
def test_linear_load_orders(monkeypatch, wl, order, n):
    """The lean linear kernel compiled at run time with every order of the
    input loads (together, each input alone, the first alone) and the general
    kernel compiled at run time, against the oracle, at a size with several
    chunks and a ragged tail."""
    import elementwise_tensor_commands_amd as ecmd
    if order == "lean0":
        monkeypatch.setenv("ECMD_LINEAR_LEAN", "0")
    else:
        monkeypatch.setenv("ECMD_LINEAR_ORDER", order)
    spec = W.WORKLOADS[wl]["spec"]
    vals, extra = W.make_inputs(wl, n)
    ref = run_oracle(spec, vals)
    _, outs = arg_dtypes(spec)
    gv = W.to_torch(vals, extra, dev())
    got = [torch.empty(n, dtype=TD[d], device=dev()) for d in outs]
    cmd = ecmd.from_spec(spec).aot(False).jit(ecmd.JIT_SYNC)
    assert cmd.prepare(*gv, *got) in (0, 1, 2)
    plan = cmd.plan(*gv, *got)
    assert plan["path"] == "linear" and plan["kernel"] == "jit_linear", plan
    cmd.launch(*gv, *got)
    torch.cuda.synchronize()
    for k, (g, r) in enumerate(zip(got, ref)):
        compare(host(g), r, 0, "%s order %s n=%d out%d" % (wl, order, n, k))


@pytest.mark.parametrize("wl", LINEAR + ["transposed_2d"])
def test_generic_interpreter(wl):
    n = 257 if wl == "transposed_2d" else (1 << 18) + 5
    plan = _check_workload(wl, n, generic=True)
    assert not plan["specialised"]


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 200, 1000])
def test_transposed_small(n):
    plan = _check_workload("transposed_2d", n)
    # 1x1 is flat; the tiled path needs 16-byte rows: X's row stride n + 64 and
    # Y's n must be multiples of 4 elements, else the gather kernel runs.
    assert plan["path"] == ("linear" if n == 1 else "tiled" if n % 4 == 0 else "gather")


@pytest.mark.parametrize("tile", ["64x64", "128x64", "64x128", "128x128", "32x128", "32x256", "64x256",
                                  "128x128x512", "64x128x512", "64x256x512", "32x256x512", "32x512x512"])
@pytest.mark.parametrize("walk", ["1", "3", "8"])
def test_tiled_shapes(tile, walk):
    """Every specialised tiled instantiation and tile order against the oracle,
    on a square that is not a multiple of any tile (edge tiles in both
    directions) and on one that is."""
    env = {"ECMD_TILE": tile, "ECMD_TILE_WALK": walk}
    old = {k: os.environ.get(k) for k in env}
    os.environ.update(env)
    try:
        for n in (1000, 512):
            plan = _check_workload("transposed_2d", n)
            assert plan["kernel"] == "tiled_add_scaled_f32"
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v


@pytest.mark.parametrize("n", [64, 200, 1000])
def test_transposed_cached_policy(n):
    """The tiled kernels with ordinary (not nontemporal) global accesses."""
    old = os.environ.get("ECMD_TILED_NT")
    os.environ["ECMD_TILED_NT"] = "0"
    try:
        _check_workload("transposed_2d", n)
        _check_workload("transposed_2d", n + 4, generic=True)
    finally:
        if old is None:
            os.environ.pop("ECMD_TILED_NT", None)
        else:
            os.environ["ECMD_TILED_NT"] = old


@pytest.mark.parametrize("wl", ["add_f32", "int_fused", "axpby_f32", "mixed_two_out", "transposed_2d"])
def test_full_size(wl):
    """The configuration sizes, in the launch configuration the benchmark times,
    compared with the oracle on every element."""
    n = W.WORKLOADS[wl]["n"]
    print("  full size %s n=%d" % (wl, n), flush=True)
    plan = _check_workload(wl, n)
    assert plan["specialised"]


@pytest.mark.parametrize("wl", ["classify_u32", "fill_f32"])
@pytest.mark.parametrize("n", [1, 1027, (1 << 20) + 5, 1 << 28])
def test_widened_workloads(wl, n):
    """The compare and fill Commands, from a few elements to full size."""
    if n == 1 << 28:
        print("  full size %s" % wl, flush=True)
    plan = _check_workload(wl, n)
    assert plan["specialised"]


@pytest.mark.parametrize("dt", ["f32", "i32", "f16"])
def test_fill_generic_and_2d(dt):
    """Fills that the specialised kernel does not cover: int32 and binary16
    values (interpreter), and a rank-2 strided output (gather)."""
    import elementwise_tensor_commands_amd as ecmd
    val = {"f32": -0.0, "i32": -7, "f16": 65504.0}[dt]
    c = ecmd.Command()
    s_ = c.scalar(dt)
    c.store(s_, 2)
    out = torch.zeros((33, 70), dtype=TD[dt], device=dev())
    view = out[:, 3:67]
    c.launch(val, view)
    torch.cuda.synchronize()
    ref = np.zeros((33, 70), NPD[dt])
    ref[:, 3:67] = np.array(val, dtype=NPD[dt])
    compare(host(out), ref, 0, "fill %s" % dt)


# ---------------------------------------------------------------------------
# Edge cases.

def test_zero_length_launches_nothing():
    spec = W.ADD_F32
    x = torch.empty(0, device=dev())
    out = torch.empty(0, device=dev())
    run_gpu(spec, [x, x], None, outputs=[out])
    cmd = __import__("elementwise_tensor_commands_amd").from_spec(spec)
    assert cmd.plan(x, x, out)["path"] == "none"


@pytest.mark.parametrize("off", [1, 2, 3])
@pytest.mark.parametrize("n", [5, 1000, 65537])
def test_unaligned_bases_and_guards(off, n):
    """Views starting off a 16-byte boundary take the per-element variant; 4 KiB
    guard bands around the output must stay untouched."""
    rng = np.random.default_rng(off * 100 + n)
    xs = rng.random(n + off, dtype=np.float32)
    ys = rng.random(n + off, dtype=np.float32)
    guard = 1024
    buf = torch.full((n + 2 * guard + off,), 7.5, device=dev())
    out = buf[guard + off: guard + off + n]
    x, y = to_dev(xs)[off:], to_dev(ys)[off:]
    cmd, _ = run_gpu(W.ADD_F32, [x, y], None, outputs=[out])
    assert not cmd.plan(x, y, out)["vector"]
    compare(host(out), xs[off:] + ys[off:], 0, "unaligned add")
    b = host(buf)
    assert np.all(b[: guard + off] == 7.5) and np.all(b[guard + off + n:] == 7.5)


@pytest.mark.parametrize("n", [8 * 256 * 2048 + 13, 100])
def test_guards_vector_path(n):
    vals, _ = W.make_inputs("mixed_two_out", n)
    ref = run_oracle(W.MIXED_TWO_OUT, vals)
    guard = 2048
    b0 = torch.full((n + 2 * guard,), 1.0, dtype=torch.float16, device=dev())
    b1 = torch.full((n + 2 * guard,), 3.0, dtype=torch.float32, device=dev())
    outs = [b0[guard:guard + n], b1[guard:guard + n]]
    run_gpu(W.MIXED_TWO_OUT, [to_dev(v) if isinstance(v, np.ndarray) else v for v in vals], None, outputs=outs)
    compare(host(outs[0]), ref[0], 2, "out0")
    compare(host(outs[1]), ref[1], 2, "out1")
    h0, h1 = host(b0), host(b1)
    assert np.all(h0[:guard] == 1.0) and np.all(h0[guard + n:] == 1.0)
    assert np.all(h1[:guard] == 3.0) and np.all(h1[guard + n:] == 3.0)


def test_in_place_identical_view():
    n = 100003
    vals, _ = W.make_inputs("axpby_f32", n)
    ref = run_oracle(W.AXPBY_F32, vals)[0]
    x = to_dev(vals[0])
    run_gpu(W.AXPBY_F32, [x, to_dev(vals[1]), vals[2], vals[3]], None, outputs=[x])
    compare(host(x), ref, 0, "in place")


def test_non_default_stream():
    n = 1 << 20
    vals, _ = W.make_inputs("int_fused", n)
    ref = run_oracle(W.INT_FUSED, vals)[0]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gv = [to_dev(v) if isinstance(v, np.ndarray) else v for v in vals]
        out = torch.empty(n, dtype=torch.int32, device=dev())
    s.synchronize()
    run_gpu(W.INT_FUSED, gv, None, outputs=[out], stream=s)
    s.synchronize()
    compare(host(out), ref, 0, "side stream")


def test_bound_launch_repeated():
    """The marshal-once launcher, launched repeatedly on one stream."""
    n = (1 << 20) + 9
    vals, _ = W.make_inputs("mixed_two_out", n)
    ref = run_oracle(W.MIXED_TWO_OUT, vals)
    import elementwise_tensor_commands_amd as ecmd
    gv = [to_dev(v) if isinstance(v, np.ndarray) else v for v in vals]
    outs = [torch.empty(n, dtype=torch.float16, device=dev()), torch.empty(n, dtype=torch.float32, device=dev())]
    bound = ecmd.from_spec(W.MIXED_TWO_OUT).bind(*gv, *outs)
    for _ in range(5):
        bound.launch()
    torch.cuda.synchronize()
    compare(host(outs[0]), ref[0], 2, "bound out0")
    compare(host(outs[1]), ref[1], 2, "bound out1")


@pytest.mark.parametrize("wl", ["axpby_f32", "mixed_two_out", "axpby_f16"])
def test_staggered_operands(wl):
    """Operands cut by ecmd.empty_staggered from one allocation (starts 4 KiB
    apart modulo 32 KiB) through the linear kernels, against the oracle, at a
    size with a ragged tail; the bytes between the operands stay untouched."""
    import elementwise_tensor_commands_amd as ecmd
    n = (1 << 20) + 9
    spec = W.WORKLOADS[wl]["spec"]
    vals, _ = W.make_inputs(wl, n)
    ref = run_oracle(spec, vals)
    ins, outs = arg_dtypes(spec)
    specs = [((n,), TD[d]) for d, v in zip(ins, vals) if isinstance(v, np.ndarray)]
    specs += [((n,), TD[d]) for d in outs]
    placed = ecmd.empty_staggered(specs)
    storage = torch.empty(0, dtype=torch.uint8, device=dev()).set_(placed[0].untyped_storage())
    storage.fill_(0xA5)
    it = iter(placed)
    gv = []
    for v in vals:
        if isinstance(v, np.ndarray):
            t = next(it)
            t.copy_(to_dev(v))
            gv.append(t)
        else:
            gv.append(v)
    got = list(it)
    p0 = placed[0].data_ptr()
    assert [(t.data_ptr() - p0) % ecmd.STAGGER_PERIOD for t in placed] == [
        (4096 * k) % ecmd.STAGGER_PERIOD for k in range(len(placed))]
    plan = ecmd.from_spec(spec).plan(*gv, *got)
    assert plan["path"] == "linear" and plan["vector"], plan
    ecmd.from_spec(spec).launch(*gv, *got)
    torch.cuda.synchronize()
    for k, (g, r) in enumerate(zip(got, ref)):
        compare(host(g), r, 0, "%s staggered out%d" % (wl, k))
    # every byte outside the operands keeps the fill
    mask = torch.ones(storage.numel(), dtype=torch.bool, device=dev())
    s0 = storage.data_ptr()
    for t in placed:
        a = t.data_ptr() - s0
        mask[a:a + t.numel() * t.element_size()] = False
    assert bool((storage[mask] == 0xA5).all())


def test_rejected_launch_leaves_output():
    """Failed checks submit nothing: the output keeps its contents."""
    import elementwise_tensor_commands_amd as ecmd
    buf = torch.full((65,), 5.0, device=dev())
    x = torch.ones(64, device=dev())
    cmd = ecmd.from_spec(W.ADD_F32)
    with pytest.raises(ecmd.Error) as e:
        cmd.launch(x, torch.ones(65, device=dev()), buf[:64])
    assert e.value.name == "CMD_E_SHAPE"
    with pytest.raises(ecmd.Error) as e:
        cmd.launch(x, buf[:64], buf[1:65])      # output overlaps input y, shifted by one
    assert e.value.name == "CMD_E_ALIAS"
    with pytest.raises(ecmd.Error) as e:
        cmd.launch(x, torch.ones(64, dtype=torch.int32, device=dev()), buf[:64])
    assert e.value.name == "CMD_E_DTYPE"
    torch.cuda.synchronize()
    assert torch.all(buf == 5.0)


@pytest.mark.parametrize("shape", [(1, 1), (3, 5), (17, 33), (64, 64), (65, 63), (130, 70), (257, 129)])
@pytest.mark.parametrize("pad", [0, 1, 64])
def test_transposed_shapes(shape, pad):
    R, C = shape
    rng = np.random.default_rng(R * 7 + C + pad)
    xs = np.full((R, C + pad), np.nan, np.float32)
    xs[:, :C] = rng.random((R, C), dtype=np.float32) * 2 - 1
    Y = rng.random((C, R), dtype=np.float32) * 2 - 1
    ref = run_oracle(W.TRANSPOSED_2D, [xs[:, :C], Y.T, np.float32(2)])[0]
    X = to_dev(xs)[:, :C]
    Yt = to_dev(Y).t()
    cmd, (out,) = run_gpu(W.TRANSPOSED_2D, [X, Yt, 2.0], [((R, C), "f32")])
    compare(host(out), ref, 0, "transposed %s pad %d %s" % (shape, pad, cmd.plan(X, Yt, 2.0, out)["kernel"]))


def test_transposed_self_is_three_x_on_gpu():
    rng = np.random.default_rng(4)
    X = rng.random((320, 192), dtype=np.float32) * 2 - 1
    Xd = to_dev(X)
    Y = Xd.t().contiguous()
    _, (out,) = run_gpu(W.TRANSPOSED_2D, [Xd, Y.t(), 2.0], [((320, 192), "f32")])
    compare(host(out), np.float32(3) * X, 0, "X + 2 X")


@pytest.mark.parametrize("rteval", [False, True])
def test_tiled_generic_f16_two_staged(monkeypatch, rteval):
    """Rank 2: a binary16 and an int32 input read transposed (staged through
    LDS), a row-strided binary32 input, two outputs: the tiled path's
    interpreter, and the tiled kernel with RtEval (ECMD_TILED_RTEVAL=1)."""
    if rteval:
        monkeypatch.setenv("ECMD_TILED_RTEVAL", "1")
    spec = [("A", ("load", "f16", 2)), ("B", ("load", "f32", 2)), ("C", ("load", "i32", 2)),
            ("s", ("scalar", "f32")),
            ("af", ("cvt", "A", "f32")), ("p", ("mul", "af", "B")), ("q", ("sub", "p", "s")),
            ("ci", ("cvt", "C", "f32")), ("r", ("add", "q", "ci")), ("h", ("cvt", "r", "f16")),
            ("o0", ("store", "h", 2)), ("o1", ("store", "C", 2))]
    R, C = 300, 188
    rng = np.random.default_rng(12)
    A = (rng.random((C, R), dtype=np.float32) * 8 - 4).astype(np.float16)     # A.T: strides (1, R)
    Bs = rng.standard_normal((R, C + 4), dtype=np.float32)                      # row stride C + 4
    Cs = rng.integers(-1000, 1000, (C, R + 4), dtype=np.int32)                  # Cs[:, :R].T: strides (1, R + 4)
    vals = [A.T, Bs[:, :C], Cs[:, :R].T, np.float32(0.75)]
    ref = run_oracle(spec, vals)
    gv = [to_dev(A).t(), to_dev(Bs)[:, :C], to_dev(Cs)[:, :R].t(), 0.75]
    cmd, got = run_gpu(spec, gv, [((R, C), "f16"), ((R, C), "i32")])
    plan = cmd.plan(*gv, *got)
    assert plan["path"] == "tiled" and not plan["specialised"], plan
    assert (plan["lds_bytes"] == 2 * 64 * 64 * 4) == rteval, plan      # RtEval: two 64 x 64 staging tiles
    compare(host(got[0]), ref[0], 0, "tiled f16 out")
    compare(host(got[1]), ref[1], 0, "tiled i32 copy")


def test_gather_views():
    """Views no faster path takes: stride-0 broadcast, strided store,
    column-major output, both strides non-unit."""
    rng = np.random.default_rng(13)
    # broadcast a row vector over rows, store into every other column of a wider matrix
    R, C = 37, 45
    x = rng.random((R, C), dtype=np.float32)
    row = rng.random(C, dtype=np.float32)
    spec = [("x", ("load", "f32", 2)), ("b", ("load", "f32", 2)), ("r", ("sub", "x", "b")), ("o", ("store", "r", 2))]
    bview = np.lib.stride_tricks.as_strided(row, (R, C), (0, 4))
    wide = np.zeros((R, 2 * C), np.float32)
    run_oracle(spec, [x, bview], outputs=[wide[:, ::2]])
    rowd = to_dev(row)
    bd = rowd.as_strided((R, C), (0, 1))
    wided = torch.zeros((R, 2 * C), device=dev())
    cmd, _ = run_gpu(spec, [to_dev(x), bd], None, outputs=[wided[:, ::2]])
    assert cmd.plan(to_dev(x), bd, wided[:, ::2])["path"] == "gather"   # the store's inner stride is 2
    compare(host(wided), wide, 0, "broadcast row, strided store")
    # column-major output and a both-strided input -> gather
    xs = rng.random((2 * R, 3 * C), dtype=np.float32)
    xv = xs[::2, ::3]
    colmaj = np.zeros((C, R), np.float32)
    run_oracle(spec, [xv, bview], outputs=[colmaj.T])
    xd = to_dev(xs)[::2, ::3]
    cm = torch.zeros((C, R), device=dev())
    cmd, _ = run_gpu(spec, [xd, bd], None, outputs=[cm.t()])
    assert cmd.plan(xd, bd, cm.t())["path"] == "gather"
    compare(host(cm), colmaj, 0, "gather column-major out")
    # rank-1 strided load
    v = rng.random(3000, dtype=np.float32)
    spec1 = [("x", ("load", "f32", 1)), ("n", ("neg", "x")), ("o", ("store", "n", 1))]
    ref = run_oracle(spec1, [v[::3]])[0]
    cmd, (o,) = run_gpu(spec1, [to_dev(v)[::3]], [((1000,), "f32")])
    assert cmd.plan(to_dev(v)[::3], o)["path"] == "gather"
    compare(host(o), ref, 0, "rank-1 strided")


# ---------------------------------------------------------------------------
# Random Commands (generic interpreter coverage).

@pytest.mark.parametrize("seed", range(40))
def test_random_commands(seed):
    rng = np.random.default_rng(seed)
    rank = 2 if seed % 3 == 0 else 1
    spec = _random_spec(rng, int(rng.integers(1, 5)), int(rng.integers(1, 12)), rank)
    shape = (int(rng.integers(1, 90)), int(rng.integers(1, 90))) if rank == 2 else (int(rng.integers(1, 5000)),)
    vals = _random_inputs(rng, spec, shape)
    from oracle.oracle import OracleError
    import elementwise_tensor_commands_amd as ecmd
    gv = [to_dev(v) if isinstance(v, np.ndarray) else
          (v if v.dtype == np.uint16 else float(v) if v.dtype.kind == "f" else int(v)) for v in vals]
    if rank == 2 and seed % 2 == 0:       # transposed views of the loads
        gv = [v.t().contiguous().t() if isinstance(v, torch.Tensor) else v for v in gv]
    _, outs = arg_dtypes(spec)
    try:
        ref = run_oracle(spec, vals)
    except OracleError as e:   # the oracle refuses the Command: the library must refuse it too
        with pytest.raises(ecmd.Error) as le:
            run_gpu(spec, gv, [(shape, d) for d in outs])
        assert le.value.name != "CMD_E_LAUNCH", le.value
        return
    try:
        cmd, got = run_gpu(spec, gv, [(shape, d) for d in outs])
    except ecmd.Error as e:
        assert e.name == "CMD_E_LIMIT", e          # more live temporaries than registers
        pytest.skip(str(e))
    for k, (g, r) in enumerate(zip(got, ref)):
        compare(host(g), r, 0, "random seed %d out%d %s\n%s" % (seed, k, cmd.plan(*gv, *got)["kernel"], cmd.dump()))


# ---------------------------------------------------------------------------
# Conversions, exhaustively.

def test_f16_to_f32_all_patterns_gpu():
    from oracle import oracle
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    _, (o,) = run_gpu(SPECS["cvt_f16_f32"], [to_dev(h.view(np.float16))], [((65536,), "f32")])
    compare(host(o), oracle.f16_to_f32_all().view(np.float32), 0, "f16->f32")


def test_f32_to_f16_all_2pow32_gpu():
    """Every binary32 bit pattern through the GPU's conversion, 16 launches of
    2^28, each compared with the oracle."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import oracle
    chunk = 1 << 28
    base = torch.arange(chunk, dtype=torch.int64, device=dev())
    out = torch.empty(chunk, dtype=torch.float16, device=dev())
    sub = 1 << 24
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for k in range(16):
            first = k * chunk
            v = base + first
            x = torch.where(v >= 2**31, v - 2**32, v).to(torch.int32).view(torch.float32)
            run_gpu(SPECS["cvt_f32_f16"], [x], None, outputs=[out])
            got = host(out.view(torch.int16)).view(np.uint16)
            ref = np.concatenate(list(ex.map(lambda j: oracle.f32_to_f16_range(first + j * sub, sub), range(chunk // sub))))
            nan_r = ((ref & 0x7C00) == 0x7C00) & ((ref & 0x3FF) != 0)
            nan_g = ((got & 0x7C00) == 0x7C00) & ((got & 0x3FF) != 0)
            assert np.array_equal(nan_r, nan_g), "chunk %d NaN positions" % k
            bad = np.flatnonzero(got[~nan_r] != ref[~nan_r])
            assert bad.size == 0, "chunk %d: %d mismatches" % (k, bad.size)
            print("  f32->f16 chunk %d/16 ok" % (k + 1), flush=True)
