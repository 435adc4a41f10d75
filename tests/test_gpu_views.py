"""Rank-1 to rank-4 views on the GPU, compared with the oracle.

Every case cuts its views from contiguous storages (permuted, padded, offset
and, for loads, broadcast with stride 0), runs the Command on the GPU over
device copies of the storages and in the oracle over host copies, and compares
the whole output storages bit for bit: the elements a store view covers must
match and every other element must be left as it was."""
import os

import numpy as np
import pytest
import torch
from numpy.lib.stride_tricks import as_strided

import workloads as W
from gpu_util import NPD, compare, dev, host, run_oracle, to_dev
from random_commands import random_view_case
from specs import arg_dtypes

pytestmark = pytest.mark.gpu


def _recut(view, storage, copy):
    """The view of ``storage`` rebuilt over ``copy`` (same offset and strides)."""
    off, strides = W.layout(view, storage)
    isz = copy.itemsize
    return as_strided(copy.reshape(-1)[off:], shape=view.shape, strides=tuple(s * isz for s in strides))


def _device(view, storage):
    off, strides = W.layout(view, storage)
    flat = to_dev(np.ascontiguousarray(storage).reshape(-1))
    return flat, flat.as_strided(view.shape, strides, off)


def run_views(spec, inputs, outputs, generic=False, what="", jit=False):
    """inputs: (view, storage) pairs for loads, plain values for scalars, in
    declaration order; outputs: (view, storage) pairs in store order; jit: a
    kernel compiled at run time where no ahead-of-time one fits.
    Returns the plan the GPU launch used."""
    import elementwise_tensor_commands_amd as ecmd
    host_out = [st.copy() for _, st in outputs]
    ref_views = [_recut(v, st, c) for (v, st), c in zip(outputs, host_out)]
    vals = [x[0] if isinstance(x, tuple) else x for x in inputs]
    run_oracle(spec, vals, outputs=ref_views)
    gin = [(_device(*x)[1] if isinstance(x, tuple) else x) for x in inputs]
    gflat, gout = [], []
    for v, st in outputs:
        f, g = _device(v, st)
        gflat.append(f)
        gout.append(g)
    cmd = ecmd.from_spec(spec)
    if jit:
        cmd.jit(ecmd.JIT_SYNC)
    old = os.environ.get("ECMD_FORCE_GENERIC")
    if generic:
        os.environ["ECMD_FORCE_GENERIC"] = "1"
    try:
        plan = cmd.plan(*gin, *gout)
        print("    %s: %s dims=%d size=%s" % (what, plan["kernel"], plan["dims"], plan["size"]), flush=True)
        cmd.launch(*gin, *gout)
        torch.cuda.synchronize()
    finally:
        if generic:
            if old is None:
                del os.environ["ECMD_FORCE_GENERIC"]
            else:
                os.environ["ECMD_FORCE_GENERIC"] = old
    for k, (f, ref) in enumerate(zip(gflat, host_out)):
        compare(host(f), ref.reshape(-1), 0, "%s out%d (%s)" % (what, k, plan["kernel"]))
    return plan


def _workload_case(wl, shape):
    spec = W.WORKLOADS[wl]["spec"]
    vals, extra = W.make_inputs(wl, shape=shape)
    ins = [(v, st) if st is not None else v for v, st in zip(vals, extra["storage"])]
    _, outs = arg_dtypes(spec)
    rng = np.random.default_rng(7)
    out_pairs = []
    for d in outs:
        st = rng.integers(0, 2**32, shape, dtype=np.uint64).astype(np.uint32).view(np.float32).astype(NPD[d])
        out_pairs.append((st, st))
    return spec, ins, out_pairs


@pytest.mark.parametrize("generic", [False, True])
@pytest.mark.parametrize("wl,shape", [
    ("batched_transpose", (3, 200, 300)), ("batched_transpose", (2, 64, 64)), ("batched_transpose", (5, 33, 517)),
    ("batched_transpose", (1, 1, 1)), ("batched_transpose", (4, 1, 260)), ("batched_transpose", (7, 260, 4)),
    ("bias_nchw", (3, 37, 5, 67)), ("bias_nchw", (2, 8, 1, 1)), ("bias_nchw", (1, 1, 1, 1)),
    ("bias_nchw", (2, 3, 16, 16)), ("bias_nchw", (2, 70, 9, 12)),
    ("bias_nchw_f16", (2, 8, 4, 16)), ("bias_nchw_f16", (3, 37, 5, 24)), ("bias_nchw_f16", (2, 70, 9, 12))])
def test_workload_shapes(wl, shape, generic):
    spec, ins, outs = _workload_case(wl, shape)
    plan = run_views(spec, ins, outs, generic, "%s %s" % (wl, shape))
    if generic:
        assert not plan["specialised"]


@pytest.mark.parametrize("tile", ["64x64", "32x256x512", "128x128", "64x128x512"])
def test_batched_transpose_tiles(tile):
    """Every instantiated tile of the specialised kernel over several planes
    with ragged edges."""
    old = os.environ.get("ECMD_TILE")
    os.environ["ECMD_TILE"] = tile
    try:
        spec, ins, outs = _workload_case("batched_transpose", (3, 196, 516))
        plan = run_views(spec, ins, outs, False, "tile %s" % tile)
    finally:
        if old is None:
            del os.environ["ECMD_TILE"]
        else:
            os.environ["ECMD_TILE"] = old
    assert plan["specialised"] and plan["path"] == "tiled"


@pytest.mark.parametrize("wl", ["batched_transpose", "bias_nchw", "bias_nchw_f16", "transposed_2d_f16", "odd_rows_f32",
                                "narrow_rows_f32"])
def test_full_size_views(wl):
    """The full shapes the benchmark times, in its launch configuration
    (the binary16 workloads: compiled at run time), compared with the oracle
    on every element."""
    shape = W.shape_of(wl)
    print("  full size %s %s" % (wl, shape), flush=True)
    spec = W.WORKLOADS[wl]["spec"]
    vals, extra = W.make_inputs(wl)
    ref = run_oracle(spec, vals)
    gin = W.to_torch(vals, extra, dev())
    import elementwise_tensor_commands_amd as ecmd
    cmd = ecmd.from_spec(spec)
    if wl.endswith("_f16"):
        cmd.jit(ecmd.JIT_SYNC)
    out = torch.empty(shape, dtype=torch.float16 if wl.endswith("f16") else torch.float32, device=dev())
    plan = cmd.plan(*gin, out)
    cmd.launch(*gin, out)
    torch.cuda.synchronize()
    compare(host(out), ref[0], 0, "%s full (%s)" % (wl, plan["kernel"]))
    assert (plan["path"], plan["kernel"]) == {
        "batched_transpose": ("tiled", "tiled_add_scaled_f32"), "bias_nchw": ("rows", "rows_affine_f32"),
        "bias_nchw_f16": ("rows", "jit_rows"), "transposed_2d_f16": ("tiled", "jit_tiled"),
        "odd_rows_f32": ("gather", "gather_segments"), "narrow_rows_f32": ("gather", "gather_whole_rows")}[wl]
    if wl.endswith("_f16"):
        assert plan["elems_per_thread"] == 8, plan


def test_staged_direct_and_row_constant_together():
    """One Command with a direct binary16 input, a staged (transposed) fp32
    input and a row-constant int32 input over a batch of planes."""
    B, R, C = 3, 132, 260
    rng = np.random.default_rng(31)
    x = rng.standard_normal((B, R, C)).astype(np.float16)
    y = rng.standard_normal((B, C, R)).astype(np.float32) * 100
    k = rng.integers(-50, 50, (B, R), dtype=np.int32)
    kv = as_strided(k, shape=(B, R, C), strides=(k.strides[0], k.strides[1], 0), writeable=False)
    spec = [("x", ("load", "f16", 3)), ("y", ("load", "f32", 3)), ("k", ("load", "i32", 3)),
            ("xf", ("cvt", "x", "f32")), ("kf", ("cvt", "k", "f32")), ("p", ("mul", "xf", "y")),
            ("q", ("add", "p", "kf")), ("h", ("cvt", "q", "f16")), ("kk", ("mul", "k", "k")),
            ("o0", ("store", "h", 3)), ("o1", ("store", "kk", 3))]
    o0 = np.zeros((B, R, C), np.float16)
    o1 = np.zeros((B, R, C), np.int32)
    plan = run_views(spec, [(x, x), (y.transpose(0, 2, 1), y), (kv, k)], [(o0, o0), (o1, o1)], False, "mixed")
    assert plan["path"] == "tiled" and plan["lds_bytes"] > 0


def test_empty_rank4_leaves_outputs_alone():
    spec, ins, outs = _workload_case("bias_nchw", (3, 0, 5, 7))
    run_views(spec, ins, outs, False, "empty")


@pytest.mark.parametrize("seed", range(80))
def test_random_views(seed):
    spec, ins, outs = random_view_case(seed)
    run_views(spec, ins, outs, False, "seed %d" % seed)
    if seed % 4 == 0:
        spec, ins, outs = random_view_case(seed)
        run_views(spec, ins, outs, True, "seed %d generic" % seed)


@pytest.mark.parametrize("seed", range(30))
def test_random_transposed_views(seed):
    """Random Commands whose inputs are stored in other dimension orders than
    the outputs (mostly the tiled path's staged inputs)."""
    spec, ins, outs = random_view_case(seed, staged=True)
    run_views(spec, ins, outs, False, "staged seed %d" % seed)


@pytest.mark.parametrize("shape", [(3, 5, 1), (3, 5, 2), (3, 5, 3), (3, 5, 5), (2, 3, 7, 63), (2, 3, 7, 64),
                                   (2, 3, 7, 65), (4, 129), (1, 70001, 8), (3, 1, (1 << 20) + 3), (7, 1, 9, 4),
                                   (5, 3, 1, 260), (1,), (6,), (1 << 20,)])
def test_rows_path_shapes(shape):
    """The rows path: padded rows, a per-row broadcast and a broadcast along
    the rows, for row lengths with and without a partial last vector and row
    counts that exercise the constant divisions."""
    rng = np.random.default_rng(sum(shape) + len(shape))
    spec = [("x", ("load", "f32", len(shape))), ("s", ("load", "f32", len(shape))),
            ("b", ("load", "f32", len(shape))), ("xs", ("mul", "x", "s")), ("o", ("add", "b", "xs")),
            ("out", ("store", "o", len(shape)))]
    last = shape[-1]
    pitch = last + (-last) % 4 + 4
    lead = shape[:-1]

    def padded():
        st = rng.standard_normal(lead + (pitch,)).astype(np.float32)
        return st[..., :last], st

    x, xs = padded()
    srow = rng.standard_normal(lead if lead else (1,)).astype(np.float32)
    s = as_strided(srow, shape=shape, strides=(srow.strides if lead else ()) + (0,), writeable=False)
    bcol = rng.standard_normal(last).astype(np.float32)
    b = as_strided(bcol, shape=shape, strides=(0,) * len(lead) + (4,), writeable=False)
    o, os_ = padded()
    plan = run_views(spec, [(x, xs), (s, srow), (b, bcol)], [(o, os_)], False, "rows %s" % (shape,))
    if np.prod(shape) == 1:
        assert plan["path"] == "linear", plan
    elif last > 1:                     # rows of one element are a strided vector: gathered
        assert plan["path"] == "rows", plan


AXPBY16 = {dt: [("x", ("load", dt, 3)), ("y", ("load", dt, 3)), ("a", ("scalar", dt)), ("b", ("scalar", dt)),
                ("ax", ("mul", "a", "x")), ("by", ("mul", "b", "y")), ("s", ("add", "ax", "by")),
                ("o", ("store", "s", 3))] for dt in ("f16", "bf16")}


@pytest.mark.parametrize("which", ["f16", "bf16", "jit"])
@pytest.mark.parametrize("n3,stride", [(8, 8), (64, 72), (67, 72), (1000, 1008), (1003, 1016), (4101, 4104),
                                       (64, 68), (1001, 1004)])
def test_rows_16bit_vectors(which, n3, stride):
    """Programs whose operands are all 16-bit take 16-byte vectors of 8
    elements on the rows path when every row starts on 16 bytes (row stride a
    multiple of 8), else 8-byte vectors of 4: the binary16 / bfloat16 axpby
    (ahead-of-time kernels) and a per-row affine map compiled at run time, over
    padded rows, a partial last vector and a batch of planes; the padding of
    the output rows must stay untouched."""
    B, R = 3, 37
    rng = np.random.default_rng(n3 + stride + len(which))
    dt = "f16" if which == "jit" else which

    def draw(shape):
        f = (rng.standard_normal(shape) * 8).astype(np.float32)
        return (f.view(np.uint32) >> 16).astype(np.uint16) if dt == "bf16" else f.astype(np.float16)

    xs, ys = draw((B, R, stride)), draw((B, R + 1, stride))
    os_ = draw((B, R, stride))
    x, y, o = xs[:, :, :n3], ys[:, 1:, :n3], os_[:, :, :n3]
    if which == "jit":
        cs = draw((B, R, 1))
        c = as_strided(cs, shape=(B, R, n3), strides=(cs.strides[0], cs.strides[1], 0), writeable=False)
        spec = [("x", ("load", "f16", 3)), ("y", ("load", "f16", 3)), ("c", ("load", "f16", 3)),
                ("p", ("mul", "x", "c")), ("q", ("sub", "p", "y")), ("m", ("max", "q", "x")), ("o", ("store", "m", 3))]
        ins = [(x, xs), (y, ys), (c, cs)]
    else:
        spec = AXPBY16[dt]
        a, b = (np.float16(1.5), np.float16(-0.25)) if dt == "f16" else (np.uint16(0x3FC0), np.uint16(0xBE80))
        ins = [(x, xs), (y, ys), a, b]
    plan = run_views(spec, ins, [(o, os_)], False, "rows16 %s %d/%d" % (which, n3, stride), jit=which == "jit")
    assert plan["path"] == "rows" and plan["elems_per_thread"] == (8 if stride % 8 == 0 else 4), plan
    assert plan["kernel"] == ("jit_rows" if which == "jit" else "rows_axpby_" + dt), plan


@pytest.mark.parametrize("rc", ["0", "1"])
@pytest.mark.parametrize("dt", ["f16", "f32", "bf16"])
def test_rows_row_constant_forms(monkeypatch, rc, dt):
    """A kernel compiled at run time for the rows path, with its row-constant
    inputs read from the argument block (ECMD_ROWS_RC=0) or fixed in the
    kernel (1), over per-channel views of several batches, including rows
    with a partial last vector."""
    monkeypatch.setenv("ECMD_ROWS_RC", rc)
    rng = np.random.default_rng(600 + int(rc) + len(dt))
    N, C, L = 3, 11, 1003

    def draw(shape):
        f = (rng.standard_normal(shape) * 8).astype(np.float32)
        if dt == "bf16":
            return (f.view(np.uint32) >> 16).astype(np.uint16)
        return f.astype(np.float16) if dt == "f16" else f

    xs = draw((N, C, L + 5))                     # rows of L + 5: 16-byte aligned only for f32
    if dt != "f32":
        xs = draw((N, C, L + 13))                # L + 13 = 1016: a multiple of 8
    x = xs[:, :, :L]
    cs, bs = draw((C, 1)), draw((N, C, 1))
    c = as_strided(cs, shape=(N, C, L), strides=(0, cs.strides[0], 0), writeable=False)
    b = as_strided(bs, shape=(N, C, L), strides=(bs.strides[0], bs.strides[1], 0), writeable=False)
    spec = [("x", ("load", dt, 3)), ("c", ("load", dt, 3)), ("b", ("load", dt, 3)), ("m", ("mul", "x", "c")),
            ("a", ("sub", "m", "b")), ("o", ("store", "a", 3))]
    os_ = draw((N, C, xs.shape[2]))
    o = os_[:, :, :L]
    plan = run_views(spec, [(x, xs), (c, cs), (b, bs)], [(o, os_)], False, "rows rc=%s %s" % (rc, dt), jit=True)
    assert plan["path"] == "rows" and plan["kernel"] == "jit_rows", plan


@pytest.mark.parametrize("knob", ["ECMD_STREAM_STORE=1", "ECMD_OCC_LDS=24576"])
@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("L,pad", [(512, 0), (1024, 0), (1003, 5)])
def test_rows_store_switches(monkeypatch, knob, dt, L, pad):
    """The rows kernels with streaming stores forced below the size that
    selects them (rows of whole 128-byte lines and of a multiple of 64
    vectors: each wavefront stores its 64 vectors of one row as one buffer;
    other rows keep ordinary stores) and with occupancy bounded through LDS,
    over a per-channel affine map on several planes; padding stays untouched."""
    name, value = knob.split("=")
    monkeypatch.setenv(name, value)
    rng = np.random.default_rng(L + pad + len(dt) + len(knob))
    N, C = 3, 11

    def draw(shape):
        f = (rng.standard_normal(shape) * 8).astype(np.float32)
        return f.astype(np.float16) if dt == "f16" else f

    xs = draw((N, C, L + pad))
    x = xs[:, :, :L]
    cs, bs = draw((C, 1)), draw((N, C, 1))
    c = as_strided(cs, shape=(N, C, L), strides=(0, cs.strides[0], 0), writeable=False)
    b = as_strided(bs, shape=(N, C, L), strides=(bs.strides[0], bs.strides[1], 0), writeable=False)
    spec = [("x", ("load", dt, 3)), ("c", ("load", dt, 3)), ("b", ("load", dt, 3)), ("m", ("mul", "x", "c")),
            ("a", ("sub", "m", "b")), ("o", ("store", "a", 3))]
    os_ = draw((N, C, L + pad))
    o = os_[:, :, :L]
    plan = run_views(spec, [(x, xs), (c, cs), (b, bs)], [(o, os_)], False,
                     "rows %s %s L=%d+%d" % (knob, dt, L, pad), jit=True)
    assert plan["path"] == "rows", plan


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape,xpad,ypad", [((2, 200, 300), 4, 4), ((1, 64, 128), 0, 0), ((3, 77, 1000), 8, 3),
                                             ((1, 1000, 72), 24, 0), ((2, 130, 66), 6, 6), ((1, 96, 200), 4, 4),
                                             ((2, 70, 130), 6, 2)])
def test_tiled_16bit_vectors(dt, shape, xpad, ypad):
    """Transposed 16-bit operands on the tiled path, compiled at run time:
    vectors of 8 elements (64 x 256 tiles) when every plane's rows (X, the
    outputs: C + xpad) and staged columns (Y: R + ypad) start on 16 bytes,
    else of 4, with edge tiles on both sides, several planes, padded rows and
    two outputs; the padding must stay untouched."""
    B, R, C = shape
    pad = xpad
    rng = np.random.default_rng(sum(shape) + xpad + 3 * ypad + len(dt))

    def draw(shp):
        f = (rng.standard_normal(shp) * 8).astype(np.float32)
        return (f.view(np.uint32) >> 16).astype(np.uint16) if dt == "bf16" else f.astype(np.float16)

    xs = draw((B, R, C + pad))
    ys = draw((B, C, R + ypad))
    x, yt = xs[:, :, :C], ys[:, :, :R].transpose(0, 2, 1)
    o0s, o1s = draw((B, R, C + pad)), draw((B, R, C + pad))
    spec = [("X", ("load", dt, 3)), ("Yt", ("load", dt, 3)), ("a", ("scalar", dt)), ("ay", ("mul", "a", "Yt")),
            ("s", ("add", "X", "ay")), ("m", ("min", "s", "X")), ("n", ("neg", "m")),
            ("o0", ("store", "s", 3)), ("o1", ("store", "n", 3))]
    a = np.float16(-1.5) if dt == "f16" else np.uint16(0xBFC0)
    plan = run_views(spec, [(x, xs), (yt, ys), a], [(o0s[:, :, :C], o0s), (o1s[:, :, :C], o1s)], False,
                     "tiled16 %s %s pad %d/%d" % (dt, shape, xpad, ypad), jit=True)
    v = 8 if (C + xpad) % 8 == 0 and (R + ypad) % 8 == 0 else 4
    assert plan["path"] == "tiled" and plan["kernel"] == "jit_tiled" and plan["elems_per_thread"] == v, plan


@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("n_staged", [1, 2, 3])
def test_tiled_compiled_staged_counts(dt, n_staged):
    """One to three transposed inputs on the tiled path, compiled at run
    time: the staging tiles of all of them fit the 64 KiB of LDS (narrower
    tiles for more inputs), over a batch of planes with edge tiles."""
    B, R, C = 2, 200, 264
    rng = np.random.default_rng(70 + n_staged + len(dt))

    def draw(shp):
        return (rng.standard_normal(shp) * 4).astype(np.float16 if dt == "f16" else np.float32)

    xs = draw((B, R, C + 8))
    ins = [(xs[:, :, :C], xs)]
    spec = [("X", ("load", dt, 3))]
    acc = "X"
    for k in range(n_staged):
        ys = draw((B, C, R + 8))
        ins.append((ys[:, :, :R].transpose(0, 2, 1), ys))
        spec.append(("Y%d" % k, ("load", dt, 3)))
        spec.append(("s%d" % k, ("add", acc, "Y%d" % k)))
        acc = "s%d" % k
    spec.append(("o", ("store", acc, 3)))
    os_ = draw((B, R, C + 8))
    plan = run_views(spec, ins, [(os_[:, :, :C], os_)], False, "staged x%d %s" % (n_staged, dt), jit=True)
    assert plan["path"] == "tiled" and plan["kernel"] == "jit_tiled", plan
    assert plan["lds_bytes"] <= 65536 and plan["elems_per_thread"] == (8 if dt == "f16" else 4), plan


@pytest.mark.parametrize("dt", ["f32", "f16"])
@pytest.mark.parametrize("shape", [(2, 200, 264), (1, 64, 256), (3, 72, 136)])
def test_tiled_compiled_row_constants(dt, shape):
    """A transposed input with per-row and per-column constants (stride 0
    along the columns, stride 0 along the rows) on the tiled path, compiled
    at run time with the row-constant inputs fixed in the kernel."""
    B, R, C = shape
    rng = np.random.default_rng(80 + sum(shape) + len(dt))

    def draw(shp):
        return (rng.standard_normal(shp) * 4).astype(np.float16 if dt == "f16" else np.float32)

    xs, ys = draw((B, R, C + 8)), draw((B, C, R + 8))
    rs, cs = draw((B, R, 1)), draw((1, 1, C))
    rv = as_strided(rs, shape=(B, R, C), strides=(rs.strides[0], rs.strides[1], 0), writeable=False)
    cv = as_strided(cs, shape=(B, R, C), strides=(0, 0, cs.strides[2]), writeable=False)
    spec = [("X", ("load", dt, 3)), ("Yt", ("load", dt, 3)), ("r", ("load", dt, 3)), ("c", ("load", dt, 3)),
            ("yr", ("mul", "Yt", "r")), ("s", ("add", "X", "yr")), ("t", ("sub", "s", "c")), ("o", ("store", "t", 3))]
    os_ = draw((B, R, C + 8))
    plan = run_views(spec, [(xs[:, :, :C], xs), (ys[:, :, :R].transpose(0, 2, 1), ys), (rv, rs), (cv, cs)],
                     [(os_[:, :, :C], os_)], False, "tiled row constants %s %s" % (dt, shape), jit=True)
    assert plan["path"] == "tiled" and plan["kernel"] == "jit_tiled", plan
