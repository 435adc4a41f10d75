"""GPU parity of the linear path's interpreter (kernels_interp.hip: the
register file in LDS, binary32 inputs loaded straight into it) against the
oracle.

  * random Commands over every operation at lengths around the 256-element
    sub-chunk and the super-chunk boundaries, with one, two and four
    sub-chunks per super-chunk (ECMD_INTERP_K);
  * a large register file (six inputs, six uniform values, eight live
    temporaries), which the host fits in LDS with one sub-chunk;
  * Commands without operations (fills of int32 and binary16, a binary16
    pass-through) and outputs of both widths from one Command.
"""
import numpy as np
import pytest

from gpu_util import compare, dev, host, run_gpu, run_oracle, to_dev
from random_commands import _random_inputs, _random_spec
from specs import arg_dtypes

pytestmark = pytest.mark.gpu

LENGTHS = [1, 63, 255, 256, 511, 512, 513, 1023, 1024, 1025, 4096 + 300, 65536 + 77, (1 << 20) + 3]


def _gpu_values(vals):
    return [to_dev(v) if isinstance(v, np.ndarray) else
            (v if v.dtype == np.uint16 else float(v) if v.dtype.kind == "f" else int(v)) for v in vals]


def _run_interp(spec, vals, n, what):
    import elementwise_tensor_commands_amd as ecmd
    ref = run_oracle(spec, vals)
    gv = _gpu_values(vals)
    _, outs = arg_dtypes(spec)
    try:
        cmd, got = run_gpu(spec, gv, [((n,), d) for d in outs])
    except ecmd.Error as e:
        assert e.name == "CMD_E_LIMIT", e          # more live temporaries than registers
        pytest.skip(str(e))
    plan = cmd.plan(*gv, *got)
    assert plan["path"] == "linear" and plan["kernel"] == "linear_generic" and plan["block"] == 64, plan
    for k, (g, r) in enumerate(zip(got, ref)):
        compare(host(g), r, 0, "%s out%d\n%s" % (what, k, cmd.dump()))
    return plan


@pytest.mark.parametrize("k", [1, 2, 4])
@pytest.mark.parametrize("seed", range(13))
def test_random_commands_each_sub_chunk_count(monkeypatch, k, seed):
    monkeypatch.setenv("ECMD_FORCE_GENERIC", "1")
    monkeypatch.setenv("ECMD_INTERP_K", str(k))
    rng = np.random.default_rng(7000 + 31 * seed + k)
    spec = _random_spec(rng, int(rng.integers(1, 6)), int(rng.integers(1, 14)), 1)
    n = LENGTHS[seed]
    vals = _random_inputs(rng, spec, (n,))
    try:
        run_oracle(spec, vals)
    except Exception as e:   # the oracle front end refuses -> not a valid Command
        pytest.skip("not a valid Command: %s" % e)
    plan = _run_interp(spec, vals, n, "K=%d seed %d n=%d" % (k, seed, n))
    # k sub-chunks, or fewer where the LDS register file would run past its budget
    assert plan["elems_per_thread"] in [4 * j for j in (1, 2, 4) if j <= k], plan


def test_large_register_file():
    """t_i = x_i * s_i for six inputs and six scalars, two more temporaries, all
    eight live at once, then summed (6 + 6 + 2 = 14 CommandArguments of the 16).
    At most ten values are live at once (x0..x3 stay live for t6 and t7 while
    t0..t3 are made; t4, t5 take the entries of x4, x5): ten entries plus six
    uniform entries, which the host fits in LDS with one sub-chunk (16 KiB)."""
    spec = [("x%d" % i, ("load", "f32", 1)) for i in range(6)]
    spec += [("s%d" % i, ("scalar", "f32")) for i in range(6)]
    spec += [("t%d" % i, ("mul", "x%d" % i, "s%d" % i)) for i in range(6)]
    spec += [("t6", ("sub", "x0", "x1")), ("t7", ("add", "x2", "x3"))]
    acc = "t0"
    for i in range(1, 8):
        spec.append(("a%d" % i, ("add", acc, "t%d" % i)))
        acc = "a%d" % i
    spec += [("o0", ("store", acc, 1)), ("o1", ("store", "t3", 1))]
    n = (1 << 16) + 1000
    rng = np.random.default_rng(11)
    vals = [rng.standard_normal(n).astype(np.float32) for _ in range(6)]
    vals += [np.float32(rng.standard_normal()) for _ in range(6)]
    plan = _run_interp(spec, vals, n, "six inputs, six scalars, eight slots")
    assert plan["elems_per_thread"] == 4 and plan["lds_bytes"] == (10 + 6) * 1024, plan


@pytest.mark.parametrize("dt,val", [("i32", -123456789), ("f16", -0.0), ("bf16", np.uint16(0x7F80))])
@pytest.mark.parametrize("n", [5, 512, 70001])
def test_fill_without_inputs(dt, val, n):
    spec = [("s", ("scalar", dt)), ("o", ("store", "s", 1))]
    import torch
    from gpu_util import NPD, TD
    import elementwise_tensor_commands_amd as ecmd
    out = torch.full((n,), 3, dtype=TD[dt], device=dev())
    c = ecmd.from_spec(spec)
    gval = val if dt == "bf16" else (float(val) if dt == "f16" else int(val))
    c.launch(gval, out)
    torch.cuda.synchronize()
    plan = c.plan(gval, out)
    assert plan["kernel"] == "linear_generic", plan
    ref = run_oracle(spec, [np.uint16(val) if dt == "bf16" else NPD[dt](val)],
                     outputs=[np.zeros(n, NPD[dt])])[0]
    compare(host(out), ref, 0, "fill %s n=%d" % (dt, n))


@pytest.mark.parametrize("n", [3, 777, (1 << 18) + 9])
def test_pass_through_and_mixed_width_outputs(n):
    """out0 = x (binary16, no operation), out1 = f32(x), out2 = bf16(f32(x) * s)."""
    spec = [("x", ("load", "f16", 1)), ("s", ("scalar", "f32")), ("w", ("cvt", "x", "f32")),
            ("p", ("mul", "w", "s")), ("b", ("cvt", "p", "bf16")),
            ("o0", ("store", "x", 1)), ("o1", ("store", "w", 1)), ("o2", ("store", "b", 1))]
    rng = np.random.default_rng(n)
    vals = [(rng.standard_normal(n) * 300).astype(np.float16), np.float32(-0.375)]
    _run_interp(spec, vals, n, "pass-through n=%d" % n)


# ---------------------------------------------------------------------------
# The rows path's interpreter (k_rows_interp): padded rows, row-constant and
# column-broadcast inputs, 16-bit inputs and outputs, rows that hold whole
# wavefronts (n3 a multiple of 256), rows that do not, and partial vectors.

@pytest.mark.parametrize("dx", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("db", ["f32", "f16"])
@pytest.mark.parametrize("n3", [256, 1024, 100, 253, 7])
def test_rows_interp_views(dx, db, n3):
    import torch
    from gpu_util import NPD
    rows = 37
    ld = (n3 + 12 + 3) // 4 * 4          # padded rows whose starts keep 4-element vectors aligned
    spec = [("x", ("load", dx, 2)), ("b", ("load", db, 2)), ("c", ("load", "f32", 2)),
            ("xf", ("cvt", "x", "f32")), ("bf", ("cvt", "b", "f32")), ("t", ("mul", "xf", "bf")),
            ("u", ("add", "t", "c")), ("u16", ("cvt", "u", dx)),
            ("o0", ("store", "u", 2)), ("o1", ("store", "u16", 2))]
    rng = np.random.default_rng(n3 * 10 + len(dx) + len(db))

    def draw(dt, shape):
        f = (rng.standard_normal(shape) * 50).astype(np.float32)
        if dt == "bf16":
            return (f.view(np.uint32) >> 16).astype(np.uint16)
        return f.astype(NPD[dt])

    xs = draw(dx, (rows, ld))
    bv = draw(db, (rows, 1))
    cv = draw("f32", (1, n3))
    x_log = np.ascontiguousarray(xs[:, :n3])
    ref = run_oracle(spec, [x_log, np.ascontiguousarray(np.broadcast_to(bv, (rows, n3))),
                            np.ascontiguousarray(np.broadcast_to(cv, (rows, n3)))])
    xg = to_dev(xs)[:, :n3]
    bg = to_dev(bv).expand(rows, n3)
    cg = to_dev(cv).expand(rows, n3)
    from gpu_util import TD
    o0s = torch.full((rows, ld), float("nan"), dtype=torch.float32, device=dev())
    o1s = torch.zeros((rows, ld), dtype=TD[dx], device=dev())
    o0, o1 = o0s[:, :n3], o1s[:, :n3]
    import elementwise_tensor_commands_amd as ecmd
    cmd = ecmd.from_spec(spec)
    plan = cmd.plan(xg, bg, cg, o0, o1)
    assert plan["path"] == "rows" and plan["kernel"] == "rows_generic" and plan["block"] == 64, plan
    cmd.launch(xg, bg, cg, o0, o1)
    torch.cuda.synchronize()
    compare(host(o0), ref[0], 0, "rows interp %s/%s n3=%d out0" % (dx, db, n3))
    compare(host(o1), ref[1], 0, "rows interp %s/%s n3=%d out1" % (dx, db, n3))
    assert torch.isnan(o0s[:, n3:]).all() and (host(o1s[:, n3:]).view(np.uint16) == 0).all()   # padding untouched


# ---------------------------------------------------------------------------
# The tiled path's interpreter (k_tiled_interp, 32 x 64 tiles) and, for
# comparison, the tiled kernel with RtEval (ECMD_TILED_RTEVAL=1).

TILED_INTERP_SHAPES = ["32x64x256", "32x64x128", "64x64x256", "32x128x256", "64x64x512"]


@pytest.mark.parametrize("kernel", ["rteval"] + TILED_INTERP_SHAPES)
@pytest.mark.parametrize("shape", [(64, 128), (32, 64), (100, 68), (36, 132), (8, 300)])
def test_tiled_interp_mixed_inputs(monkeypatch, kernel, shape):
    """A binary16 direct input, a binary32 input read transposed (staged), a
    per-row constant and a scalar; binary32 and bfloat16 outputs.  Every
    instantiated tile shape of the interpreter (ECMD_TILED_INTERP; the first
    is the default) and the tiled kernel with RtEval."""
    import torch
    import elementwise_tensor_commands_amd as ecmd
    rteval = kernel == "rteval"
    if rteval:
        monkeypatch.setenv("ECMD_TILED_RTEVAL", "1")
    else:
        monkeypatch.setenv("ECMD_TILED_INTERP", kernel)
    R, C = shape
    spec = [("x", ("load", "f16", 2)), ("y", ("load", "f32", 2)), ("b", ("load", "f32", 2)),
            ("s", ("scalar", "f32")),
            ("xf", ("cvt", "x", "f32")), ("p", ("mul", "xf", "y")), ("q", ("add", "p", "b")),
            ("r", ("sub", "q", "s")), ("rb", ("cvt", "r", "bf16")),
            ("o0", ("store", "r", 2)), ("o1", ("store", "rb", 2))]
    rng = np.random.default_rng(R * 1000 + C)
    x = (rng.standard_normal((R, C)) * 30).astype(np.float16)
    yt = rng.standard_normal((C, R)).astype(np.float32)          # y = yt.T: read transposed
    b = rng.standard_normal((R, 1)).astype(np.float32)
    s = np.float32(0.625)
    ref = run_oracle(spec, [x, np.ascontiguousarray(yt.T), np.ascontiguousarray(np.broadcast_to(b, (R, C))), s])
    gv = [to_dev(x), to_dev(yt).t(), to_dev(b).expand(R, C), float(s)]
    o0 = torch.full((R, C), float("nan"), device=dev())
    o1 = torch.zeros((R, C), dtype=torch.bfloat16, device=dev())
    cmd = ecmd.from_spec(spec)
    plan = cmd.plan(*gv, o0, o1)
    assert plan["path"] == "tiled" and plan["kernel"] == "tiled_generic", plan
    assert (plan["lds_bytes"] == 64 * 64 * 4) == rteval, plan      # RtEval: one 64 x 64 staging tile
    cmd.launch(*gv, o0, o1)
    torch.cuda.synchronize()
    compare(host(o0), ref[0], 0, "tiled interp %s %s out0" % (shape, kernel))
    compare(host(o1), ref[1], 0, "tiled interp %s %s out1" % (shape, kernel))


@pytest.mark.parametrize("seed", range(24))
def test_tiled_interp_random_transposed_views(seed):
    """Random Commands over random transposed rank-2..4 views: most take the
    tiled path with the interpreter."""
    from random_commands import random_view_case
    from test_gpu_views import run_views
    spec, ins, outs = random_view_case(seed + 500, staged=True)
    run_views(spec, ins, outs, False, "tiled interp seed %d" % seed)


@pytest.mark.parametrize("k", [1, 2, 4])
@pytest.mark.parametrize("vec_per_row", [64 * 4 * 3, 64 * 3, 77])
@pytest.mark.parametrize("partial", [False, True])
def test_rows_interp_row_modes(monkeypatch, k, vec_per_row, partial):
    """Each row mode of the rows interpreter at each sub-chunk count: rows of a
    multiple of 64 K vectors (a super-chunk never spans two rows), of 64
    vectors (a sub-chunk never does), and of neither; a padded binary32
    input, a binary16 input and a per-row constant; with `partial` the last
    vector of every row holds fewer than 4 elements."""
    import torch
    import elementwise_tensor_commands_amd as ecmd
    from gpu_util import TD
    monkeypatch.setenv("ECMD_FORCE_GENERIC", "1")
    monkeypatch.setenv("ECMD_INTERP_K", str(k))
    rows = 21
    n3 = 4 * vec_per_row - (3 if partial else 0)
    ld = (n3 + 8 + 3) // 4 * 4
    spec = [("x", ("load", "f32", 2)), ("h", ("load", "f16", 2)), ("b", ("load", "f32", 2)),
            ("z", ("scalar", "f32")), ("hf", ("cvt", "h", "f32")), ("t", ("add", "x", "b")),
            ("u", ("mul", "t", "hf")), ("r", ("max", "u", "z")), ("o", ("store", "r", 2))]
    rng = np.random.default_rng(k * 1000 + vec_per_row + partial)
    xs = rng.standard_normal((rows, ld)).astype(np.float32)
    hs = (rng.standard_normal((rows, ld)) * 3).astype(np.float16)
    bv = rng.standard_normal((rows, 1)).astype(np.float32)
    ref = run_oracle(spec, [np.ascontiguousarray(xs[:, :n3]), np.ascontiguousarray(hs[:, :n3]),
                            np.ascontiguousarray(np.broadcast_to(bv, (rows, n3))), np.float32(0.0)])[0]
    os_ = torch.full((rows, ld), float("nan"), device=dev())
    gv = [to_dev(xs)[:, :n3], to_dev(hs)[:, :n3], to_dev(bv).expand(rows, n3), 0.0]
    cmd = ecmd.from_spec(spec)
    plan = cmd.plan(*gv, os_[:, :n3])
    assert plan["path"] == "rows" and plan["kernel"] == "rows_generic", plan
    cmd.launch(*gv, os_[:, :n3])
    torch.cuda.synchronize()
    compare(host(os_[:, :n3]), ref, 0, "rows modes K=%d %d vectors per row%s (K used %d)" % (
        k, vec_per_row, ", partial last" if partial else "", plan["elems_per_thread"] // 4))
    assert torch.isnan(os_[:, n3:]).all()


@pytest.mark.parametrize("n", [13 * 1024 + 77, 1024 * 10, 300])
def test_linear_interp_split_into_dispatches(monkeypatch, n):
    """The linear interpreter's work in dispatches of 5 work-groups
    (ECMD_INTERP_DISPATCH), the tail done by the last super-chunk's work-group
    (or by the only work-group when there is no whole super-chunk)."""
    monkeypatch.setenv("ECMD_FORCE_GENERIC", "1")
    monkeypatch.setenv("ECMD_INTERP_DISPATCH", "5")
    rng = np.random.default_rng(n)
    spec = [("x", ("load", "f32", 1)), ("y", ("load", "i32", 1)), ("s", ("scalar", "f32")),
            ("yf", ("cvt", "y", "f32")), ("t", ("mul", "x", "s")), ("u", ("sub", "t", "yf")),
            ("o", ("store", "u", 1))]
    vals = [rng.standard_normal(n).astype(np.float32), rng.integers(-1000, 1000, n, dtype=np.int32),
            np.float32(1.25)]
    plan = _run_interp(spec, vals, n, "dispatches of 5, n=%d" % n)
    assert plan["grid"] == min(5, max(1, n // (64 * plan["elems_per_thread"]))), plan


@pytest.mark.parametrize("shape", [(64, 128), (100, 68), (36, 300)])
def test_tiled_interp_three_staged_inputs(shape):
    """Three inputs read transposed (binary16, bfloat16, binary32), each staged
    in its own entry's LDS region and overwritten there by its entries, with
    a direct binary32 input and a per-row constant; full and edge tiles."""
    import torch
    import elementwise_tensor_commands_amd as ecmd
    R, C = shape
    spec = [("a", ("load", "f16", 2)), ("b", ("load", "bf16", 2)), ("c", ("load", "f32", 2)),
            ("d", ("load", "f32", 2)), ("r", ("load", "f32", 2)),
            ("af", ("cvt", "a", "f32")), ("bf", ("cvt", "b", "f32")), ("p", ("mul", "af", "bf")),
            ("q", ("add", "p", "c")), ("u", ("sub", "q", "d")), ("v", ("mul", "u", "r")),
            ("o", ("store", "v", 2))]
    rng = np.random.default_rng(R * 7 + C)
    at = (rng.standard_normal((C, R)) * 4).astype(np.float16)
    bt = (rng.standard_normal((C, R)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ct = rng.standard_normal((C, R)).astype(np.float32)
    d = rng.standard_normal((R, C)).astype(np.float32)
    r = rng.standard_normal((R, 1)).astype(np.float32)
    ref = run_oracle(spec, [np.ascontiguousarray(at.T), np.ascontiguousarray(bt.T), np.ascontiguousarray(ct.T), d,
                            np.ascontiguousarray(np.broadcast_to(r, (R, C)))])[0]
    gv = [to_dev(at).t(), to_dev(bt).t(), to_dev(ct).t(), to_dev(d), to_dev(r).expand(R, C)]
    out = torch.full((R, C), float("nan"), device=dev())
    cmd = ecmd.from_spec(spec)
    plan = cmd.plan(*gv, out)
    assert plan["path"] == "tiled" and plan["kernel"] == "tiled_generic", plan
    cmd.launch(*gv, out)
    torch.cuda.synchronize()
    compare(host(out), ref, 0, "three staged inputs %s (lds %d)" % (shape, plan["lds_bytes"]))


@pytest.mark.parametrize("n", [9 * 1024 + 5, 700])
def test_linear_interp_split_16bit(monkeypatch, n):
    """Dispatches of 3 work-groups with binary16 and bfloat16 inputs (2-byte
    direct loads) and both output widths."""
    monkeypatch.setenv("ECMD_INTERP_DISPATCH", "3")
    rng = np.random.default_rng(n + 1)
    spec = [("h", ("load", "f16", 1)), ("b", ("load", "bf16", 1)), ("hf", ("cvt", "h", "f32")),
            ("bf", ("cvt", "b", "f32")), ("t", ("sub", "hf", "bf")), ("m", ("max", "t", "hf")),
            ("mh", ("cvt", "m", "bf16")), ("o0", ("store", "t", 1)), ("o1", ("store", "mh", 1))]
    vals = [(rng.standard_normal(n) * 8).astype(np.float16),
            (rng.standard_normal(n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)]
    plan = _run_interp(spec, vals, n, "16-bit dispatches of 3, n=%d" % n)
    assert plan["grid"] == min(3, max(1, n // (64 * plan["elems_per_thread"]))), plan
