"""GPU parity of the gather path's interpreter (k_gather_interp in
kernels_interp.hip) against the oracle.

Views no vector path takes: rows whose starts are off 16 bytes, strided
columns, stride-0 broadcasts along a row, outputs with padded or strided
rows.  Every mode of the interpreter — segments of one row, whole rows of a
plane, whole rows over three row dimensions — with one, two and four
sub-chunks per super-chunk (ECMD_INTERP_K), rows that end inside a segment,
planes whose last super-chunk holds fewer rows, binary16 and bfloat16 inputs
(2-byte direct loads to LDS) and outputs of both widths.  Row padding and
the elements between strided columns of the outputs must stay untouched.
The per-element kernel (ECMD_GATHER_MODE=0) runs the same cases.
"""
import numpy as np
import pytest
import torch

from gpu_util import NPD, TD, compare, dev, host, run_oracle, to_dev

pytestmark = pytest.mark.gpu

SPEC = [("x", ("load", "f16", 3)), ("y", ("load", "f32", 3)), ("b", ("load", "bf16", 3)),
        ("i", ("load", "i32", 3)), ("s", ("scalar", "f32")),
        ("xf", ("cvt", "x", "f32")), ("bf", ("cvt", "b", "f32")), ("p", ("mul", "xf", "y")),
        ("q", ("add", "p", "bf")), ("r", ("sub", "q", "s")), ("rh", ("cvt", "r", "bf16")),
        ("ii", ("add", "i", "i")),
        ("o0", ("store", "r", 3)), ("o1", ("store", "rh", 3)), ("o2", ("store", "ii", 3))]

# (batch, rows, n3): segments (n3 above half a super-chunk of 256 K elements),
# whole rows of one plane (batch 1), whole rows over a batch.
SHAPES = [(1, 37, 2100), (1, 5, 1025), (1, 3, 257), (1, 300, 6), (1, 77, 1), (1, 19, 200),
          (3, 41, 7), (2, 9, 130), (4, 5, 600)]


def _draw(rng, dt, shape):
    f = (rng.standard_normal(shape) * 40).astype(np.float32)
    if dt == "bf16":
        return (f.view(np.uint32) >> 16).astype(np.uint16)
    if dt == "i32":
        return rng.integers(-(1 << 30), 1 << 30, shape, dtype=np.int32)
    return f.astype(NPD[dt])


def _case(shape, seed):
    """Inputs and outputs as (host view, device view) over padded storage."""
    B, R, C = shape
    rng = np.random.default_rng(seed)
    xs = _draw(rng, "f16", (B, R, C + 3))            # rows 2 (C + 3) bytes apart: off 16 bytes
    ys = _draw(rng, "f32", (B, R, 2 * C))             # every other column
    bs = _draw(rng, "bf16", (B, R, 1))                # one value per row (stride 0 along the row)
    is_ = _draw(rng, "i32", (B, R + 1, C + 1))        # padded rows and a spare row per batch
    s = np.float32(0.375)
    hx, hy = xs[:, :, :C], ys[:, :, ::2]
    hb = np.ascontiguousarray(np.broadcast_to(bs, (B, R, C)))
    hi = is_[:, :R, :C]
    ref = run_oracle(SPEC, [np.ascontiguousarray(hx), np.ascontiguousarray(hy), hb, np.ascontiguousarray(hi), s])
    gx = to_dev(xs)[:, :, :C]
    gy = to_dev(ys)[:, :, ::2]
    gb = to_dev(bs).expand(B, R, C)
    gi = to_dev(is_)[:, :R, :C]
    return [gx, gy, gb, gi, float(s)], ref


def _outputs(shape):
    B, R, C = shape
    o0s = torch.full((B, R, C + 1), float("nan"), dtype=torch.float32, device=dev())   # padded rows
    o1s = torch.zeros((B, R, 2 * C), dtype=torch.bfloat16, device=dev())              # every other column
    o2s = torch.full((B, R, C + 5), -7, dtype=torch.int32, device=dev())
    return (o0s, o1s, o2s), [o0s[:, :, :C], o1s[:, :, ::2], o2s[:, :, :C]]


def _check(shape, store, outs, ref, what):
    B, R, C = shape
    o0s, o1s, o2s = store
    compare(host(outs[0]), ref[0], 0, what + " out0")
    compare(host(outs[1]), ref[1], 0, what + " out1")
    compare(host(outs[2]), ref[2], 0, what + " out2")
    assert torch.isnan(o0s[:, :, C:]).all(), what + ": out0 padding written"
    assert (o1s[:, :, 1::2].view(torch.int16) == 0).all(), what + ": out1 gaps written"
    assert (o2s[:, :, C:] == -7).all(), what + ": out2 padding written"


@pytest.mark.parametrize("k", [1, 2, 4])
@pytest.mark.parametrize("shape", SHAPES)
def test_gather_interp_modes(monkeypatch, k, shape):
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_INTERP_K", str(k))
    vals, ref = _case(shape, 100 * k + sum(shape))
    store, outs = _outputs(shape)
    cmd = ecmd.from_spec(SPEC)
    plan = cmd.plan(*vals, *outs)
    B, R, C = shape
    kk = plan["elems_per_thread"] // 4      # K, or fewer where the register file would outgrow LDS
    want = "gather_segments" if C > 128 * kk else "gather_whole_rows"
    assert kk <= k and plan["path"] == "gather" and plan["kernel"] == want and plan["block"] == 64, plan
    print("    gather K=%d %s: %s grid %d" % (k, shape, plan["kernel"], plan["grid"]), flush=True)
    cmd.launch(*vals, *outs)
    torch.cuda.synchronize()
    _check(shape, store, outs, ref, "gather K=%d %s" % (k, shape))


@pytest.mark.parametrize("shape", SHAPES[:4] + SHAPES[6:7])
def test_gather_per_element_kernel(monkeypatch, shape):
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_GATHER_MODE", "0")
    vals, ref = _case(shape, 7 + sum(shape))
    store, outs = _outputs(shape)
    cmd = ecmd.from_spec(SPEC)
    plan = cmd.plan(*vals, *outs)
    assert plan["kernel"] == "gather_generic", plan
    cmd.launch(*vals, *outs)
    torch.cuda.synchronize()
    _check(shape, store, outs, ref, "per-element gather %s" % (shape,))


@pytest.mark.parametrize("dt,bits", [("i32", 0x89ABCDEF), ("f16", 0xBC00), ("bf16", 0x7F80)])
@pytest.mark.parametrize("shape", [(1, 50, 1000), (2, 33, 5)])
def test_gather_fill_strided(dt, bits, shape):
    """A Command without inputs (a scalar stored) into every other column: the
    output entry is the uniform value's."""
    import elementwise_tensor_commands_amd as ecmd
    B, R, C = shape
    spec = [("v", ("scalar", dt)), ("o", ("store", "v", 3))]
    store = torch.zeros((B, R, 2 * C), dtype=TD[dt], device=dev())
    out = store[:, :, ::2]
    val = bits if dt == "i32" else -1.0 if dt == "f16" else np.uint16(bits)     # 0xBC00 is binary16 -1.0
    cmd = ecmd.from_spec(spec)
    plan = cmd.plan(val, out)
    assert plan["path"] == "gather", plan
    cmd.launch(val, out)
    torch.cuda.synchronize()
    h = host(store)
    w = h.view(np.uint32) if dt == "i32" else h.view(np.uint16)
    assert (w[:, :, ::2] == bits).all() and (w[:, :, 1::2] == 0).all()


@pytest.mark.parametrize("n", [1, 255, 256, 257, 511, 512, 513, 100003])
@pytest.mark.parametrize("k", [1, 2, 4])
def test_gather_rank1_stride(monkeypatch, n, k):
    """x[::3] - y[::2] over one row: segments with a ragged last one."""
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_INTERP_K", str(k))
    rng = np.random.default_rng(n + k)
    xs = rng.standard_normal(3 * n).astype(np.float32)
    ys = rng.standard_normal(2 * n).astype(np.float32)
    spec = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)), ("d", ("sub", "x", "y")), ("o", ("store", "d", 1))]
    ref = run_oracle(spec, [np.ascontiguousarray(xs[::3]), np.ascontiguousarray(ys[::2])])[0]
    out = torch.full((n,), float("nan"), device=dev())
    cmd = ecmd.from_spec(spec)
    gx, gy = to_dev(xs)[::3], to_dev(ys)[::2]
    plan = cmd.plan(gx, gy, out)
    assert plan["path"] == ("gather" if n > 1 else "linear"), plan
    cmd.launch(gx, gy, out)
    torch.cuda.synchronize()
    compare(host(out), ref, 0, "rank-1 stride n=%d K=%d" % (n, k))


@pytest.mark.parametrize("shape", [(1, 37, 2100), (3, 400, 7), (2, 90, 130)])
def test_gather_split_into_dispatches(monkeypatch, shape):
    """The work split into dispatches of 7 work-groups (ECMD_GATHER_DISPATCH),
    each starting at its own super-chunk."""
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_GATHER_DISPATCH", "7")
    vals, ref = _case(shape, 31 + sum(shape))
    store, outs = _outputs(shape)
    cmd = ecmd.from_spec(SPEC)
    plan = cmd.plan(*vals, *outs)
    assert plan["path"] == "gather" and plan["grid"] == 7, plan
    cmd.launch(*vals, *outs)
    torch.cuda.synchronize()
    _check(shape, store, outs, ref, "gather in dispatches of 7, %s" % (shape,))


@pytest.mark.parametrize("shape", SHAPES)
def test_gather_compiled(monkeypatch, shape):
    """The gather kernel compiled at run time for the Program (k_gather_cc:
    the same element placement, the values in registers), every mode, on
    the same cases as the interpreter; and split into dispatches of 2
    work-groups."""
    import elementwise_tensor_commands_amd as ecmd
    vals, ref = _case(shape, 900 + sum(shape))
    for dispatch in (None, "2"):
        if dispatch:
            monkeypatch.setenv("ECMD_GATHER_DISPATCH", dispatch)
        store, outs = _outputs(shape)
        cmd = ecmd.from_spec(SPEC).jit()
        plan = cmd.plan(*vals, *outs)
        assert plan["path"] == "gather" and plan["kernel"] == "jit_gather" and plan["block"] == 256, plan
        if dispatch:
            assert plan["grid"] <= 2, plan
        cmd.prepare(*vals, *outs)
        cmd.launch(*vals, *outs)
        torch.cuda.synchronize()
        _check(shape, store, outs, ref, "compiled gather %s dispatch %s" % (shape, dispatch))


@pytest.mark.parametrize("e", [4, 16])
@pytest.mark.parametrize("shape", [(1, 37, 2100), (3, 41, 7)])
def test_gather_compiled_other_widths(monkeypatch, e, shape):
    """The compiled gather kernel at the other elements-per-work-item choices
    (ECMD_GATHER_JIT_E, for A/B runs)."""
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_GATHER_JIT_E", str(e))
    vals, ref = _case(shape, 700 + e + sum(shape))
    store, outs = _outputs(shape)
    cmd = ecmd.from_spec(SPEC).jit()
    plan = cmd.plan(*vals, *outs)
    assert plan["kernel"] == "jit_gather" and plan["elems_per_thread"] == e, plan
    cmd.prepare(*vals, *outs)
    cmd.launch(*vals, *outs)
    torch.cuda.synchronize()
    _check(shape, store, outs, ref, "compiled gather E=%d %s" % (e, shape))


@pytest.mark.parametrize("shape", [(1, 37, 2100), (3, 41, 7), (2, 9, 130)])
def test_gather_compiled_64bit_offsets(monkeypatch, shape):
    """The compiled gather kernel's 64-bit offset arithmetic (taken by views
    spanning 2^32 elements and more; ECMD_GATHER_S32=0 forces it here)."""
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_GATHER_S32", "0")
    vals, ref = _case(shape, 900 + sum(shape))
    store, outs = _outputs(shape)
    cmd = ecmd.from_spec(SPEC).jit()
    plan = cmd.plan(*vals, *outs)
    assert plan["kernel"] == "jit_gather", plan
    cmd.prepare(*vals, *outs)
    cmd.launch(*vals, *outs)
    torch.cuda.synchronize()
    _check(shape, store, outs, ref, "compiled gather, 64-bit offsets %s" % (shape,))


CONTIG_SPEC = [("x", ("load", "f32", 3)), ("i", ("load", "i32", 3)), ("s", ("scalar", "f32")),
               ("p", ("mul", "x", "s")), ("ii", ("sub", "i", "i")), ("j", ("add", "ii", "i")),
               ("h", ("cvt", "p", "f16")),
               ("o0", ("store", "p", 3)), ("o1", ("store", "j", 3)), ("o2", ("store", "h", 3))]


@pytest.mark.parametrize("shape", [(1, 37, 2100), (1, 5, 1025), (1, 37, 1000), (1, 300, 6), (1, 77, 1),
                                   (1, 19, 200), (3, 41, 7), (2, 9, 130)])
@pytest.mark.parametrize("off", [0, 1, 5, 31])
def test_gather_compiled_contiguous_outputs(shape, off):
    """Contiguous outputs of the compiled gather kernel (every mode: unit-stride
    rows for segments, outputs contiguous across rows for whole rows): two
    32-bit outputs and a binary16 one, each starting `off` elements into a
    guard-banded buffer, so rows start at every place in a line.  Segments
    are laid from out0's lines, so a row's first segment starts before the
    row and 1000-column rows end with an empty segment; whole-row chunks end
    on out0's lines.  The guards must stay untouched."""
    import elementwise_tensor_commands_amd as ecmd
    B, R, C = shape
    rng = np.random.default_rng(40 + off + sum(shape))
    xs = (rng.standard_normal((B, R, C + 1)) * 10).astype(np.float32)     # rows 4 bytes off: the gather path
    ins = rng.integers(-(1 << 30), 1 << 30, (B, R, C), dtype=np.int32)
    hx = np.ascontiguousarray(xs[:, :, :C])
    ref = run_oracle(CONTIG_SPEC, [hx, ins, np.float32(0.75)])
    n, guard = B * R * C, 64
    bufs = [torch.full((n + off + 2 * guard,), v, dtype=d, device=dev())
            for v, d in ((float("nan"), torch.float32), (-7, torch.int32), (float("nan"), torch.float16))]
    outs = [b[guard + off:guard + off + n].view(B, R, C) for b in bufs]
    vals = [to_dev(xs)[:, :, :C], to_dev(ins), 0.75]
    cmd = ecmd.from_spec(CONTIG_SPEC).jit()
    plan = cmd.plan(*vals, *outs)
    assert plan["path"] == "gather" and plan["kernel"] == "jit_gather", plan
    cmd.prepare(*vals, *outs)
    cmd.launch(*vals, *outs)
    torch.cuda.synchronize()
    for k, (o, r) in enumerate(zip(outs, ref)):
        compare(host(o), r, 0, "contiguous outputs %s off %d out%d" % (shape, off, k))
    for k, b in enumerate(bufs):
        hb = host(b)
        for part in (hb[:guard + off], hb[guard + off + n:]):
            if k == 1:
                assert (part == -7).all(), "out%d guard written (%s, off %d)" % (k, shape, off)
            else:
                assert np.isnan(part.astype(np.float32)).all(), "out%d guard written (%s, off %d)" % (k, shape, off)


RUNS_SPEC = [("x", ("load", "f32", 3)), ("y", ("load", "i32", 3)), ("h", ("load", "f16", 3)),
             ("b", ("load", "f32", 3)), ("s", ("scalar", "f32")),
             ("xs", ("mul", "x", "s")), ("t", ("add", "xs", "b")), ("hf", ("cvt", "h", "f32")),
             ("u", ("sub", "t", "hf")), ("yy", ("add", "y", "y")),
             ("o0", ("store", "u", 3)), ("o1", ("store", "yy", 3))]


@pytest.mark.parametrize("shape", [(1, 37, 2100), (1, 5, 1025), (1, 3, 4097), (1, 37, 1000), (1, 300, 6),
                                   (1, 77, 1), (1, 19, 200), (3, 41, 7), (2, 9, 130)])
@pytest.mark.parametrize("off", [0, 1, 5, 31])
@pytest.mark.parametrize("pad", [0, 3])
def test_gather_compiled_contiguous_inputs(shape, off, pad):
    """Inputs of the compiled gather kernel in every layout next to line-laid
    segments: contiguous inputs starting `off` elements into their storage
    (at every place in a 128-byte line), x with rows padded by `pad` elements
    (contiguous per segment, not across whole rows), a binary16 input (rows
    padded, a spare row per batch, 2 bytes off alignment: no vector path
    takes the views, and batches do not merge into one plane) and a per-row
    constant (stride 0 along the row)."""
    import elementwise_tensor_commands_amd as ecmd
    B, R, C = shape
    rng = np.random.default_rng(90 + off + 7 * pad + sum(shape))
    cp = C + pad
    xs = np.full(off + B * R * cp, np.nan, dtype=np.float32)
    xs[off:] = (rng.standard_normal(B * R * cp) * 10).astype(np.float32)
    ys = np.zeros(off + B * R * C, dtype=np.int32)
    ys[off:] = rng.integers(-(1 << 31), 1 << 31, B * R * C, dtype=np.int64).astype(np.int32)
    hs = (rng.standard_normal(1 + B * (R + 1) * (C + 3)) * 4).astype(np.float16)
    bb = (rng.standard_normal((B, R, 1)) * 3).astype(np.float32)
    hx = xs[off:].reshape(B, R, cp)[:, :, :C]
    hy = ys[off:].reshape(B, R, C)
    hh = hs[1:].reshape(B, R + 1, C + 3)[:, :R, :C]
    ref = run_oracle(RUNS_SPEC, [hx, hy, hh, np.broadcast_to(bb, (B, R, C)), np.float32(-1.25)])
    dx, dy = to_dev(xs), to_dev(ys)
    vals = [dx[off:].view(B, R, cp)[:, :, :C], dy[off:].view(B, R, C), to_dev(hs)[1:].view(B, R + 1, C + 3)[:, :R, :C],
            to_dev(bb).expand(B, R, C), -1.25]
    outs = [torch.empty((B, R, C), dtype=torch.float32, device=dev()),
            torch.empty((B, R, C), dtype=torch.int32, device=dev())]
    cmd = ecmd.from_spec(RUNS_SPEC).jit()
    plan = cmd.plan(*vals, *outs)
    assert plan["path"] == "gather" and plan["kernel"] == "jit_gather", plan
    cmd.prepare(*vals, *outs)
    cmd.launch(*vals, *outs)
    torch.cuda.synchronize()
    for k, (o, r) in enumerate(zip(outs, ref)):
        compare(host(o), r, 0, "contiguous inputs %s off %d pad %d out%d" % (shape, off, pad, k))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 37, 2100), (1, 5, 1025), (1, 37, 960), (1, 300, 6), (1, 19, 200),
                                   (3, 41, 7), (2, 9, 130)])
@pytest.mark.parametrize("off", [0, 1, 7, 63])
@pytest.mark.parametrize("wide", [False, True])
def test_gather_compiled_16bit_runs(dt, shape, off, wide):
    """16-bit operands on the compiled gather kernel: segments are laid from
    the 16-bit output's lines of 64 elements when no 32-bit output has unit
    stride (wide: a binary32 output too, which then sets the lines); whole
    rows per chunk fill the lines of both.  y and the outputs start `off`
    elements into guard-banded storage; x's rows are padded by one element."""
    import elementwise_tensor_commands_amd as ecmd
    B, R, C = shape
    rng = np.random.default_rng(300 + off + sum(shape) + 5 * wide + len(dt))

    def draw(n):
        f = (rng.standard_normal(n) * 6).astype(np.float32)
        return (f.view(np.uint32) >> 16).astype(np.uint16) if dt == "bf16" else f.astype(np.float16)

    xs = draw(B * R * (C + 1)).reshape(B, R, C + 1)
    ys = draw(off + B * R * C)
    hx, hy = xs[:, :, :C], ys[off:].reshape(B, R, C)
    spec = [("x", ("load", dt, 3)), ("y", ("load", dt, 3)), ("p", ("mul", "x", "y")), ("q", ("sub", "p", "x")),
            ("o0", ("store", "q", 3))]
    if wide:
        spec += [("w", ("cvt", "q", "f32")), ("o1", ("store", "w", 3))]
    ref = run_oracle(spec, [hx, hy])
    n, guard = B * R * C, 64
    tdt = torch.bfloat16 if dt == "bf16" else torch.float16
    bufs = [torch.full((n + off + 2 * guard,), -3.0, dtype=tdt, device=dev())]
    if wide:
        bufs.append(torch.full((n + off + 2 * guard,), float("nan"), dtype=torch.float32, device=dev()))
    outs = [b[guard + off:guard + off + n].view(B, R, C) for b in bufs]
    vals = [to_dev(xs)[:, :, :C], to_dev(ys)[off:].view(B, R, C)]
    cmd = ecmd.from_spec(spec).jit()
    plan = cmd.plan(*vals, *outs)
    assert plan["path"] == "gather" and plan["kernel"] == "jit_gather", plan
    cmd.prepare(*vals, *outs)
    cmd.launch(*vals, *outs)
    torch.cuda.synchronize()
    for k, (o, r) in enumerate(zip(outs, ref)):
        compare(host(o), r, 0, "16-bit runs %s %s off %d out%d" % (dt, shape, off, k))
    for k, b in enumerate(bufs):
        hb = host(b).astype(np.float32) if k == 0 and dt == "f16" else host(b)
        for part in (hb[:guard + off], hb[guard + off + n:]):
            if k == 0:
                want = np.uint16(0xC040) if dt == "bf16" else np.float32(-3.0)
                assert (part == want).all(), "out0 guard written (%s, off %d)" % (shape, off)
            else:
                assert np.isnan(part).all(), "out1 guard written (%s, off %d)" % (shape, off)
