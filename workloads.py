"""Seeded synthetic workloads for elementwise tensor Commands.

This module holds *inputs only*: the declarative shape of each Command (which
loads, scalars, E_ operations and stores, in declaration order) and seeded
NumPy generators for its tensors and scalars.  It holds none of the arithmetic:
the oracle and the GPU library each turn a spec into their own Command with
their own code.

Spec format: a list of ``(name, step)`` pairs.  ``step`` is one of
``("load", dtype, rank)``, ``("scalar", dtype)``, a binary operation
``(op, a, b)`` (add sub mul min max and the comparisons eq ne lt le gt ge ltu
leu gtu geu), ``("neg"|"abs", a)``, ``("cvt", a, dtype)``,
``("select", cond, a, b)`` or ``("store", value, rank)``, where ``a``, ``b``,
``cond`` and ``value`` name earlier steps.  CommandArguments are the loads,
scalars and stores in the order they appear.

Generators follow one recipe: ``np.random.default_rng(seed)`` (PCG64), with
``seed = 1000 + k`` for workload k, drawing the tensors in declaration order.
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# The Commands.

ADD_F32 = [
    ("x", ("load", "f32", 1)),
    ("y", ("load", "f32", 1)),
    ("z", ("add", "x", "y")),
    ("out", ("store", "z", 1)),
]

INT_FUSED = [
    ("x", ("load", "i32", 1)),
    ("y", ("load", "i32", 1)),
    ("w", ("load", "i32", 1)),
    ("s", ("scalar", "i32")),
    ("a", ("add", "x", "y")),
    ("m", ("mul", "a", "w")),
    ("z", ("sub", "m", "s")),
    ("out", ("store", "z", 1)),
]

AXPBY_F32 = [
    ("x", ("load", "f32", 1)),
    ("y", ("load", "f32", 1)),
    ("alpha", ("scalar", "f32")),
    ("beta", ("scalar", "f32")),
    ("ax", ("mul", "alpha", "x")),
    ("by", ("mul", "beta", "y")),
    ("r", ("add", "ax", "by")),
    ("out", ("store", "r", 1)),
]

MIXED_TWO_OUT = [
    ("x", ("load", "f16", 1)),
    ("y", ("load", "f16", 1)),
    ("z", ("load", "f16", 1)),
    ("s", ("scalar", "f32")),
    ("xf", ("cvt", "x", "f32")),
    ("yf", ("cvt", "y", "f32")),
    ("zf", ("cvt", "z", "f32")),
    ("t", ("mul", "xf", "yf")),
    ("u", ("add", "t", "zf")),
    ("v", ("sub", "t", "zf")),
    ("uv", ("mul", "u", "v")),
    ("o0", ("cvt", "uv", "f16")),
    ("o1", ("add", "u", "s")),
    ("out0", ("store", "o0", 1)),
    ("out1", ("store", "o1", 1)),
]

TRANSPOSED_2D = [
    ("X", ("load", "f32", 2)),
    ("Yt", ("load", "f32", 2)),
    ("alpha", ("scalar", "f32")),
    ("ay", ("mul", "alpha", "Yt")),
    ("o", ("add", "X", "ay")),
    ("out", ("store", "o", 2)),
]

COPY_F32 = [
    ("x", ("load", "f32", 1)),
    ("out", ("store", "x", 1)),
]

# The threshold classifier of the Silk AMDGPU page's example kernels: an
# unsigned comparison of every element against a scalar threshold.
CLASSIFY_U32 = [
    ("x", ("load", "i32", 1)),
    ("t", ("scalar", "i32")),
    ("r", ("gtu", "x", "t")),
    ("out", ("store", "r", 1)),
]

# A fill: one scalar stored to every element.
FILL_F32 = [
    ("s", ("scalar", "f32")),
    ("out", ("store", "s", 1)),
]

# Native binary16 / bfloat16 arithmetic: out = alpha*x + beta*y computed in
# the 16-bit format itself (each operation rounded once to it).
AXPBY_F16 = [
    ("x", ("load", "f16", 1)),
    ("y", ("load", "f16", 1)),
    ("alpha", ("scalar", "f16")),
    ("beta", ("scalar", "f16")),
    ("ax", ("mul", "alpha", "x")),
    ("by", ("mul", "beta", "y")),
    ("r", ("add", "ax", "by")),
    ("out", ("store", "r", 1)),
]
AXPBY_BF16 = [(n, (st[0], "bf16") + st[2:]) if st[0] in ("load", "scalar") else (n, st) for n, st in AXPBY_F16]

# A fused bias + ReLU, out = max(x*s + y, 0): a Command with no ahead-of-time
# kernel, for the interpreter and the run-time compiled kernel.
BIAS_RELU_F32 = [
    ("x", ("load", "f32", 1)),
    ("y", ("load", "f32", 1)),
    ("s", ("scalar", "f32")),
    ("zero", ("scalar", "f32")),
    ("xs", ("mul", "x", "s")),
    ("u", ("add", "xs", "y")),
    ("r", ("max", "u", "zero")),
    ("out", ("store", "r", 1)),
]

# The transposed configuration's views with a Command the tiled path has no
# ahead-of-time kernel for: out[i,j] = max(X[i,j] + alpha*Y[j,i], 0).
TRANSPOSED_RELU = TRANSPOSED_2D[:3] + [
    ("zero", ("scalar", "f32")),
    ("ay", ("mul", "alpha", "Yt")),
    ("o", ("add", "X", "ay")),
    ("r", ("max", "o", "zero")),
    ("out", ("store", "r", 2)),
]

# Views of rank 3 and 4.  A batch of transposed planes: out[b] = X[b] + alpha * Y[b]^T.
BATCHED_TRANSPOSE = [
    ("X", ("load", "f32", 3)),
    ("Yt", ("load", "f32", 3)),
    ("alpha", ("scalar", "f32")),
    ("ay", ("mul", "alpha", "Yt")),
    ("o", ("add", "X", "ay")),
    ("out", ("store", "o", 3)),
]

# A per-channel affine map over an NCHW activation: scale and bias hold one
# value per channel and are read through stride-0 (broadcast) views.
BIAS_NCHW = [
    ("x", ("load", "f32", 4)),
    ("scale", ("load", "f32", 4)),
    ("bias", ("load", "f32", 4)),
    ("xs", ("mul", "x", "scale")),
    ("o", ("add", "xs", "bias")),
    ("out", ("store", "o", 4)),
]

# The same map in binary16 (scale and bias binary16 too; every operation
# rounds to binary16).
BIAS_NCHW_F16 = [
    ("x", ("load", "f16", 4)),
    ("scale", ("load", "f16", 4)),
    ("bias", ("load", "f16", 4)),
    ("xs", ("mul", "x", "scale")),
    ("o", ("add", "xs", "bias")),
    ("out", ("store", "o", 4)),
]

# The transposed add in binary16 (every operation rounds to binary16).
TRANSPOSED_2D_F16 = [
    ("X", ("load", "f16", 2)),
    ("Yt", ("load", "f16", 2)),
    ("alpha", ("scalar", "f16")),
    ("ay", ("mul", "alpha", "Yt")),
    ("o", ("add", "X", "ay")),
    ("out", ("store", "o", 2)),
]

# z = x + y over rank-2 views (the gather path's workloads below).
ADD2_F32 = [
    ("x", ("load", "f32", 2)),
    ("y", ("load", "f32", 2)),
    ("z", ("add", "x", "y")),
    ("out", ("store", "z", 2)),
]

WORKLOADS = {
    "add_f32": dict(index=0, spec=ADD_F32, n=65536,
                    label="z = x + y, fp32, n=65536 contiguous"),
    "int_fused": dict(index=1, spec=INT_FUSED, n=1 << 24,
                      label="z = (x + y) * w - s, int32, n=2^24, s=12345"),
    "axpby_f32": dict(index=2, spec=AXPBY_F32, n=1 << 28,
                      label="out = alpha*x + beta*y, fp32, n=2^28, alpha=1.5, beta=-0.25"),
    "mixed_two_out": dict(index=3, spec=MIXED_TWO_OUT, n=1 << 27,
                          label="fp16 x,y,z -> out0=fp16(u*v), out1=u+s, t=x*y shared, n=2^27"),
    "transposed_2d": dict(index=4, spec=TRANSPOSED_2D, n=16384,
                          label="out[i,j] = X[i,j] + alpha*Y[j,i], fp32 16384x16384, X row stride 16448"),
    # Not one of the five configurations: a plain copy of known size, the
    # bandwidth reference and the calibration kernel for the HBM counters.
    "copy_f32": dict(index=5, spec=COPY_F32, n=1 << 28,
                     label="out = x, fp32, n=2^28 (plain copy reference)"),
    # Further Commands of the widened op set (compare/select, fill).
    "classify_u32": dict(index=6, spec=CLASSIFY_U32, n=1 << 28,
                         label="out = (x >u t) ? 1 : 0, int32 x uniform over all 2^32 patterns, t = 2^31, n=2^28"),
    "fill_f32": dict(index=7, spec=FILL_F32, n=1 << 28, label="out = s, fp32, s = 1.25, n=2^28"),
    # Rank-3 and rank-4 views.  ``shape`` is the logical shape; ``varies``
    # lists, for each broadcast load, the dimensions its storage spans.
    "batched_transpose": dict(index=8, spec=BATCHED_TRANSPOSE, shape=(64, 2048, 2048),
                              label="out[b,i,j] = X[b,i,j] + alpha*Y[b,j,i], fp32, 64 x 2048 x 2048, alpha=2"),
    "bias_nchw": dict(index=9, spec=BIAS_NCHW, shape=(32, 256, 128, 256), varies={"scale": (1,), "bias": (1,)},
                      label="out = x*scale[c] + bias[c], fp32 NCHW 32 x 256 x 128 x 256, per-channel broadcast"),
    # Native 16-bit arithmetic.
    "axpby_f16": dict(index=10, spec=AXPBY_F16, n=1 << 28,
                      label="out = alpha*x + beta*y in binary16, n=2^28, alpha=1.5, beta=-0.25"),
    "axpby_bf16": dict(index=11, spec=AXPBY_BF16, n=1 << 28,
                       label="out = alpha*x + beta*y in bfloat16, n=2^28, alpha=1.5, beta=-0.25"),
    # No ahead-of-time kernel: interpreter, or compiled at run time.
    "bias_relu_f32": dict(index=12, spec=BIAS_RELU_F32, n=1 << 28,
                          label="out = max(x*s + y, 0), fp32, n=2^28, s=0.5 (no ahead-of-time kernel)"),
    "transposed_relu": dict(index=13, spec=TRANSPOSED_RELU, n=16384,
                            label="out[i,j] = max(X[i,j] + alpha*Y[j,i], 0), fp32 16384x16384, X row stride 16448 "
                                  "(no ahead-of-time kernel)"),
    # Views no vector path takes (the gather path): rows 4 bytes off 16-byte
    # alignment, and rows shorter than a wavefront's elements.
    "odd_rows_f32": dict(index=14, spec=ADD2_F32, shape=(8192, 8191),
                         label="out = x + y, fp32 8192 x 8191, x a column slice of 8192-wide rows, "
                               "y and out contiguous (rows start 4 bytes off 16-byte alignment)"),
    "narrow_rows_f32": dict(index=15, spec=ADD2_F32, shape=(1 << 23, 6),
                            label="out = x + y, fp32 2^23 x 6, x in rows of 8 (row stride 8), y and out contiguous"),
    "bias_nchw_f16": dict(index=16, spec=BIAS_NCHW_F16, shape=(32, 256, 128, 256), varies={"scale": (1,), "bias": (1,)},
                          label="out = x*scale[c] + bias[c], binary16 NCHW 32 x 256 x 128 x 256, per-channel broadcast"),
    "transposed_2d_f16": dict(index=17, spec=TRANSPOSED_2D_F16, n=16384,
                              label="out[i,j] = X[i,j] + alpha*Y[j,i], binary16 16384x16384, X row stride 16448, "
                                    "alpha=2"),
}
CONFIGS = ["add_f32", "int_fused", "axpby_f32", "mixed_two_out", "transposed_2d"]

SCALARS = {
    "int_fused": {"s": np.int32(12345)},
    "axpby_f32": {"alpha": np.float32(1.5), "beta": np.float32(-0.25)},
    "mixed_two_out": {"s": np.float32(0.5)},
    "transposed_2d": {"alpha": np.float32(2.0)},
    "transposed_2d_f16": {"alpha": np.float16(2.0)},
    "transposed_relu": {"alpha": np.float32(2.0), "zero": np.float32(0.0)},
    "classify_u32": {"t": np.int32(-2**31)},          # 0x80000000 as unsigned
    "fill_f32": {"s": np.float32(1.25)},
    "batched_transpose": {"alpha": np.float32(2.0)},
    "axpby_f16": {"alpha": np.float16(1.5), "beta": np.float16(-0.25)},
    "bias_relu_f32": {"s": np.float32(0.5), "zero": np.float32(0.0)},
    # bfloat16 values are uint16 bit patterns: 1.5 = 0x3fc0, -0.25 = 0xbe80
    "axpby_bf16": {"alpha": np.uint16(0x3FC0), "beta": np.uint16(0xBE80)},
}


def shape_of(workload: str, n: int | None = None, shape=None) -> tuple:
    """Logical shape: ``shape`` (or the workload's) for the rank-3/4 workloads,
    (n, n) for the 2-D one, (n,) otherwise."""
    w = WORKLOADS[workload]
    if "shape" in w:
        return tuple(w["shape"] if shape is None else shape)
    n = w["n"] if n is None else n
    return (n, n) if workload in ("transposed_2d", "transposed_relu", "transposed_2d_f16") else (n,)


def layout(view: np.ndarray, storage: np.ndarray):
    """(element offset, element strides) of ``view`` inside the contiguous
    ``storage`` it was cut from, for rebuilding the same view over a device
    copy of the storage."""
    isz = storage.itemsize
    off = view.__array_interface__["data"][0] - storage.__array_interface__["data"][0]
    assert storage.flags.c_contiguous and off % isz == 0 and off >= 0
    strides = tuple(st // isz for st in view.strides)
    assert all(st * isz == b for st, b in zip(strides, view.strides))
    span = off // isz + sum((sz - 1) * st for sz, st in zip(view.shape, strides)) if view.size else 0
    assert span < storage.size or view.size == 0
    return off // isz, strides


def seed_of(workload: str) -> int:
    return 1000 + WORKLOADS[workload]["index"]


def arg_names(spec, outputs: bool = False):
    """Names of the input (or output) CommandArguments in declaration order."""
    if outputs:
        return [name for name, st in spec if st[0] == "store"]
    return [name for name, st in spec if st[0] in ("load", "scalar")]


def _uniform_pm1_f32(rng, shape):
    # rng.random(float32) is k * 2^-24 on [0, 1); *2 - 1 is exact in binary32.
    return rng.random(shape, dtype=np.float32) * np.float32(2) - np.float32(1)


def _uniform_pm4_f16(rng, n):
    a = (rng.random(n, dtype=np.float32) * np.float32(8) - np.float32(4)).astype(np.float16)
    bits = a.view(np.uint16)
    bits[bits == 0x4400] = 0x43FF        # +4.0 after rounding -> largest fp16 below 4
    return a


def make_inputs(workload: str, n: int | None = None, seed: int | None = None,
                row_pad: int = 64, shape=None):
    """Host inputs for one workload, in declaration order.

    Returns ``(values, extra)``: ``values`` is the list of input argument values
    (numpy arrays for loads, numpy scalars for scalars); for the 2-D workload,
    ``values[0]`` is the X *view* (a slice of a padded row-major storage whose
    padding is NaN) and ``values[1]`` is the transposed view ``Y.T`` of a
    contiguous Y; ``extra`` holds the backing storages.  ``n`` overrides the
    length (the 2-D side length for the 2-D workload) and ``shape`` the shape
    of the rank-3/4 workloads.  ``extra["storage"]`` lists, per input value,
    the contiguous array a view was cut from (the value itself when it is
    contiguous, None for scalars); ``layout`` gives the view inside it.
    bfloat16 tensors are uint16 arrays of bit patterns, bfloat16 scalars
    numpy.uint16 bit patterns.
    """
    w = WORKLOADS[workload]
    n = w.get("n") if n is None else n
    rng = np.random.default_rng(seed_of(workload) if seed is None else seed)
    sc = SCALARS.get(workload, {})
    extra = {}
    if workload == "add_f32":
        vals = [_uniform_pm1_f32(rng, n), _uniform_pm1_f32(rng, n)]
    elif workload == "int_fused":
        vals = [rng.integers(-32768, 32768, n, dtype=np.int32) for _ in range(3)]
        vals.append(sc["s"])
    elif workload == "axpby_f32":
        vals = [rng.standard_normal(n, dtype=np.float32), rng.standard_normal(n, dtype=np.float32)]
        vals += [sc["alpha"], sc["beta"]]
    elif workload == "mixed_two_out":
        vals = [_uniform_pm4_f16(rng, n) for _ in range(3)]
        vals.append(sc["s"])
    elif workload == "axpby_f16":
        vals = [rng.standard_normal(n, dtype=np.float32).astype(np.float16) for _ in range(2)]
        vals += [sc["alpha"], sc["beta"]]
    elif workload == "axpby_bf16":
        # bfloat16 bit patterns: the upper half of binary32 normal draws
        vals = [(rng.standard_normal(n, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
                for _ in range(2)]
        vals += [sc["alpha"], sc["beta"]]
    elif workload == "bias_relu_f32":
        vals = [rng.standard_normal(n, dtype=np.float32), rng.standard_normal(n, dtype=np.float32)]
        vals += [sc["s"], sc["zero"]]
    elif workload == "copy_f32":
        vals = [_uniform_pm1_f32(rng, n)]
    elif workload == "classify_u32":
        vals = [rng.integers(0, 2**32, n, dtype=np.uint64).astype(np.uint32).view(np.int32), sc["t"]]
    elif workload == "fill_f32":
        vals = [sc["s"]]
    elif workload in ("transposed_2d", "transposed_relu", "transposed_2d_f16"):
        rows = cols = n
        xs = np.full((rows, cols + row_pad), np.nan, dtype=np.float32)
        xs[:, :cols] = _uniform_pm1_f32(rng, (rows, cols))
        y = _uniform_pm1_f32(rng, (cols, rows))
        if workload == "transposed_2d_f16":
            xs, y = xs.astype(np.float16), y.astype(np.float16)
        vals = [xs[:, :cols], y.T, sc["alpha"]] + ([sc["zero"]] if workload == "transposed_relu" else [])
        extra = {"X_storage": xs, "Y": y, "storage": [xs, y] + [None] * (len(vals) - 2)}
        return vals, extra
    elif workload == "batched_transpose":
        b, r, c = shape_of(workload, shape=shape)
        x = _uniform_pm1_f32(rng, (b, r, c))
        y = _uniform_pm1_f32(rng, (b, c, r))
        extra = {"storage": [x, y, None]}
        return [x, y.transpose(0, 2, 1), sc["alpha"]], extra
    elif workload in ("bias_nchw", "bias_nchw_f16"):
        shp = shape_of(workload, shape=shape)
        x = _uniform_pm1_f32(rng, shp)
        scale = rng.standard_normal(shp[1], dtype=np.float32)
        bias = rng.standard_normal(shp[1], dtype=np.float32)
        if workload == "bias_nchw_f16":
            x, scale, bias = x.astype(np.float16), scale.astype(np.float16), bias.astype(np.float16)
        per_channel = lambda v: np.broadcast_to(v.reshape(1, -1, 1, 1), shp)
        extra = {"storage": [x, scale, bias]}
        return [x, per_channel(scale), per_channel(bias)], extra
    elif workload in ("odd_rows_f32", "narrow_rows_f32"):
        r, c = shape_of(workload, shape=shape)
        xs = np.full((r, c + (1 if workload == "odd_rows_f32" else 2)), np.nan, dtype=np.float32)
        xs[:, :c] = _uniform_pm1_f32(rng, (r, c))
        y = _uniform_pm1_f32(rng, (r, c))
        extra = {"storage": [xs, y]}
        return [xs[:, :c], y], extra
    else:
        raise KeyError(workload)
    extra["storage"] = [v if isinstance(v, np.ndarray) else None for v in vals]
    return vals, extra


def algorithmic_read_write(workload: str, n: int | None = None, shape=None):
    """(bytes read, bytes written) by one launch: every tensor's distinct
    elements x its element size, summed over the loads and over the stores --
    logical elements for ordinary views, the stored elements for broadcast
    loads; row padding and scalars are not counted."""
    w = WORKLOADS[workload]
    shp = shape_of(workload, n, shape)
    elems = int(np.prod(shp, dtype=np.int64))
    varies = w.get("varies", {})
    size = {"f16": 2, "bf16": 2, "f32": 4, "i32": 4}
    dt = {}
    rd = wr = 0
    for name, st in w["spec"]:
        if st[0] == "load":
            dt[name] = st[1]
            if name in varies:
                rd += size[st[1]] * int(np.prod([shp[d] for d in varies[name]], dtype=np.int64))
            else:
                rd += size[st[1]] * elems
        elif st[0] == "scalar":
            dt[name] = st[1]
        elif st[0] in ("add", "sub", "mul", "neg", "abs", "min", "max"):
            dt[name] = dt[st[1]]
        elif st[0] in ("eq", "ne", "lt", "le", "gt", "ge", "ltu", "leu", "gtu", "geu"):
            dt[name] = "i32"
        elif st[0] == "select":
            dt[name] = dt[st[2]]
        elif st[0] == "cvt":
            dt[name] = st[2]
        elif st[0] == "store":
            wr += size[dt[st[1]]] * elems
    return rd, wr


def algorithmic_bytes(workload: str, n: int | None = None, shape=None) -> int:
    """Bytes read + bytes written by one launch (see algorithmic_read_write)."""
    return sum(algorithmic_read_write(workload, n, shape))


def elements(workload: str, n: int | None = None, shape=None) -> int:
    return int(np.prod(shape_of(workload, n, shape), dtype=np.int64))


def to_torch(vals, extra, device):
    """The input values as torch tensors on ``device``: each storage is copied
    once and every view is rebuilt over the copy with the same offset and
    strides (broadcast views keep their stride 0).  Scalars pass through."""
    import torch
    out = []
    for v, st in zip(vals, extra["storage"]):
        if st is None:
            out.append(v)
            continue
        off, strides = layout(v, st)
        flat = np.ascontiguousarray(st).reshape(-1)
        if flat.dtype == np.uint16:          # bfloat16 bit patterns
            flat = torch.from_numpy(flat.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            flat = torch.from_numpy(flat).to(device)
        out.append(flat.as_strided(v.shape, strides, off))
    return out
