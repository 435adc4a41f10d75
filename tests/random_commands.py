"""Random valid Commands and inputs (test inputs only; no arithmetic)."""
import numpy as np


def _random_spec(rng, n_in, n_ops, rank):
    spec, dts, names = [], {}, []
    for i in range(n_in):
        dt = rng.choice(["f16", "bf16", "f32", "i32"])
        spec.append(("in%d" % i, ("load", dt, rank)))
        dts["in%d" % i] = dt
        names.append("in%d" % i)
    for i in range(rng.integers(0, 3)):
        dt = rng.choice(["f32", "i32", "f16", "bf16"])
        spec.append(("s%d" % i, ("scalar", dt)))
        dts["s%d" % i] = dt
        names.append("s%d" % i)
    for i in range(n_ops):
        a = names[rng.integers(len(names))]
        kind = rng.choice(["add", "sub", "mul", "neg", "cvt", "cvt", "min", "max", "abs", "cmp", "select"])
        nm = "t%d" % i
        if kind == "cmp":
            same = [x for x in names if dts[x] == dts[a]]
            b = same[rng.integers(len(same))]
            how = rng.choice(["eq", "ne", "lt", "le", "gt", "ge"] + (["ltu", "leu", "gtu", "geu"] if dts[a] == "i32" else []))
            spec.append((nm, (how, a, b)))
            dts[nm] = "i32"
            names.append(nm)
            continue
        if kind == "select":
            conds = [x for x in names if dts[x] == "i32"]
            if conds:
                cnd = conds[rng.integers(len(conds))]
                same = [x for x in names if dts[x] == dts[a]]
                b = same[rng.integers(len(same))]
                spec.append((nm, ("select", cnd, a, b)))
                dts[nm] = dts[a]
                names.append(nm)
                continue
            kind = "neg"
        if kind == "abs":
            kind = "neg" if rng.random() < 0.3 else "abs"
            spec.append((nm, (kind, a)))
            dts[nm] = dts[a]
            names.append(nm)
            continue
        if kind in ("add", "sub", "mul", "min", "max"):
            same = [x for x in names if dts[x] == dts[a]]
            b = same[rng.integers(len(same))]
            spec.append((nm, (kind, a, b)))
            dts[nm] = dts[a]
        elif kind == "neg":
            spec.append((nm, ("neg", a)))
            dts[nm] = dts[a]
        else:
            to = rng.choice(["f16", "bf16", "f32", "i32"])
            spec.append((nm, ("cvt", a, to)))
            dts[nm] = to
        names.append(nm)
    vals = [x for x in names if not x.startswith("s")]
    for k in range(rng.integers(1, 4)):
        v = vals[-1 - k] if k < len(vals) else vals[0]
        spec.append(("o%d" % k, ("store", v, rank)))
    return spec


def _random_inputs(rng, spec, shape):
    out = []
    for _, st in spec:
        if st[0] == "load":
            if st[1] == "i32":
                out.append(rng.integers(-2**31, 2**31, shape, dtype=np.int64).astype(np.int32))
            else:
                b = rng.integers(0, 2**32, shape, dtype=np.uint64).astype(np.uint32)
                f = b.view(np.float32)
                f = np.where(rng.random(shape) < 0.5, rng.standard_normal(shape).astype(np.float32) * 100, f)
                if st[1] == "bf16":          # bfloat16 bit patterns: the upper halves of the draws
                    out.append((f.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
                else:
                    out.append(f.astype(np.float16) if st[1] == "f16" else f.astype(np.float32))
        elif st[0] == "scalar":
            out.append(random_scalar(rng, st[1]))
    return out


def random_scalar(rng, dt):
    """A scalar CommandArgument value (bfloat16: a numpy.uint16 bit pattern)."""
    if dt == "i32":
        return np.int32(rng.integers(-1000, 1000))
    f = np.float32(rng.standard_normal() * 4)
    if dt == "f16":
        return np.float16(f)
    if dt == "bf16":
        return np.uint16(int(np.array(f).view(np.uint32)) >> 16)
    return f


def random_view(rng, storage_fill, shape, dtype, broadcast=False, align=False, permute=True):
    """A random view of logical ``shape`` cut from a fresh contiguous storage:
    the storage holds the dimensions in a random order, each padded and
    started at a random offset; broadcast views also get stride 0 along a
    random subset of dimensions.  ``align`` keeps offsets at multiples of 4
    elements and pads every storage dimension to a multiple of 4.  Returns (view, storage); ``storage_fill(shape)``
    makes the storage's contents."""
    from numpy.lib.stride_tricks import as_strided
    r = len(shape)
    perm = rng.permutation(r) if permute else np.arange(r)   # storage dimension i holds logical dimension perm[i]
    step = 4 if align else 1
    starts = [int(rng.choice([0, 0, 1])) * step for _ in range(r)]
    pads = [int(rng.choice([0, 0, 1, 3])) * step for _ in range(r)]
    if align:                                  # padded storage dimensions of whole vectors
        pads = [(-(shape[p] + starts[i])) % 4 + p_ for i, (p, p_) in enumerate(zip(perm, pads))]
    st_shape = tuple(shape[p] + starts[i] + pads[i] for i, p in enumerate(perm))
    storage = np.ascontiguousarray(storage_fill(st_shape).astype(dtype))
    v = storage[tuple(slice(starts[i], starts[i] + shape[p]) for i, p in enumerate(perm))]
    v = v.transpose(np.argsort(perm))
    if broadcast:
        zero = rng.random(r) < 0.35
        strides = tuple(0 if z else s for z, s in zip(zero, v.strides))
        v = as_strided(v, shape=v.shape, strides=strides, writeable=False)
    return v, storage


_NPD = {"f16": np.float16, "bf16": np.uint16, "f32": np.float32, "i32": np.int32}


def _arg_dtypes(spec):
    """Input argument dtypes (loads and scalars) and output dtypes, in order."""
    dts, ins, outs = {}, [], []
    for name, st in spec:
        if st[0] in ("load", "scalar"):
            dts[name] = st[1]
            ins.append(st[1])
        elif st[0] == "cvt":
            dts[name] = st[2]
        elif st[0] == "select":
            dts[name] = dts[st[2]]
        elif st[0] in ("eq", "ne", "lt", "le", "gt", "ge", "ltu", "leu", "gtu", "geu"):
            dts[name] = "i32"
        elif st[0] == "store":
            outs.append(dts[st[1]])
        else:
            dts[name] = dts[st[1]]
    return ins, outs


def _fill_for(rng, dt):
    if dt == "i32":
        return lambda sh: rng.integers(-2**31, 2**31, sh, dtype=np.int64).astype(np.int32)

    def f(sh):
        b = rng.integers(0, 2**32, sh, dtype=np.uint64).astype(np.uint32).view(np.float32)
        v = np.where(rng.random(sh) < 0.5, rng.standard_normal(sh).astype(np.float32) * 100, b)
        if dt == "bf16":            # bfloat16 bit patterns: the upper halves
            return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
        return v
    return f


SIZES = [1, 2, 3, 4, 5, 8, 12, 16, 33, 64, 68, 100, 132, 260]


def random_view_case(seed, staged=False):
    """A random Command of random rank over random views (inputs only).
    ``staged``: rank 2 to 4, aligned, no broadcasts and outputs in logical
    order, so that inputs stored in another order need a transpose."""
    rng = np.random.default_rng((9000 if staged else 5000) + seed)
    r = int(rng.integers(2 if staged else 1, 5))
    while True:
        shape = tuple(int(rng.choice(SIZES)) for _ in range(r))
        if np.prod(shape) <= 300_000:
            break
    spec = _random_spec(rng, int(rng.integers(1, 4)), int(rng.integers(1, 7)), r)
    in_dt, out_dt = _arg_dtypes(spec)
    align = staged or rng.random() < 0.6
    ins = []
    for (_, st), dt in zip([s for s in spec if s[1][0] in ("load", "scalar")], in_dt):
        if st[0] == "scalar":
            ins.append(random_scalar(rng, dt))
        else:
            ins.append(random_view(rng, _fill_for(rng, dt), shape, _NPD[dt], broadcast=not staged, align=align))
    outs = [random_view(rng, _fill_for(rng, dt), shape, _NPD[dt], align=align, permute=not staged)
            for dt in out_dt]
    return spec, ins, outs
