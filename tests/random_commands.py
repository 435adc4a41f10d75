"""Random valid Commands and inputs (test inputs only; no arithmetic)."""
import numpy as np


def _random_spec(rng, n_in, n_ops, rank):
    spec, dts, names = [], {}, []
    for i in range(n_in):
        dt = rng.choice(["f16", "f32", "i32"])
        spec.append(("in%d" % i, ("load", dt, rank)))
        dts["in%d" % i] = dt
        names.append("in%d" % i)
    for i in range(rng.integers(0, 3)):
        dt = rng.choice(["f32", "i32"])
        spec.append(("s%d" % i, ("scalar", dt)))
        dts["s%d" % i] = dt
        names.append("s%d" % i)
    for i in range(n_ops):
        a = names[rng.integers(len(names))]
        kind = rng.choice(["add", "sub", "mul", "neg", "cvt", "cvt", "min", "max", "abs", "cmp", "select"])
        nm = "t%d" % i
        if kind == "cmp":
            if dts[a] == "f16":
                kind = "cvt"
            else:
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
            if dts[a] == "f16":
                spec.append((nm, ("cvt", a, "f32")))
                dts[nm] = "f32"
            else:
                same = [x for x in names if dts[x] == dts[a]]
                b = same[rng.integers(len(same))]
                spec.append((nm, (kind, a, b)))
                dts[nm] = dts[a]
        elif kind == "neg":
            spec.append((nm, ("neg", a)))
            dts[nm] = dts[a]
        else:
            to = rng.choice(["f16", "f32", "i32"])
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
                out.append(f.astype(np.float16) if st[1] == "f16" else f.astype(np.float32))
        elif st[0] == "scalar":
            out.append(np.float32(rng.standard_normal()) if st[1] == "f32" else np.int32(rng.integers(-1000, 1000)))
    return out
