"""Small Command specs used by the tests (inputs only: no arithmetic here).

Same format as the workload specs in ``workloads.py``; the hand-worked pins in
``tests/golden/hand_worked.txt`` and the invariant tests name these.
"""
import workloads as W


def unary(op, dt_in, dt_out=None):
    if op == "cvt":
        return [("x", ("load", dt_in, 1)), ("r", ("cvt", "x", dt_out)), ("o", ("store", "r", 1))]
    return [("x", ("load", dt_in, 1)), ("r", (op, "x")), ("o", ("store", "r", 1))]


def binary(op, dt):
    return [("x", ("load", dt, 1)), ("y", ("load", dt, 1)), ("r", (op, "x", "y")),
            ("o", ("store", "r", 1))]


def select(dt):
    return [("c", ("load", "i32", 1)), ("x", ("load", dt, 1)), ("y", ("load", dt, 1)),
            ("r", ("select", "c", "x", "y")), ("o", ("store", "r", 1))]


COMPARES = ["eq", "ne", "lt", "le", "gt", "ge"]
UNSIGNED = ["ltu", "leu", "gtu", "geu"]

# The threshold classifier of the Silk AMDGPU page's example kernels: an
# unsigned comparison of every element against a scalar threshold.
CLASSIFY_U32 = [("x", ("load", "i32", 1)), ("t", ("scalar", "i32")), ("r", ("gtu", "x", "t")),
                ("o", ("store", "r", 1))]


SPECS = {
    "add_f32": W.ADD_F32,
    "int_fused": W.INT_FUSED,
    "axpby_f32": W.AXPBY_F32,
    "mixed_two_out": W.MIXED_TWO_OUT,
    "transposed_2d": W.TRANSPOSED_2D,
    "copy_f32": W.COPY_F32,
    "sub_f32": binary("sub", "f32"),
    "mul_f32": binary("mul", "f32"),
    "add_i32": binary("add", "i32"),
    "sub_i32": binary("sub", "i32"),
    "mul_i32": binary("mul", "i32"),
    "neg_f32": unary("neg", "f32"),
    "neg_i32": unary("neg", "i32"),
    "neg_f16": unary("neg", "f16"),
}
DTYPES = ("f16", "bf16", "f32", "i32")
for a in DTYPES:
    for b in DTYPES:
        SPECS["cvt_%s_%s" % (a, b)] = unary("cvt", a, b)
for c in COMPARES:
    for dt in DTYPES:
        SPECS["cmp_%s_%s" % (c, dt)] = binary(c, dt)
for c in UNSIGNED:
    SPECS["cmp_%s_i32" % c] = binary(c, "i32")
for dt in DTYPES:
    SPECS["min_" + dt] = binary("min", dt)
    SPECS["max_" + dt] = binary("max", dt)
    SPECS["abs_" + dt] = unary("abs", dt)
    SPECS["select_" + dt] = select(dt)
# binary16 and bfloat16 arithmetic (native compute types)
for dt in ("f16", "bf16"):
    for op in ("add", "sub", "mul"):
        SPECS["%s_%s" % (op, dt)] = binary(op, dt)
SPECS["neg_bf16"] = unary("neg", "bf16")
SPECS["axpby_f16"] = W.AXPBY_F16
SPECS["axpby_bf16"] = W.AXPBY_BF16
SPECS["classify_u32"] = CLASSIFY_U32

DT = {"f16": "f16", "bf16": "bf16", "f32": "f32", "i32": "i32"}


def arg_dtypes(spec):
    """dtype of each input argument and of each output, in declaration order."""
    dt = {}
    ins, outs = [], []
    for name, st in spec:
        k = st[0]
        if k in ("load", "scalar"):
            dt[name] = st[1]
            ins.append(st[1])
        elif k in ("add", "sub", "mul", "neg", "abs", "min", "max"):
            dt[name] = dt[st[1]]
        elif k in COMPARES or k in UNSIGNED:
            dt[name] = "i32"
        elif k == "select":
            dt[name] = dt[st[2]]
        elif k == "cvt":
            dt[name] = st[2]
        elif k == "store":
            outs.append(dt[st[1]])
    return ins, outs


def input_kinds(spec):
    return [st[0] for _, st in spec if st[0] in ("load", "scalar")]
