"""Oracle front end: a plain CPU evaluator of elementwise tensor Commands.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this module.  It shares no code
with the GPU library (``elementwise_tensor_commands_amd``) and never imports it.

The model follows rocRoller's "Design Overview" (sections "Command Class",
"Operations", "CommandArgument"): operations are appended to a Command in
order, each gets a tag, later operations refer to earlier tags, and loads,
scalars and stores allocate CommandArguments whose values are supplied when the
Command is executed, in declaration order.  ``T_Execute`` holds the ``E_``
operations: Add, Sub, Mul, Neg and type conversions (Cvt).

This module does its own checking (earlier tags only, matching dtypes, one
common logical shape) and then hands a flat node list to the C core
``ecmd_oracle.c``, which walks every element in row-major order.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ecmd_oracle.c")
LIB = os.path.join(HERE, "libecmd_oracle.so")

F16, F32, I32, BF16 = 1, 2, 3, 4
DTYPE_CODE = {"f16": F16, "f32": F32, "i32": I32, "bf16": BF16}
# NumPy has no bfloat16: bfloat16 tensors are uint16 arrays of bit patterns,
# bfloat16 scalars uint16 bit patterns.
NP_DTYPE = {F16: np.float16, F32: np.float32, I32: np.int32, BF16: np.uint16}
NP_BITS = {F16: np.uint16, F32: np.uint32, I32: np.uint32, BF16: np.uint16}

LOAD, SCALAR, OP = 1, 2, 3
ADD, SUB, MUL, NEG, CVT = 1, 2, 3, 4, 5
CMP = {"eq": 6, "ne": 7, "lt": 8, "le": 9, "gt": 10, "ge": 11, "ltu": 12, "leu": 13, "gtu": 14, "geu": 15}
MIN, MAX, ABS, SELECT = 16, 17, 18, 19
OP_CODE = {"add": ADD, "sub": SUB, "mul": MUL, "neg": NEG, "cvt": CVT, "min": MIN, "max": MAX,
           "abs": ABS, "select": SELECT, **CMP}

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
             "-Wall", "-Wextra", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile the C core with gcc.  No -march=native: the host's FMA units must
    never be used for binary32 arithmetic, and -ffp-contract=off forbids fusing."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, SRC, "-lm"], check=True)
        os.replace(tmp, LIB)
    return LIB


class _Node(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32), ("op", ctypes.c_int32),
                ("a", ctypes.c_int32), ("b", ctypes.c_int32), ("c", ctypes.c_int32),
                ("arg", ctypes.c_int32)]


class _Store(ctypes.Structure):
    _fields_ = [("tag", ctypes.c_int32), ("arg", ctypes.c_int32)]


class _Arg(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride", ctypes.c_int64 * 4),
                ("bits", ctypes.c_uint32), ("dtype", ctypes.c_int32)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = _load(LIB if os.path.exists(LIB) else build())
    return _lib


def use_library(path):
    """Swap in another build of the C core (the mutation tests plant mistakes
    in copies of it); returns the previously loaded library handle."""
    global _lib
    prev = _lib
    _lib = _load(path) if isinstance(path, str) else path
    return prev


def _load(path):
    L = ctypes.CDLL(path)
    L.oracle_eval.restype = ctypes.c_int
    L.oracle_eval.argtypes = [ctypes.POINTER(_Node), ctypes.c_int, ctypes.POINTER(_Store),
                              ctypes.c_int, ctypes.POINTER(_Arg), ctypes.POINTER(ctypes.c_int64),
                              ctypes.c_int]
    L.oracle_f16_to_f32.restype = ctypes.c_uint32
    L.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_f32_to_f16.restype = ctypes.c_uint16
    L.oracle_f32_to_f16.argtypes = [ctypes.c_uint32]
    L.oracle_f32_to_f16_range.restype = None
    L.oracle_f32_to_f16_range.argtypes = [ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p]
    L.oracle_f16_to_f32_all.restype = None
    L.oracle_f16_to_f32_all.argtypes = [ctypes.c_void_p]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_f32_to_bf16.argtypes = [ctypes.c_uint32]
    L.oracle_bf16_to_f32.restype = ctypes.c_uint32
    L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_f32_to_bf16_range.restype = None
    L.oracle_f32_to_bf16_range.argtypes = [ctypes.c_uint32, ctypes.c_uint64, ctypes.c_void_p]
    L.oracle_check_fpenv.restype = ctypes.c_int
    for name, cls in (("node", _Node), ("store", _Store), ("arg", _Arg)):
        fn = getattr(L, "oracle_sizeof_" + name)
        fn.restype = ctypes.c_int
        assert fn() == ctypes.sizeof(cls), name
    return L


class OracleError(ValueError):
    pass


def _dt(d) -> int:
    if isinstance(d, str):
        return DTYPE_CODE[d]
    return int(d)


class OracleCommand:
    """A Command for the oracle.  Tags are indexes into ``self.nodes``; argument
    indexes count loads, scalars and stores in declaration order."""

    def __init__(self):
        self.nodes: list[tuple] = []      # (kind, dtype, op, a, b, c, arg)
        self.stores: list[tuple] = []     # (tag, arg)
        self.args: list[tuple] = []       # ("tensor"|"scalar", dtype, rank, is_output)

    # -- building ------------------------------------------------------------
    def load(self, dtype, rank: int = 1) -> int:
        dt = _dt(dtype)
        if rank not in (1, 2, 3, 4):
            raise OracleError("rank must be 1 to 4")
        self.args.append(("tensor", dt, rank, False))
        self.nodes.append((LOAD, dt, 0, -1, -1, -1, len(self.args) - 1))
        return len(self.nodes) - 1

    def scalar(self, dtype) -> int:
        dt = _dt(dtype)
        self.args.append(("scalar", dt, 0, False))
        self.nodes.append((SCALAR, dt, 0, -1, -1, -1, len(self.args) - 1))
        return len(self.nodes) - 1

    def _check_tag(self, t):
        if not (0 <= t < len(self.nodes)):
            raise OracleError("tag %r does not name an earlier result" % (t,))

    def op(self, name: str, a: int, b: int | None = None, dtype=None, c: int | None = None) -> int:
        code = OP_CODE[name]
        self._check_tag(a)
        da = self.nodes[a][1]
        if code in (ADD, SUB, MUL, MIN, MAX) or code in CMP.values():
            if b is None:
                raise OracleError("binary op needs two operands")
            self._check_tag(b)
            db = self.nodes[b][1]
            if da != db:
                raise OracleError("operand dtypes differ")
            if code in (CMP["ltu"], CMP["leu"], CMP["gtu"], CMP["geu"]) and da != I32:
                raise OracleError("unsigned comparison needs int32 operands")
            res = I32 if code in CMP.values() else da
        elif code == SELECT:
            if b is None or c is None:
                raise OracleError("select takes a condition and two values")
            self._check_tag(b)
            self._check_tag(c)
            if da != I32:
                raise OracleError("select condition must be int32")
            if self.nodes[b][1] != self.nodes[c][1]:
                raise OracleError("select values differ in dtype")
            res = self.nodes[b][1]
        elif code in (NEG, ABS):
            if b is not None:
                raise OracleError("neg / abs are unary")
            res = da
        else:
            if b is not None or dtype is None:
                raise OracleError("cvt takes one operand and a target dtype")
            res = _dt(dtype)
        if dtype is not None and _dt(dtype) != res:
            raise OracleError("result dtype mismatch")
        self.nodes.append((OP, res, code, a, -1 if b is None else b, -1 if c is None else c, -1))
        return len(self.nodes) - 1

    def add(self, a, b): return self.op("add", a, b)
    def sub(self, a, b): return self.op("sub", a, b)
    def mul(self, a, b): return self.op("mul", a, b)
    def neg(self, a): return self.op("neg", a)
    def abs(self, a): return self.op("abs", a)
    def cvt(self, a, dtype): return self.op("cvt", a, None, dtype)
    def select(self, cond, x, y): return self.op("select", cond, x, None, y)

    def store(self, tag: int, rank: int = 1) -> int:
        self._check_tag(tag)
        if rank not in (1, 2, 3, 4):
            raise OracleError("rank must be 1 to 4")
        self.args.append(("tensor", self.nodes[tag][1], rank, True))
        self.stores.append((tag, len(self.args) - 1))
        return len(self.args) - 1

    # -- running -------------------------------------------------------------
    def run(self, *values, outputs=None, nthreads: int = 1):
        """Evaluate on host data.

        ``values`` holds one entry per *input* argument in declaration order:
        a numpy array (any strides, including views and transposes) for a load
        and a number or a numpy scalar for a scalar.  Outputs are freshly
        allocated contiguous arrays of the common shape unless ``outputs``
        supplies arrays (views allowed) in store order.  Returns the list of
        output arrays.
        """
        in_idx = [k for k, a in enumerate(self.args) if not a[3]]
        out_idx = [k for k, a in enumerate(self.args) if a[3]]
        if len(values) != len(in_idx):
            raise OracleError("expected %d input values, got %d" % (len(in_idx), len(values)))
        shape = None
        keep = []
        cargs = (_Arg * max(1, len(self.args)))()

        def view_of(k, arr):
            nonlocal shape
            kind, dt, rank, _ = self.args[k]
            arr = np.asarray(arr)
            if arr.dtype != np.dtype(NP_DTYPE[dt]):
                raise OracleError("argument %d: dtype %s, declared %s" % (k, arr.dtype, NP_DTYPE[dt]))
            if arr.ndim != rank:
                raise OracleError("argument %d: rank %d, declared %d" % (k, arr.ndim, rank))
            shp = (1,) * (4 - rank) + tuple(arr.shape)          # right-aligned 4-D shape
            if shape is None:
                shape = shp
            elif shape != shp:
                raise OracleError("argument %d: shape %s differs from %s" % (k, shp, shape))
            isz = arr.itemsize
            st = [0] * (4 - rank) + [s_ // isz for s_ in arr.strides]
            cargs[k].ptr = arr.__array_interface__["data"][0]
            for d in range(4):
                cargs[k].stride[d] = st[d]
            cargs[k].dtype = dt
            keep.append(arr)

        for k, v in zip(in_idx, values):
            kind, dt = self.args[k][0], self.args[k][1]
            if kind == "scalar":
                if dt == BF16 and np.asarray(v).dtype != np.uint16:
                    raise OracleError("scalar argument %d: bfloat16 scalars are uint16 bit patterns" % k)
                s = np.asarray(v).astype(NP_DTYPE[dt]) if not isinstance(v, np.ndarray) else v
                if s.dtype != np.dtype(NP_DTYPE[dt]):
                    raise OracleError("scalar argument %d: dtype %s" % (k, s.dtype))
                cargs[k].bits = int(np.asarray(s).reshape(()).view(NP_BITS[dt]))
                cargs[k].dtype = dt
            else:
                view_of(k, v)
        if shape is None and outputs is None:
            raise OracleError("no tensor argument fixes the shape")
        if outputs is None:
            outputs = []
            for k in out_idx:
                rank, dt = self.args[k][2], self.args[k][1]
                if any(d != 1 for d in shape[: 4 - rank]):
                    raise OracleError("rank-%d output for the shape %s" % (rank, shape))
                outputs.append(np.zeros(shape[4 - rank:], dtype=NP_DTYPE[dt]))
        if len(outputs) != len(out_idx):
            raise OracleError("expected %d outputs" % len(out_idx))
        for k, o in zip(out_idx, outputs):
            view_of(k, o)
        nodes = (_Node * max(1, len(self.nodes)))(*[_Node(*n) for n in self.nodes])
        stores = (_Store * max(1, len(self.stores)))(*[_Store(*s) for s in self.stores])
        cshape = (ctypes.c_int64 * 4)(*shape)
        rc = lib().oracle_eval(nodes, len(self.nodes), stores, len(self.stores), cargs, cshape,
                               int(nthreads))
        if rc != 0:
            raise OracleError("host floating-point environment is not IEEE default (code %d)" % rc)
        return list(outputs)


def f16_to_f32_bits(h: int) -> int:
    return int(lib().oracle_f16_to_f32(h))


def f32_to_f16_bits(u: int) -> int:
    return int(lib().oracle_f32_to_f16(u))


def f32_to_f16_range(first: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    lib().oracle_f32_to_f16_range(first, count, out.ctypes.data)
    return out


def f32_to_bf16_range(first: int, count: int) -> np.ndarray:
    out = np.empty(count, dtype=np.uint16)
    lib().oracle_f32_to_bf16_range(first, count, out.ctypes.data)
    return out


def f16_to_f32_all() -> np.ndarray:
    out = np.empty(65536, dtype=np.uint32)
    lib().oracle_f16_to_f32_all(out.ctypes.data)
    return out


def from_spec(spec) -> OracleCommand:
    """Build an OracleCommand from a declarative workload spec: a list of
    (name, step) pairs with steps ("load", dtype, rank), ("scalar", dtype),
    (binary op, a, b) for add sub mul min max and the comparisons, ("neg", a),
    ("abs", a), ("cvt", a, dtype), ("select", cond, x, y), ("store", value,
    rank)."""
    cmd = OracleCommand()
    tags = {}
    for name, step in spec:
        kind = step[0]
        if kind == "load":
            tags[name] = cmd.load(step[1], step[2] if len(step) > 2 else 1)
        elif kind == "scalar":
            tags[name] = cmd.scalar(step[1])
        elif kind in ("add", "sub", "mul", "min", "max") or kind in CMP:
            tags[name] = cmd.op(kind, tags[step[1]], tags[step[2]])
        elif kind in ("neg", "abs"):
            tags[name] = cmd.op(kind, tags[step[1]])
        elif kind == "select":
            tags[name] = cmd.select(tags[step[1]], tags[step[2]], tags[step[3]])
        elif kind == "cvt":
            tags[name] = cmd.cvt(tags[step[1]], step[2])
        elif kind == "store":
            cmd.store(tags[step[1]], step[2] if len(step) > 2 else 1)
        else:
            raise OracleError("unknown step %r" % (kind,))
    return cmd
