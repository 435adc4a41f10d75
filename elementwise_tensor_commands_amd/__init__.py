"""Python binding for libecmd.so: elementwise tensor Commands on MI355X.

A thin ctypes layer over the C ABI declared in ``include/ecmd.h``; it only
marshals arguments (tensor pointers, sizes and strides, scalar bit patterns,
the current HIP stream).  Every step of the evaluation runs in the library's
gfx950 kernels.  There is no fallback: if the library has not been built, the
import fails.

    import elementwise_tensor_commands_amd as ecmd
    c = ecmd.Command()
    x = c.load("f32"); y = c.load("f32")
    c.store(c.add(x, y))
    c.launch(x_t, y_t, out_t)          # torch tensors on the GPU, declaration order

The Command model is rocRoller's (rocRoller "Design Overview", sections
"Command Class", "Operations", "CommandArgument", "Command Kernel").
"""
from __future__ import annotations

import ctypes
import os
import struct

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libecmd.so")

F16, F32, I32, BF16 = 1, 2, 3, 4
E_ADD, E_SUB, E_MUL, E_NEG, E_CVT = 1, 2, 3, 4, 5
E_CMP = {"eq": 6, "ne": 7, "lt": 8, "le": 9, "gt": 10, "ge": 11, "ltu": 12, "leu": 13, "gtu": 14, "geu": 15}
E_MIN, E_MAX, E_ABS, E_SELECT = 16, 17, 18, 19
ARG_TENSOR, ARG_SCALAR = 1, 2
PATH_NONE, PATH_LINEAR, PATH_TILED, PATH_GATHER, PATH_ROWS = 0, 1, 2, 3, 4
OPT_JIT, OPT_AOT = 1, 2
JIT_OFF, JIT_SYNC, JIT_BACKGROUND = 0, 1, 2
PATH_NAMES = {0: "none", 1: "linear", 2: "tiled", 3: "gather", 4: "rows"}
STATUS = {
    0: "CMD_OK", -1: "CMD_E_ARG", -2: "CMD_E_TAG", -3: "CMD_E_DTYPE", -4: "CMD_E_SHAPE",
    -5: "CMD_E_STRIDE", -6: "CMD_E_ALIAS", -7: "CMD_E_LIMIT", -8: "CMD_E_NOSTORE",
    -9: "CMD_E_STATE", -10: "CMD_E_LAUNCH", -11: "CMD_E_NOMEM",
}
DTYPES = {"f16": F16, "f32": F32, "i32": I32, "bf16": BF16}
DTYPE_NAMES = {F16: "f16", F32: "f32", I32: "i32", BF16: "bf16"}


class Error(RuntimeError):
    """A non-zero status from the C ABI."""

    def __init__(self, code: int, msg: str):
        super().__init__("%s (%d): %s" % (STATUS.get(code, "?"), code, msg))
        self.code = code
        self.name = STATUS.get(code, "?")


class cmd_arg(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32), ("ptr", ctypes.c_void_p),
                ("size", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4),
                ("bits", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class cmd_plan_info(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("specialised", ctypes.c_int32), ("vector", ctypes.c_int32),
                ("elems_per_thread", ctypes.c_int32), ("grid", ctypes.c_int64),
                ("block", ctypes.c_int32), ("lds_bytes", ctypes.c_int32), ("dims", ctypes.c_int32),
                ("compiled", ctypes.c_int32), ("size", ctypes.c_int64 * 4), ("kernel", ctypes.c_char * 64)]


def _load_library():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            "libecmd.so is not built (%s); build it with "
            "`python elementwise_tensor_commands_amd/build.py`" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    vp, i32p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int32)
    sig = {
        "cmd_create": (ctypes.c_int, [ctypes.POINTER(vp)]),
        "cmd_destroy": (ctypes.c_int, [vp]),
        "cmd_load": (ctypes.c_int, [vp, ctypes.c_int32, ctypes.c_int32, i32p, i32p]),
        "cmd_scalar": (ctypes.c_int, [vp, ctypes.c_int32, i32p, i32p]),
        "cmd_op": (ctypes.c_int, [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i32p]),
        "cmd_store": (ctypes.c_int, [vp, ctypes.c_int32, ctypes.c_int32, i32p]),
        "cmd_select": (ctypes.c_int, [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, i32p]),
        "cmd_launch": (ctypes.c_int, [vp, ctypes.POINTER(cmd_arg), ctypes.c_int32, vp]),
        "cmd_launch_timed": (ctypes.c_int, [vp, ctypes.POINTER(cmd_arg), ctypes.c_int32, vp, vp, vp]),
        "cmd_plan": (ctypes.c_int, [vp, ctypes.POINTER(cmd_arg), ctypes.c_int32, ctypes.POINTER(cmd_plan_info)]),
        "cmd_dump": (ctypes.c_int64, [vp, ctypes.c_char_p, ctypes.c_int64]),
        "cmd_last_error": (ctypes.c_char_p, [vp]),
        "cmd_version": (ctypes.c_int32, []),
        "cmd_to_yaml": (ctypes.c_int64, [vp, ctypes.c_char_p, ctypes.c_int64]),
        "cmd_from_yaml": (ctypes.c_int32, [ctypes.c_char_p, ctypes.POINTER(vp)]),
        "cmd_program_yaml": (ctypes.c_int64, [vp, ctypes.c_char_p, ctypes.c_int64]),
        "cmd_program_hash": (ctypes.c_int32, [vp, ctypes.POINTER(ctypes.c_uint64)]),
        "cmd_num_args": (ctypes.c_int32, [vp]),
        "cmd_set_option": (ctypes.c_int32, [vp, ctypes.c_int32, ctypes.c_int64]),
        "cmd_prepare": (ctypes.c_int32, [vp, ctypes.POINTER(cmd_arg), ctypes.c_int32, i32p]),
        "cmd_arg_info": (ctypes.c_int32, [vp, ctypes.c_int32, i32p, i32p, i32p, i32p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


lib = _load_library()

# Raw C entry points under their C names (argument marshalling is the caller's).
cmd_create = lib.cmd_create
cmd_destroy = lib.cmd_destroy
cmd_load = lib.cmd_load
cmd_scalar = lib.cmd_scalar
cmd_op = lib.cmd_op
cmd_store = lib.cmd_store
cmd_select = lib.cmd_select
cmd_launch = lib.cmd_launch
cmd_launch_timed = lib.cmd_launch_timed
cmd_plan = lib.cmd_plan
cmd_dump = lib.cmd_dump
cmd_last_error = lib.cmd_last_error
cmd_version = lib.cmd_version


def _dt(d) -> int:
    return DTYPES[d] if isinstance(d, str) else int(d)


def _torch_dtype_code(t) -> int:
    import torch
    return {torch.float16: F16, torch.float32: F32, torch.int32: I32, torch.bfloat16: BF16}.get(t.dtype, 0)


def scalar_bits(value, dtype: int) -> int:
    """Bit pattern of a scalar CommandArgument value of the declared dtype."""
    if dtype == F32:
        return struct.unpack("<I", struct.pack("<f", float(value)))[0]
    if dtype == I32:
        return int(value) & 0xFFFFFFFF
    if dtype == BF16:
        # a bfloat16 value is given as its bit pattern (numpy.uint16) or as a
        # 0-d torch.bfloat16 tensor; a Python float is rejected rather than
        # rounded here
        if hasattr(value, "dtype") and str(value.dtype) == "uint16":
            return int(value)
        import torch
        if isinstance(value, torch.Tensor) and value.dtype == torch.bfloat16 and value.numel() == 1:
            return int(value.reshape(()).view(torch.int16).item()) & 0xFFFF
        raise TypeError("bfloat16 scalars are numpy.uint16 bit patterns or 0-d torch.bfloat16 tensors")
    return struct.unpack("<H", struct.pack("<e", float(value)))[0]


class Command:
    """One Command.  Tags are ints; CommandArguments are numbered in the order
    load / scalar / store are called."""

    def __init__(self):
        h = ctypes.c_void_p()
        rc = lib.cmd_create(ctypes.byref(h))
        if rc:
            raise Error(rc, lib.cmd_last_error(None).decode())
        self._h = h
        self.arg_kinds: list[tuple[int, int, int]] = []   # (kind, dtype, rank) per argument

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and lib is not None:
            lib.cmd_destroy(h)
            self._h = None

    def _check(self, rc: int):
        if rc:
            raise Error(rc, lib.cmd_last_error(self._h).decode())

    def _arg_decl(self, index: int) -> tuple[int, int, int]:
        kind, dt, rank, out = (ctypes.c_int32() for _ in range(4))
        self._check(lib.cmd_arg_info(self._h, index, ctypes.byref(kind), ctypes.byref(dt), ctypes.byref(rank),
                                     ctypes.byref(out)))
        return kind.value, dt.value, rank.value

    def load(self, dtype, rank: int = 1) -> int:
        tag, arg = ctypes.c_int32(), ctypes.c_int32()
        self._check(lib.cmd_load(self._h, _dt(dtype), rank, ctypes.byref(tag), ctypes.byref(arg)))
        self.arg_kinds.append(self._arg_decl(arg.value))
        return tag.value

    def scalar(self, dtype) -> int:
        tag, arg = ctypes.c_int32(), ctypes.c_int32()
        self._check(lib.cmd_scalar(self._h, _dt(dtype), ctypes.byref(tag), ctypes.byref(arg)))
        self.arg_kinds.append(self._arg_decl(arg.value))
        return tag.value

    def op(self, opcode: int, a: int, b: int = -1, dtype=None) -> int:
        """An E_ operation; dtype None is the default result type (int32 for
        comparisons, the operands' dtype otherwise)."""
        tag = ctypes.c_int32()
        self._check(lib.cmd_op(self._h, opcode, 0 if dtype is None else _dt(dtype), a, b, ctypes.byref(tag)))
        return tag.value

    def add(self, a, b): return self.op(E_ADD, a, b)
    def sub(self, a, b): return self.op(E_SUB, a, b)
    def mul(self, a, b): return self.op(E_MUL, a, b)
    def min(self, a, b): return self.op(E_MIN, a, b)
    def max(self, a, b): return self.op(E_MAX, a, b)
    def neg(self, a): return self.op(E_NEG, a)
    def abs(self, a): return self.op(E_ABS, a)
    def cvt(self, a, dtype): return self.op(E_CVT, a, -1, dtype)

    def cmp(self, how: str, a, b):
        """Comparison how in eq ne lt le gt ge (signed / IEEE) or ltu leu gtu geu
        (int32 as unsigned): an int32 value, 1 or 0."""
        return self.op(E_CMP[how], a, b, I32)

    def select(self, cond, x, y) -> int:
        tag = ctypes.c_int32()
        self._check(lib.cmd_select(self._h, cond, x, y, ctypes.byref(tag)))
        return tag.value

    def store(self, tag: int, rank: int = 1) -> int:
        arg = ctypes.c_int32()
        self._check(lib.cmd_store(self._h, tag, rank, ctypes.byref(arg)))
        self.arg_kinds.append(self._arg_decl(arg.value))
        return arg.value

    # -- run-time compiled kernels ---------------------------------------------
    def jit(self, mode=JIT_SYNC) -> "Command":
        """How a program with no ahead-of-time kernel runs (CMD_OPT_JIT):
        JIT_SYNC (or True) compiles its kernel at the first launch, JIT_BACKGROUND
        (the default) compiles it in a background thread and runs the
        interpreter meanwhile, JIT_OFF (or False) always interprets; returns self."""
        mode = JIT_SYNC if mode is True else JIT_OFF if mode is False else int(mode)
        self._check(lib.cmd_set_option(self._h, OPT_JIT, mode))
        return self

    def aot(self, enable: bool = True) -> "Command":
        """Whether a program on the ahead-of-time list runs its specialised
        kernel (CMD_OPT_AOT); off, it is compiled at run time or interpreted
        like any other program (for comparisons); returns self."""
        self._check(lib.cmd_set_option(self._h, OPT_AOT, 1 if enable else 0))
        return self

    def prepare(self, *values) -> int:
        """Compile (or find) the kernel a launch with these values would use,
        without touching the GPU: -1 none needed, 0 in memory, 1 from disk,
        2 compiled now (cmd_prepare)."""
        arr, n = self._args(values)
        where = ctypes.c_int32()
        self._check(lib.cmd_prepare(self._h, arr, n, ctypes.byref(where)))
        return where.value

    # -- serialisation ---------------------------------------------------------
    def _text(self, fn) -> str:
        n = fn(self._h, None, 0)
        if n < 0:
            self._check(int(n))
        buf = ctypes.create_string_buffer(int(n) + 1)
        fn(self._h, buf, n + 1)
        return buf.value.decode()

    def to_yaml(self) -> str:
        """The Command as a YAML document (cmd_to_yaml)."""
        return self._text(lib.cmd_to_yaml)

    @classmethod
    def from_yaml(cls, text: str) -> "Command":
        """A new Command built from a cmd_to_yaml document (cmd_from_yaml)."""
        h = ctypes.c_void_p()
        rc = lib.cmd_from_yaml(text.encode(), ctypes.byref(h))
        if rc:
            raise Error(rc, lib.cmd_last_error(None).decode())
        obj = cls.__new__(cls)
        obj._h = h
        obj.arg_kinds = [obj._arg_decl(i) for i in range(lib.cmd_num_args(h))]
        return obj

    def program_yaml(self) -> str:
        """The lowered program as YAML (cmd_program_yaml); freezes the Command."""
        return self._text(lib.cmd_program_yaml)

    def program_hash(self) -> int:
        x = ctypes.c_uint64()
        self._check(lib.cmd_program_hash(self._h, ctypes.byref(x)))
        return x.value

    # -- argument marshalling --------------------------------------------------
    def _args(self, values):
        n = len(values)
        arr = (cmd_arg * max(1, n))()
        for i, v in enumerate(values):
            kind, dt, rank = self.arg_kinds[i] if i < len(self.arg_kinds) else (ARG_TENSOR, 0, 1)
            a = arr[i]
            if kind == ARG_SCALAR:
                a.kind, a.dtype, a.bits = ARG_SCALAR, dt, scalar_bits(v, dt)
                continue
            a.kind = ARG_TENSOR
            a.dtype = _torch_dtype_code(v)
            a.ptr = v.data_ptr() if v.numel() > 0 else (v.data_ptr() or None)
            shape, strides = tuple(v.shape), tuple(v.stride())
            for d in range(min(4, len(shape))):
                a.size[d] = shape[d]
                a.stride[d] = strides[d]
            if len(shape) != rank:
                # the C side checks shapes per declared rank; a rank mismatch is an argument error
                for d in range(4):
                    a.size[d] = -1
        return arr, n

    def launch(self, *values, stream=None):
        """Enqueue the Command on ``stream`` (default: torch's current stream)
        with one value per CommandArgument in declaration order: GPU tensors
        for loads and stores, numbers for scalars."""
        arr, n = self._args(values)
        if stream is None:
            import torch
            stream = torch.cuda.current_stream()
        handle = stream if isinstance(stream, int) else getattr(stream, "cuda_stream", stream)
        self._check(lib.cmd_launch(self._h, arr, n, ctypes.c_void_p(handle)))

    def bind(self, *values, stream=None) -> "BoundLaunch":
        """Marshal the argument values once; the returned object launches the
        Command with them in a single C call (for repeated launches)."""
        return BoundLaunch(self, values, stream)

    def plan(self, *values) -> dict:
        """What launch would do with these values (host only, no GPU needed)."""
        arr, n = self._args(values)
        info = cmd_plan_info()
        self._check(lib.cmd_plan(self._h, arr, n, ctypes.byref(info)))
        return {"path": PATH_NAMES[info.path], "specialised": bool(info.specialised),
                "vector": bool(info.vector), "elems_per_thread": info.elems_per_thread,
                "grid": info.grid, "block": info.block, "lds_bytes": info.lds_bytes,
                "dims": info.dims, "size": tuple(info.size), "compiled": bool(info.compiled),
                "kernel": info.kernel.decode()}

    def dump(self) -> str:
        """Text listing of the lowered program (cmd_dump); freezes the Command."""
        return self._text(lib.cmd_dump)


class BoundLaunch:
    """A Command with its argument values marshalled (rocRoller "Design
    Overview", section "Command Kernel": a kernel launched with a prepared
    block of runtime arguments)."""

    def __init__(self, cmd: Command, values, stream=None):
        self.cmd = cmd
        self.values = values                   # keeps the tensors alive
        self.arr, self.n = cmd._args(values)
        if stream is None:
            import torch
            stream = torch.cuda.current_stream()
        handle = stream if isinstance(stream, int) else getattr(stream, "cuda_stream", stream)
        self.stream = ctypes.c_void_p(handle)

    def launch(self):
        rc = lib.cmd_launch(self.cmd._h, self.arr, self.n, self.stream)
        if rc:
            self.cmd._check(rc)

    def launch_timed(self, start, stop):
        """Launch with the kernel execution timed by the dispatches
        (cmd_launch_timed): start and stop are torch.cuda.Event(enable_timing=
        True) objects already recorded once (torch creates events lazily);
        afterwards start.elapsed_time(stop) is the kernel's own duration."""
        rc = lib.cmd_launch_timed(self.cmd._h, self.arr, self.n, self.stream, _event_handle(start),
                                  _event_handle(stop))
        if rc:
            self.cmd._check(rc)


def _event_handle(ev):
    if ev is None:
        return None
    h = getattr(ev, "cuda_event", 0)
    if not h:
        raise ValueError("record the event once before a timed launch (torch creates its events lazily)")
    return ctypes.c_void_p(h)


def from_spec(spec) -> Command:
    """Build a Command from a declarative list of ``(name, step)`` pairs, steps
    being ("load", dtype, rank), ("scalar", dtype), (op, a, b) for add sub mul
    min max and the comparisons, ("neg", a), ("abs", a), ("cvt", a, dtype),
    ("select", cond, x, y) or ("store", value, rank)."""
    c = Command()
    tags = {}
    for name, st in spec:
        k = st[0]
        if k == "load":
            tags[name] = c.load(st[1], st[2] if len(st) > 2 else 1)
        elif k == "scalar":
            tags[name] = c.scalar(st[1])
        elif k == "add":
            tags[name] = c.add(tags[st[1]], tags[st[2]])
        elif k == "sub":
            tags[name] = c.sub(tags[st[1]], tags[st[2]])
        elif k == "mul":
            tags[name] = c.mul(tags[st[1]], tags[st[2]])
        elif k == "min":
            tags[name] = c.min(tags[st[1]], tags[st[2]])
        elif k == "max":
            tags[name] = c.max(tags[st[1]], tags[st[2]])
        elif k in E_CMP:
            tags[name] = c.cmp(k, tags[st[1]], tags[st[2]])
        elif k == "neg":
            tags[name] = c.neg(tags[st[1]])
        elif k == "abs":
            tags[name] = c.abs(tags[st[1]])
        elif k == "select":
            tags[name] = c.select(tags[st[1]], tags[st[2]], tags[st[3]])
        elif k == "cvt":
            tags[name] = c.cvt(tags[st[1]], st[2])
        elif k == "store":
            c.store(tags[st[1]], st[2] if len(st) > 2 else 1)
        else:
            raise ValueError("unknown step %r" % (k,))
    return c


# Placement of the operands of one launch.  On MI355X a streaming Command whose
# operands start at addresses that agree modulo 32 KiB -- as large tensors from
# torch's caching allocator do: it aligns them to 2 MiB -- ran measurably
# slower, with every input's loads issued at once, than the same Command over
# operands whose starts are 4 KiB apart modulo 32 KiB: the axpby 2.4-2.8%
# (binary16: 6%), bias + ReLU 1.7%, the int32 fused Command 1.5%, a copy or the
# classifier 0.7-0.9%; the mixed-precision Command within +-1.3% either way;
# steps of 8 KiB were slower on some machines.  The linear kernel now issues an
# input's loads after the previous input's have returned, which avoids that
# collision in time (the axpby: 497.2 us as torch places it, 498.3 staggered);
# the helper below remains for callers that allocate their own operands and
# for kernels that read their inputs together.
STAGGER_PERIOD = 32768


def empty_staggered(specs, device="cuda", step=4096):
    """Uninitialised contiguous tensors for the operands of one launch, cut
    from one allocation so that their start addresses differ modulo 32 KiB:
    tensor k starts ``(k * step) % 32768`` bytes past a 32 KiB boundary.

    specs: ``(shape, torch dtype)`` pairs; step: a positive multiple of 256
    bytes.  The tensors share one storage, which lives as long as any of them;
    they never overlap.  Plumbing only: no kernel runs."""
    import torch
    step = int(step)
    if step <= 0 or step % 256:
        raise ValueError("step must be a positive multiple of 256 bytes, got %d" % step)
    sizes = []
    for shape, dt in specs:
        n = 1
        for d in shape:
            if int(d) < 0:
                raise ValueError("negative dimension in %r" % (shape,))
            n *= int(d)
        sizes.append(n * torch.empty((), dtype=dt).element_size())
    offsets, end = [], 0
    for k, nbytes in enumerate(sizes):
        start = -(-end // STAGGER_PERIOD) * STAGGER_PERIOD + (k * step) % STAGGER_PERIOD
        offsets.append(start)
        end = start + nbytes
    buf = torch.empty(end + STAGGER_PERIOD, dtype=torch.uint8, device=device)
    base = (-buf.data_ptr()) % STAGGER_PERIOD
    return [buf[base + o:base + o + nbytes].view(dt).view(tuple(int(d) for d in shape))
            for (shape, dt), o, nbytes in zip(specs, offsets, sizes)]
