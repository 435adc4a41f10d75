"""Run-time compiled kernels on the host: compile without a GPU, the memory
and disk caches, the plan's report, and our own gfx950 code in the code
objects (no fused multiply-add, no scratch, 16-byte accesses; LDS staging
and a barrier in the compiled tiled kernel)."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import elementwise_tensor_commands_amd as E
import workloads as W

LLVM_OBJDUMP = "/opt/rocm/llvm/bin/llvm-objdump"


@pytest.fixture
def cache_dir(tmp_path, monkeypatch):
    d = tmp_path / "jit-cache"
    monkeypatch.setenv("ECMD_CACHE_DIR", str(d))
    return d


def _bias_relu(n=1 << 16, jit=True):
    c = E.from_spec(W.BIAS_RELU_F32)
    if jit:
        c.jit()
    x, y, o = torch.zeros(n), torch.zeros(n), torch.zeros(n)
    return c, [x, y, 0.5, 0.0, o]


def test_plan_reports_the_compiled_kernel(cache_dir):
    c, vals = _bias_relu()
    p = c.plan(*vals)
    assert p["kernel"] == "jit_linear" and p["compiled"] and p["specialised"]
    c2, vals2 = _bias_relu(jit=False)
    p2 = c2.plan(*vals2)
    assert p2["kernel"] == "linear_generic" and not p2["compiled"]
    # programs with an ahead-of-time kernel never compile
    c3 = E.from_spec(W.AXPBY_F32).jit()
    n = 1024
    assert c3.prepare(torch.zeros(n), torch.zeros(n), 1.5, -0.25, torch.zeros(n)) == -1
    assert c3.plan(torch.zeros(n), torch.zeros(n), 1.5, -0.25, torch.zeros(n))["kernel"] == "linear_axpby_f32"


def test_compile_then_memory_then_disk(cache_dir):
    c, vals = _bias_relu()
    assert c.prepare(*vals) == 2                       # compiled
    assert c.prepare(*vals) == 0                       # memory
    files = os.listdir(cache_dir)
    assert len(files) == 1 and files[0].endswith(".ecmdjit")
    same = E.Command.from_yaml(c.to_yaml()).jit()       # another Command, same program
    assert same.prepare(*vals) == 0
    code = ("import sys; sys.path[:0] = [%r]\n"
            "import torch, elementwise_tensor_commands_amd as E, workloads as W\n"
            "c = E.from_spec(W.BIAS_RELU_F32).jit(); n = 1 << 16\n"
            "print('FROM', c.prepare(torch.zeros(n), torch.zeros(n), 0.5, 0.0, torch.zeros(n)))\n"
            % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ECMD_CACHE_DIR=str(cache_dir)))
    assert "FROM 1" in r.stdout, r.stdout + r.stderr    # read from disk in a new process


def test_each_variant_and_program_has_its_own_entry(cache_dir):
    # (the small variant may already sit in this process's memory cache)
    c, vals = _bias_relu(1 << 16)
    compiled = int(c.prepare(*vals) == 2)
    big, bvals = _bias_relu(1 << 28)                    # beyond the last-level cache: nontemporal loads
    assert big.plan(*bvals)["kernel"] == "jit_linear"
    assert big.prepare(*bvals) == 2
    rows = E.from_spec([("x", ("load", "f32", 2)), ("b", ("load", "f32", 2)), ("s", ("scalar", "f32")),
                        ("p", ("mul", "x", "s")), ("q", ("sub", "p", "b")), ("o", ("store", "q", 2))]).jit()
    x = torch.zeros(64, 72)[:, :64]
    bias = torch.zeros(64, 1).expand(64, 64)
    out = torch.zeros(64, 64)
    assert rows.plan(x, bias, 2.0, out)["kernel"] == "jit_rows"
    assert rows.prepare(x, bias, 2.0, out) == 2
    tiled = E.from_spec(TILED_SPEC).jit()
    tv = _tiled_values()
    p = tiled.plan(*tv)
    assert p["kernel"] == "jit_tiled" and p["compiled"] and p["block"] == 512 and p["lds_bytes"] == 32 * 256 * 4, p
    assert tiled.prepare(*tv) == 2
    gather = E.from_spec(GATHER_SPEC).jit()
    gv = _gather_values()
    p = gather.plan(*gv)
    assert p["kernel"] == "jit_gather" and p["compiled"] and p["block"] == 256 and p["lds_bytes"] == 0, p
    assert gather.prepare(*gv) == 2
    assert len(os.listdir(cache_dir)) == 4 + compiled


# out = min(X + Y^T, s) - Y^T: a program the tiled path has no ahead-of-time kernel for
TILED_SPEC = [("X", ("load", "f32", 2)), ("Y", ("load", "f32", 2)), ("s", ("scalar", "f32")),
              ("a", ("add", "X", "Y")), ("m", ("min", "a", "s")), ("d", ("sub", "m", "Y")),
              ("o", ("store", "d", 2))]


def _tiled_values(R=64, C=512):
    return [torch.zeros(R, C), torch.zeros(C, R).t(), 1.0, torch.zeros(R, C)]


# out = max(x - y, x * y) over a strided x: a program and views for the gather path
GATHER_SPEC = [("x", ("load", "f32", 2)), ("y", ("load", "f32", 2)), ("d", ("sub", "x", "y")),
               ("p", ("mul", "x", "y")), ("m", ("max", "d", "p")), ("o", ("store", "m", 2))]


def _gather_values(R=64, C=1000):
    return [torch.zeros(R, 2 * C)[:, ::2], torch.zeros(R, C), torch.zeros(R, C)]


STALE_SPEC = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)), ("p", ("mul", "x", "y")),
              ("q", ("min", "p", "x")), ("o", ("store", "q", 1))]      # used by this test only


def test_stale_cache_file_is_recompiled(cache_dir):
    n = 4096
    c = E.from_spec(STALE_SPEC).jit()
    assert c.prepare(torch.zeros(n), torch.zeros(n), torch.zeros(n)) == 2
    (f,) = [cache_dir / name for name in os.listdir(cache_dir)]
    data = f.read_bytes()
    lines = data.split(b"\n")
    lines[3] = lines[3][:-2] + (b"00" if lines[3][-2:] != b"00" else b"01")   # another program's bytes
    f.write_bytes(b"\n".join(lines))
    code = ("import sys; sys.path[:0] = [%r, %r]\n"
            "import torch, elementwise_tensor_commands_amd as E, test_jit_host as T\n"
            "c = E.from_spec(T.STALE_SPEC).jit(); n = 4096\n"
            "print('FROM', c.prepare(torch.zeros(n), torch.zeros(n), torch.zeros(n)))\n"
            % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))), os.path.dirname(os.path.abspath(__file__))))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120,
                       env=dict(os.environ, ECMD_CACHE_DIR=str(cache_dir)))
    assert "FROM 2" in r.stdout, r.stdout + r.stderr
    assert f.read_bytes() != b"\n".join(lines)          # rewritten


def test_option_errors():
    c = E.Command()
    with pytest.raises(E.Error) as e:
        E.lib.cmd_set_option(c._h, 1, 5) and c._check(E.lib.cmd_set_option(c._h, 1, 5))
    assert e.value.name == "CMD_E_ARG"
    assert E.lib.cmd_set_option(c._h, 99, 0) == -1


def _code_object(path):
    data = path.read_bytes()
    pos = 0
    for _ in range(6):
        pos = data.index(b"\n", pos) + 1
    return data[pos:]


@pytest.mark.parametrize("spec_name", ["bias_relu", "mixed16", "tiled", "gather"])
def test_compiled_code_is_our_rules(cache_dir, tmp_path, spec_name):
    """Disassemble the run-time compiled code objects (built here): no fused
    multiply-add, no scratch, no packed binary32, 16-byte vector accesses."""
    if not os.path.exists(LLVM_OBJDUMP):
        pytest.skip("llvm-objdump not installed")
    if spec_name == "bias_relu":          # max(x*s + y, 0) - y: a program only this test compiles
        spec = W.BIAS_RELU_F32[:-1] + [("d", ("sub", "r", "y")), ("out", ("store", "d", 1))]
        c = E.from_spec(spec).jit()
        n = 1 << 16
        vals = [torch.zeros(n), torch.zeros(n), 0.5, 0.0, torch.zeros(n)]
    elif spec_name == "tiled":            # max instead of min: a program only this test compiles
        spec = [st if st[0] != "m" else ("m", ("max", "a", "s")) for st in TILED_SPEC]
        c = E.from_spec(spec).jit()
        vals = _tiled_values()
    elif spec_name == "gather":           # min instead of max: a program only this test compiles
        spec = [st if st[0] != "m" else ("m", ("min", "d", "p")) for st in GATHER_SPEC]
        c = E.from_spec(spec).jit()
        vals = _gather_values()
    else:
        spec = [("x", ("load", "f16", 1)), ("y", ("load", "bf16", 1)), ("a", ("cvt", "x", "f32")),
                ("b", ("cvt", "y", "f32")), ("m", ("mul", "a", "b")), ("s", ("add", "m", "a")),
                ("o", ("store", "s", 1))]
        c = E.from_spec(spec).jit()
        n = 4096
        vals = [torch.zeros(n, dtype=torch.float16), torch.zeros(n, dtype=torch.bfloat16), torch.zeros(n)]
    assert c.prepare(*vals) == 2
    (f,) = [cache_dir / n for n in os.listdir(cache_dir)]
    co = tmp_path / "k.co"
    co.write_bytes(_code_object(f))
    asm = subprocess.run([LLVM_OBJDUMP, "-d", str(co)], capture_output=True, text=True, check=True).stdout
    # the gather kernel accesses elements one by one, the others 16 bytes per lane
    assert "global_load_dword" in asm and ("global_store_dword" if spec_name == "gather" else "global_store_dwordx4") in asm
    if spec_name == "tiled":
        assert "ds_write" in asm and "ds_read" in asm and "s_barrier" in asm
    for bad in ("v_fma", "v_fmac", "v_pk_fma_f32", "v_pk_mul_f32", "v_pk_add_f32", "scratch_", "v_fma_mix"):
        assert bad not in asm, bad


def test_options_pick_the_kernel_kind(cache_dir, monkeypatch):
    """CMD_OPT_AOT 0 sends an ahead-of-time program to the interpreter or to
    run-time compilation; CMD_OPT_JIT 0 / 1 / 2 (off, at first launch, in the
    background); bad values are refused."""
    n = 4096
    vals = [torch.zeros(n), torch.zeros(n), 1.5, -0.25, torch.zeros(n)]
    assert E.from_spec(W.AXPBY_F32).plan(*vals)["kernel"] == "linear_axpby_f32"
    assert E.from_spec(W.AXPBY_F32).aot(False).jit(E.JIT_OFF).plan(*vals)["kernel"] == "linear_generic"
    c = E.from_spec(W.AXPBY_F32).aot(False).jit(E.JIT_SYNC)
    assert c.plan(*vals)["kernel"] == "jit_linear"
    # background mode: the plan names the interpreter until the kernel exists
    b = E.from_spec(W.AXPBY_F32).aot(False).jit(E.JIT_BACKGROUND)
    assert b.plan(*vals)["kernel"] == "linear_generic"
    assert b.prepare(*vals) == 2
    assert b.plan(*vals)["kernel"] == "jit_linear"
    for opt, bad in ((E.OPT_JIT, 3), (E.OPT_JIT, -1), (E.OPT_AOT, 2), (99, 0)):
        rc = E.lib.cmd_set_option(c._h, opt, bad)
        assert rc == -1 and E.lib.cmd_last_error(c._h)


def test_environment_sets_the_starting_mode(cache_dir, monkeypatch):
    n = 4096
    vals = [torch.zeros(n), torch.zeros(n), 0.5, 0.0, torch.zeros(n)]
    monkeypatch.setenv("ECMD_JIT", "1")
    assert E.from_spec(W.BIAS_RELU_F32).plan(*vals)["kernel"] == "jit_linear"
    monkeypatch.setenv("ECMD_JIT", "0")
    assert E.from_spec(W.BIAS_RELU_F32).plan(*vals)["kernel"] == "linear_generic"
    monkeypatch.delenv("ECMD_JIT")                    # default: background compile
    # a program no other test compiles (the process keeps compiled kernels in memory)
    spec = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)), ("s", ("scalar", "f32")),
            ("t", ("scalar", "f32")), ("p", ("mul", "x", "s")), ("q", ("sub", "p", "y")),
            ("r", ("min", "q", "t")), ("o", ("store", "r", 1))]
    c = E.from_spec(spec)
    assert c.plan(*vals)["kernel"] == "linear_generic"  # not compiled yet (fresh cache directory)
    assert c.prepare(*vals) == 2
    assert c.plan(*vals)["kernel"] == "jit_linear"
