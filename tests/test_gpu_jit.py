"""Kernels compiled at run time for programs without an ahead-of-time kernel,
against the oracle: random Commands on the linear path, random views on the
rows path, and the bias + ReLU workload up to full size."""
import os

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, dev, host, run_oracle, to_dev
from random_commands import _random_inputs, _random_spec, random_view_case
from specs import arg_dtypes
from test_gpu_views import run_views

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _jit_cache(tmp_path_factory, monkeypatch):
    monkeypatch.setenv("ECMD_CACHE_DIR", str(tmp_path_factory.getbasetemp() / "jit-cache"))
    monkeypatch.setenv("ECMD_JIT", "1")          # every Command built in these tests compiles


@pytest.mark.parametrize("seed", range(30))
def test_random_commands_compiled(seed):
    import elementwise_tensor_commands_amd as ecmd
    rng = np.random.default_rng(9100 + seed)
    spec = _random_spec(rng, int(rng.integers(1, 5)), int(rng.integers(1, 12)), 1)
    n = int(rng.integers(1, 70000))
    vals = _random_inputs(rng, spec, (n,))
    try:
        ref = run_oracle(spec, vals)
    except Exception as e:
        pytest.skip("not a valid Command: %s" % e)
    gv = [to_dev(v) if isinstance(v, np.ndarray) else
          (v if v.dtype == np.uint16 else float(v) if v.dtype.kind == "f" else int(v)) for v in vals]
    _, outs = arg_dtypes(spec)
    cmd = ecmd.from_spec(spec)
    got = [torch.empty(n, dtype={"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32,
                                 "i32": torch.int32}[d], device=dev()) for d in outs]
    try:
        plan = cmd.plan(*gv, *got)
    except ecmd.Error as e:
        assert e.name == "CMD_E_LIMIT", e
        pytest.skip(str(e))
    print("    seed %d: %s" % (seed, plan["kernel"]), flush=True)
    cmd.launch(*gv, *got)
    torch.cuda.synchronize()
    for k, (g, r) in enumerate(zip(got, ref)):
        compare(host(g), r, 0, "compiled seed %d out%d %s\n%s" % (seed, k, plan["kernel"], cmd.dump()))


@pytest.mark.parametrize("seed", range(20))
def test_random_views_compiled(seed):
    spec, ins, outs = random_view_case(seed)
    run_views(spec, ins, outs, False, "compiled seed %d" % seed)


@pytest.mark.parametrize("n", [1, 1000, (1 << 20) + 7, 1 << 28])
def test_bias_relu_compiled_and_interpreted(n, monkeypatch):
    import elementwise_tensor_commands_amd as ecmd
    if n == 1 << 28:
        print("  full size bias_relu_f32", flush=True)
    vals, extra = W.make_inputs("bias_relu_f32", n)
    ref = run_oracle(W.BIAS_RELU_F32, vals)[0]
    gv = W.to_torch(vals, extra, dev())
    for jit in (True, False):
        cmd = ecmd.from_spec(W.BIAS_RELU_F32).jit(jit)
        out = torch.empty(n, device=dev())
        plan = cmd.plan(*gv, out)
        assert plan["compiled"] == jit
        cmd.launch(*gv, out)
        cmd.launch(*gv, out)                     # the second launch finds the kernel in memory
        torch.cuda.synchronize()
        compare(host(out), ref, 0, "bias_relu n=%d %s" % (n, plan["kernel"]))


@pytest.mark.parametrize("seed", range(20))
def test_random_transposed_views_compiled(seed):
    """Random Commands over transposed views: the tiled kernel compiled at run
    time for each (inputs staged through LDS with the compile-time mask)."""
    spec, ins, outs = random_view_case(seed + 300, staged=True)
    run_views(spec, ins, outs, False, "compiled tiled seed %d" % seed)


@pytest.mark.parametrize("n", [200, 1000, 16384])
def test_transposed_relu_compiled_and_interpreted(n):
    """max(X + 2 Y^T, 0) on the transposed configuration's views (row-padded
    X, Y read transposed), compiled and on the tiled interpreter, up to the
    full 16384 x 16384."""
    import elementwise_tensor_commands_amd as ecmd
    if n == 16384:
        print("  full size transposed_relu", flush=True)
    vals, extra = W.make_inputs("transposed_relu", n)
    ref = run_oracle(W.TRANSPOSED_RELU, vals)[0]
    gv = W.to_torch(vals, extra, dev())
    for jit in (True, False):
        cmd = ecmd.from_spec(W.TRANSPOSED_RELU).jit(jit)
        out = torch.empty((n, n), device=dev())
        plan = cmd.plan(*gv, out)
        assert plan["compiled"] == jit and plan["kernel"] == ("jit_tiled" if jit else "tiled_generic"), plan
        cmd.launch(*gv, out)
        torch.cuda.synchronize()
        compare(host(out), ref, 0, "transposed_relu n=%d %s" % (n, plan["kernel"]))


def _unique_spec(k):
    """A program no other test compiles (compiled kernels stay in the
    process's memory): out = min(x * s - y, t) + k-th constant chain."""
    spec = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)), ("s", ("scalar", "f32")),
            ("t", ("scalar", "f32")), ("p", ("mul", "x", "s")), ("q", ("sub", "p", "y"))]
    last = "q"
    for j in range(k):
        spec.append(("a%d" % j, ("abs", last)))
        last = "a%d" % j
    spec += [("r", ("min", last, "t")), ("o", ("store", "r", 1))]
    return spec


def _background_case(tmp_path, monkeypatch, k, n):
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_CACHE_DIR", str(tmp_path / "bg-cache"))
    monkeypatch.setenv("ECMD_JIT", "2")
    spec = _unique_spec(k)
    rng = np.random.default_rng(500 + k)
    x, y = rng.standard_normal(n, dtype=np.float32), rng.standard_normal(n, dtype=np.float32)
    ref = run_oracle(spec, [x, y, np.float32(0.75), np.float32(0.5)])[0]
    out = torch.empty(n, device=dev())
    args = [to_dev(x), to_dev(y), 0.75, 0.5, out]
    cmd = ecmd.from_spec(spec)
    assert cmd.plan(*args)["kernel"] == "linear_generic"
    return cmd, args, out, ref


def _wait_compiled(cmd, args, limit_s=120):
    import time
    t0 = time.time()
    while not cmd.plan(*args)["compiled"]:
        assert time.time() - t0 < limit_s, "the background compile did not finish in %d s" % limit_s
        time.sleep(0.05)


def test_background_compile_switches_kernels(tmp_path, monkeypatch, capfd):
    """Default mode: the first launch of a program with no ahead-of-time
    kernel runs the interpreter while a worker thread compiles; once the
    compile is done, the next launch with the same argument values switches
    to the compiled kernel.  Both results equal the oracle."""
    n = (1 << 20) + 7
    cmd, args, out, ref = _background_case(tmp_path, monkeypatch, 1, n)
    monkeypatch.setenv("ECMD_DUMP_TAPE", "1")
    bound = cmd.bind(*args)
    bound.launch()
    torch.cuda.synchronize()
    compare(host(out), ref, 0, "interpreter while compiling")
    _wait_compiled(cmd, args)
    out.zero_()
    bound.launch()
    torch.cuda.synchronize()
    compare(host(out), ref, 0, "compiled after the switch")
    err = capfd.readouterr().err
    assert "linear_generic" in err and "compiled kernel ready: jit_linear replaces linear_generic" in err, err


def test_background_compile_and_graph_capture(tmp_path, monkeypatch):
    """A launch captured while its kernel compiles records the interpreter
    (no module is loaded during capture); replays stay correct after the
    compile ends, and eager launches then use the compiled kernel."""
    n = (1 << 18) + 3
    cmd, args, out, ref = _background_case(tmp_path, monkeypatch, 2, n)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        cmd.bind(*args).launch()
    for _ in range(2):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        compare(host(out), ref, 0, "replay while compiling")
    _wait_compiled(cmd, args)
    for _ in range(2):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        compare(host(out), ref, 0, "replay after the compile")
    out.zero_()
    cmd.launch(*args)
    torch.cuda.synchronize()
    compare(host(out), ref, 0, "eager, compiled")
    assert cmd.plan(*args)["kernel"] == "jit_linear"
