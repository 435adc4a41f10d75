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
