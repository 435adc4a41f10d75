"""Separate handles used from separate threads at the same time.

Each thread owns one Command handle and one stream (default priority) and
launches its Command back to back; the binding's C calls release the
interpreter lock, so the launches, the selection of kernels and the
background compilation of the Programs without an ahead-of-time kernel all
overlap.  Every result is compared with the oracle."""
import threading

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, dev, host, run_oracle, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _jit_cache(tmp_path_factory, monkeypatch):
    monkeypatch.setenv("ECMD_CACHE_DIR", str(tmp_path_factory.getbasetemp() / "jit-cache-threads"))


def _cases(rng):
    """(spec, host inputs, output dtypes) of four Commands: two with an
    ahead-of-time kernel, two without (one flat, one transposed)."""
    n = (1 << 20) + 3
    x, y = rng.standard_normal(n).astype(np.float32), rng.standard_normal(n).astype(np.float32)
    relu3 = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)), ("s", ("scalar", "f32")),
             ("m", ("mul", "x", "s")), ("a", ("sub", "m", "y")), ("z", ("scalar", "f32")),
             ("r", ("max", "a", "z")), ("t", ("min", "r", "x")), ("o", ("store", "t", 1))]
    R, C = 300, 520
    X = rng.standard_normal((R, C)).astype(np.float32)
    Y = rng.standard_normal((C, R)).astype(np.float32)
    tspec = [("X", ("load", "f32", 2)), ("Yt", ("load", "f32", 2)), ("p", ("mul", "X", "Yt")),
             ("q", ("sub", "p", "X")), ("o", ("store", "q", 2))]
    return [
        (W.AXPBY_F32, [x, y, np.float32(1.5), np.float32(-0.25)], [(n,)]),
        (W.ADD_F32, [x, y], [(n,)]),
        (relu3, [x, y, np.float32(0.75), np.float32(0.0)], [(n,)]),
        (tspec, [X, Y.T], [(R, C)]),
    ]


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_handles_on_threads(mode):
    """Four threads, four handles, four streams, 40 launches each, JIT mode
    0 / 1 / 2 (interpreter, compile at first launch, compile in the
    background) for the two Commands without an ahead-of-time kernel."""
    import elementwise_tensor_commands_amd as ecmd
    rng = np.random.default_rng(77 + mode)
    cases = _cases(rng)
    refs = [run_oracle(spec, vals) for spec, vals, _ in cases]
    start = threading.Barrier(len(cases))
    errors, outs = [None] * len(cases), [None] * len(cases)

    def work(i):
        try:
            spec, vals, shapes = cases[i]
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                gv = [to_dev(v) if isinstance(v, np.ndarray) else float(v) for v in vals]
                if i == 3:
                    gv[1] = to_dev(np.ascontiguousarray(vals[1].T)).t()     # a transposed view
                got = [torch.empty(s, device=dev()) for s in shapes]
                cmd = ecmd.from_spec(spec).jit(mode)
                stream.synchronize()
                start.wait()
                for _ in range(40):
                    cmd.launch(*gv, *got, stream=stream)
                stream.synchronize()
                outs[i] = (cmd.plan(*gv, *got)["kernel"], [host(g) for g in got])
        except Exception as e:          # reported by the main thread
            errors[i] = e

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a launching thread did not finish"
    for i, e in enumerate(errors):
        assert e is None, "thread %d: %r" % (i, e)
    for i, ((kernel, got), ref) in enumerate(zip(outs, refs)):
        print("    thread %d (mode %d): %s" % (i, mode, kernel), flush=True)
        for k, (g, r) in enumerate(zip(got, ref)):
            compare(g, r, 0, "thread %d mode %d out%d (%s)" % (i, mode, k, kernel))
