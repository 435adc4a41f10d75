"""Launches captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library allocates nothing, keeps no pointer after a launch and puts all
its work on the caller's stream, so launches can be captured.  Captured here:
a specialised linear kernel, the linear interpreter, a run-time compiled
kernel, the tiled kernel (X + 2 Y^T) and the rows interpreter.  The graph is
replayed several times with eager work on the inputs and synchronisations in
between, and every replay is compared bit for bit with eager launches of the
same Commands on the same inputs (no memset or library reduction is captured).
"""
import pytest
import torch

import workloads as W
from gpu_util import compare, dev, host

pytestmark = pytest.mark.gpu


def _commands():
    import elementwise_tensor_commands_amd as ecmd
    n, R, C = (1 << 20) + 77, 320, 192
    g = torch.Generator(device=dev()).manual_seed(77)
    x = torch.randn(n, device=dev(), generator=g)
    y = torch.randn(n, device=dev(), generator=g)
    X = torch.randn(R, C, device=dev(), generator=g)
    Yt = torch.randn(C, R, device=dev(), generator=g)
    P = torch.randn(R, C + 4, device=dev(), generator=g)        # padded rows
    b = torch.randn(R, 1, device=dev(), generator=g)
    relu = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)), ("s", ("scalar", "f32")),
            ("z", ("scalar", "f32")), ("t", ("mul", "x", "s")), ("u", ("add", "t", "y")),
            ("r", ("max", "u", "z")), ("o", ("store", "r", 1))]
    rows = [("p", ("load", "f32", 2)), ("b", ("load", "f32", 2)), ("z", ("scalar", "f32")),
            ("u", ("add", "p", "b")), ("r", ("min", "u", "z")), ("o", ("store", "r", 2))]
    jit = ecmd.from_spec(relu).jit()
    cases = [
        (ecmd.from_spec(W.AXPBY_F32), [x, y, 1.5, -0.25], (n,), "linear_axpby_f32"),
        (ecmd.from_spec(relu), [x, y, 0.5, 0.0], (n,), "linear_generic"),
        (jit, [y, x, -0.5, 0.25], (n,), "jit_linear"),
        (ecmd.from_spec(W.TRANSPOSED_2D), [X, Yt.t(), 2.0], (R, C), "tiled_add_scaled_f32"),
        (ecmd.from_spec(rows), [P[:, :C], b.expand(R, C), 0.75], (R, C), "rows_generic"),
    ]
    for cmd, vals, shape, kernel in cases:
        out = torch.empty(shape, device=dev())
        assert cmd.plan(*vals, out)["kernel"] == kernel
        if cmd is jit:
            cmd.prepare(*vals, out)                 # compile before the capture
    return (x, y, X, Yt, P, b), cases


def test_graph_capture_and_replay():
    inputs, cases = _commands()
    outs = [torch.full(shape, float("nan"), device=dev()) for _, _, shape, _ in cases]
    refs = [torch.empty(shape, device=dev()) for _, _, shape, _ in cases]
    # eager warm-up on a side stream, as graph capture expects
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for (cmd, vals, _, _), o in zip(cases, outs):
            cmd.launch(*vals, o)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for (cmd, vals, _, _), o in zip(cases, outs):
            cmd.launch(*vals, o)
    for rep in range(4):
        for t in inputs:                            # eager work between replays
            t.mul_(1.0625).add_(0.125 * (rep + 1))
        torch.cuda.synchronize()
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for (cmd, vals, _, _), r in zip(cases, refs):
            cmd.launch(*vals, r)
        torch.cuda.synchronize()
        for (_, _, _, kernel), o, r in zip(cases, outs, refs):
            compare(host(o), host(r), 0, "replay %d %s" % (rep, kernel))


def test_graph_of_many_small_launches():
    """The launch-bound 65,536-element add, 200 launches in one graph: every
    output of a replay equals the eager launch's."""
    import elementwise_tensor_commands_amd as ecmd
    vals, _ = W.make_inputs("add_f32", 1 << 16)
    x, y = (torch.from_numpy(v).to(dev()) for v in vals)
    cmd = ecmd.from_spec(W.ADD_F32)
    outs = [torch.empty(1 << 16, device=dev()) for _ in range(200)]
    cmd.launch(x, y, outs[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k, o in enumerate(outs):
            cmd.launch(x if k % 2 == 0 else y, y, o)
    for rep in range(3):
        x.add_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = torch.empty(1 << 16, device=dev())
        for k, o in enumerate(outs):
            cmd.launch(x if k % 2 == 0 else y, y, ref)
            torch.cuda.synchronize()
            compare(host(o), host(ref), 0, "replay %d graph launch %d" % (rep, k))


def test_graph_of_split_dispatches(monkeypatch):
    """Launches the host splits into several dispatches (the linear
    interpreter with ECMD_INTERP_DISPATCH=4, the gather interpreter with
    ECMD_GATHER_DISPATCH=3) captured in one graph: every replay equals the
    eager launches bit for bit."""
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_INTERP_DISPATCH", "4")
    monkeypatch.setenv("ECMD_GATHER_DISPATCH", "3")
    g = torch.Generator(device=dev()).manual_seed(5)
    n = 37 * 1024 + 11
    x = torch.randn(n, device=dev(), generator=g)
    y = torch.randn(n, device=dev(), generator=g)
    P = torch.randn(300, 513, device=dev(), generator=g)          # rows 4 bytes off 16-byte alignment
    Q = torch.randn(300, 512, device=dev(), generator=g)
    relu = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)), ("z", ("scalar", "f32")),
            ("u", ("sub", "x", "y")), ("r", ("max", "u", "z")), ("o", ("store", "r", 1))]
    add2 = [("p", ("load", "f32", 2)), ("q", ("load", "f32", 2)), ("u", ("add", "p", "q")), ("o", ("store", "u", 2))]
    cases = [(ecmd.from_spec(relu), [x, y, 0.0], (n,), "linear_generic", 4),
             (ecmd.from_spec(add2), [P[:, 1:], Q], (300, 512), "gather_whole_rows", 3)]
    outs = [torch.full(shape, float("nan"), device=dev()) for _, _, shape, _, _ in cases]
    for (cmd, vals, _, kernel, grid), o in zip(cases, outs):
        plan = cmd.plan(*vals, o)
        assert plan["kernel"] == kernel and plan["grid"] == grid, plan
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for (cmd, vals, _, _, _), o in zip(cases, outs):
            cmd.launch(*vals, o)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for (cmd, vals, _, _, _), o in zip(cases, outs):
            cmd.launch(*vals, o)
    refs = [torch.empty_like(o) for o in outs]
    for rep in range(3):
        for t in (x, y, P, Q):
            t.mul_(0.875).add_(0.25 * (rep + 1))
        torch.cuda.synchronize()
        for o in outs:
            o.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        for (cmd, vals, _, _, _), r in zip(cases, refs):
            cmd.launch(*vals, r)
        torch.cuda.synchronize()
        for (_, _, _, kernel, _), o, r in zip(cases, outs, refs):
            compare(host(o), host(r), 0, "replay %d %s" % (rep, kernel))
