"""Timed launches (cmd_launch_timed): the results equal an ordinary launch's,
and the events the dispatches record bracket the kernel execution -- a
positive interval no longer than ordinary events recorded around the launch,
covering every dispatch of a launch the host splits."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, dev, host, run_oracle, to_dev

pytestmark = pytest.mark.gpu


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for ev in evs:
        ev.record()
    return evs


@pytest.mark.parametrize("wl", ["axpby_f32", "mixed_two_out", "transposed_2d"])
def test_timed_launch_matches_and_brackets_the_kernel(wl):
    import elementwise_tensor_commands_amd as ecmd
    n = {"transposed_2d": 1000}.get(wl, (1 << 20) + 7)
    vals, extra = W.make_inputs(wl, n)
    ref = run_oracle(W.WORKLOADS[wl]["spec"], vals)
    gv = W.to_torch(vals, extra, dev())
    dts = {"float16": torch.float16, "float32": torch.float32}
    outs = [torch.empty(r.shape, dtype=dts[str(r.dtype)], device=dev()) for r in ref]
    bound = ecmd.from_spec(W.WORKLOADS[wl]["spec"]).bind(*gv, *outs)
    ks, ke, s, e = _events(4)
    torch.cuda.synchronize()
    for _ in range(3):
        for o in outs:
            o.zero_()
        s.record()
        bound.launch_timed(ks, ke)
        e.record()
        e.synchronize()
        kernel_ms, around_ms = ks.elapsed_time(ke), s.elapsed_time(e)
        assert 0 < kernel_ms <= around_ms, (kernel_ms, around_ms)
        for o, r in zip(outs, ref):
            compare(host(o), r, 0, "%s timed" % wl)


def test_timed_launch_of_split_dispatches(monkeypatch):
    """The linear interpreter split into dispatches of 5 work-groups: the
    interval runs from the first dispatch's start to the last one's end, so
    it is at least as long as the untimed sum of a single dispatch would
    suggest and the result is complete."""
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_FORCE_GENERIC", "1")
    monkeypatch.setenv("ECMD_INTERP_DISPATCH", "5")
    n = 64 * 1024 + 13
    rng = np.random.default_rng(3)
    x, y = rng.standard_normal(n, dtype=np.float32), rng.standard_normal(n, dtype=np.float32)
    ref = run_oracle(W.ADD_F32, [x, y])[0]
    out = torch.zeros(n, device=dev())
    cmd = ecmd.from_spec(W.ADD_F32)
    args = [to_dev(x), to_dev(y), out]
    plan = cmd.plan(*args)
    assert plan["kernel"] == "linear_generic" and plan["grid"] == 5
    ks, ke = _events(2)
    torch.cuda.synchronize()
    cmd.bind(*args).launch_timed(ks, ke)
    ke.synchronize()
    assert ks.elapsed_time(ke) > 0
    compare(host(out), ref, 0, "split dispatches, timed")


def test_timed_launch_refused_records_nothing():
    import elementwise_tensor_commands_amd as ecmd
    x = torch.ones(64, device=dev())
    cmd = ecmd.from_spec(W.ADD_F32)
    ks, ke = _events(2)
    bound = cmd.bind(x, torch.ones(65, device=dev()), torch.empty(64, device=dev()))
    with pytest.raises(ecmd.Error) as err:
        bound.launch_timed(ks, ke)
    assert err.value.name == "CMD_E_SHAPE"
