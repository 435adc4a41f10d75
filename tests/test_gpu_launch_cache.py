"""The handle's cache of its last launch: a launch with the same argument
values goes straight to the kernel (no new selection, no new argument
block); new values, or a changed compile option, select again.  The cache
holds the argument values, never the data: new contents at the same
addresses are read by the next launch.  ECMD_DUMP_TAPE=1 prints one line per
selection, which is what these tests count."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import compare, dev, host, run_oracle

pytestmark = pytest.mark.gpu


def _selections(text):
    return sum(1 for line in text.splitlines() if line.startswith("[ecmd] ") and " grid=" in line)


def test_repeat_launch_reuses_the_selection(capfd, monkeypatch):
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_DUMP_TAPE", "1")
    n = (1 << 16) + 3
    x = torch.randn(n, device=dev())
    y = torch.randn(n, device=dev())
    out = torch.empty(n, device=dev())
    cmd = ecmd.from_spec(W.AXPBY_F32)
    capfd.readouterr()
    for _ in range(3):
        cmd.launch(x, y, 1.5, -0.25, out)
    torch.cuda.synchronize()
    assert _selections(capfd.readouterr().err) == 1
    # new contents at the same addresses: read by the next (cached) launch
    x.copy_(torch.randn(n, device=dev()))
    cmd.launch(x, y, 1.5, -0.25, out)
    torch.cuda.synchronize()
    assert _selections(capfd.readouterr().err) == 0
    ref = run_oracle(W.AXPBY_F32, [host(x), host(y), np.float32(1.5), np.float32(-0.25)])[0]
    compare(host(out), ref, 0, "cached launch after new input contents")
    # another scalar value: a new selection; the old value again: another
    cmd.launch(x, y, 2.0, -0.25, out)
    cmd.launch(x, y, 1.5, -0.25, out)
    torch.cuda.synchronize()
    assert _selections(capfd.readouterr().err) == 2
    ref = run_oracle(W.AXPBY_F32, [host(x), host(y), np.float32(1.5), np.float32(-0.25)])[0]
    compare(host(out), ref, 0, "launch after a changed scalar")
    # another view of the same storage: a new selection
    cmd.launch(x[1:], y[1:], 1.5, -0.25, out[1:])
    torch.cuda.synchronize()
    assert _selections(capfd.readouterr().err) == 1


def test_option_change_selects_again(capfd, monkeypatch, tmp_path):
    """cmd_set_option drops the cached launch: the next launch with the same
    values takes the newly allowed kernel."""
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_DUMP_TAPE", "1")
    monkeypatch.setenv("ECMD_CACHE_DIR", str(tmp_path))
    n = 1 << 16
    x = torch.randn(n, device=dev())
    y = torch.randn(n, device=dev())
    out = torch.empty(n, device=dev())
    cmd = ecmd.from_spec(W.AXPBY_F32).jit(ecmd.JIT_OFF)
    capfd.readouterr()
    cmd.launch(x, y, 1.5, -0.25, out)
    cmd.launch(x, y, 1.5, -0.25, out)
    assert _selections(capfd.readouterr().err) == 1
    cmd.aot(False)                                  # interpreter: a new selection
    cmd.launch(x, y, 1.5, -0.25, out)
    err = capfd.readouterr().err
    assert _selections(err) == 1 and "linear_generic" in err, err
    cmd.jit(ecmd.JIT_SYNC)                          # compiled at this launch
    cmd.launch(x, y, 1.5, -0.25, out)
    cmd.launch(x, y, 1.5, -0.25, out)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert _selections(err) == 1 and "jit_linear" in err, err
    ref = run_oracle(W.AXPBY_F32, [host(x), host(y), np.float32(1.5), np.float32(-0.25)])[0]
    compare(host(out), ref, 0, "after option changes")


def test_failed_launch_keeps_no_stale_cache(capfd, monkeypatch):
    """A refused launch (a view of the wrong dtype) leaves the cache as it was:
    the next good launch with the cached values still goes straight to the
    kernel, and the refusal is reported without any GPU work."""
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_DUMP_TAPE", "1")
    n = 4096
    x = torch.randn(n, device=dev())
    y = torch.randn(n, device=dev())
    out = torch.empty(n, device=dev())
    cmd = ecmd.from_spec(W.AXPBY_F32)
    cmd.launch(x, y, 1.5, -0.25, out)
    capfd.readouterr()
    with pytest.raises(ecmd.Error) as e:
        cmd.launch(x.half(), y, 1.5, -0.25, out)
    assert e.value.name == "CMD_E_DTYPE"
    cmd.launch(x, y, 1.5, -0.25, out)
    torch.cuda.synchronize()
    assert _selections(capfd.readouterr().err) == 0
    ref = run_oracle(W.AXPBY_F32, [host(x), host(y), np.float32(1.5), np.float32(-0.25)])[0]
    compare(host(out), ref, 0, "after a refused launch")
