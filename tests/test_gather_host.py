"""Host-side selection of the gather path (CPU only, no launch).

plan() names the gather interpreter's mode and gives its grid: one work-group
per super-chunk of 256 K elements (K = elems_per_thread / 4).  The grid is
checked by walking the kernel's element positions on the host (segments:
super-chunk w is columns 256 K seg .. of row w / segs; whole rows: super-chunk
w is rows w m .. w m + m - 1, m = floor(256 K / n3)): every element of the
view is reached exactly once.  Extents of 2^31 and more keep the per-element
kernel.
"""
import numpy as np
import pytest
import torch

import elementwise_tensor_commands_amd as E

ADD2 = [("x", ("load", "f32", 2)), ("y", ("load", "f32", 2)), ("r", ("add", "x", "y")), ("o", ("store", "r", 2))]


def _cover(rows, n3, span, kernel, grid):
    """Elements reached by the positions of `grid` super-chunks, each once."""
    seen = np.zeros((rows, n3), np.int32)
    lanes = np.arange(span)
    if kernel == "gather_segments":
        segs = -(-n3 // span)
        assert grid == rows * segs
        for w in range(grid):
            q, seg = divmod(w, segs)
            c = seg * span + lanes
            c = c[c < n3]
            np.add.at(seen, (np.full(c.size, q), c), 1)
    else:
        m = span // n3
        assert m >= 1 and grid == -(-rows // m)
        for w in range(grid):
            count = min(m, rows - w * m) * n3
            p = lanes[lanes < count]
            np.add.at(seen, (w * m + p // n3, p % n3), 1)
    return seen


@pytest.mark.parametrize("k", [1, 2, 4])
@pytest.mark.parametrize("rows,n3", [(37, 2100), (5, 1025), (3, 257), (300, 6), (77, 1), (19, 200), (2, 129),
                                     (1000, 128), (8, 513)])
def test_gather_grid_reaches_every_element_once(monkeypatch, k, rows, n3):
    monkeypatch.setenv("ECMD_INTERP_K", str(k))
    x = torch.zeros(rows, n3 + 1)[:, :n3]          # rows 4 (n3 + 1) bytes apart: no vector path
    plan = E.from_spec(ADD2).plan(x, torch.zeros(rows, n3), torch.zeros(rows, n3))
    assert plan["path"] == "gather" and plan["block"] == 64, plan
    assert plan["elems_per_thread"] == 4 * k and plan["lds_bytes"] == 2 * k * 1024, plan   # x, y; z takes x's entry
    span = 256 * k
    assert plan["kernel"] == ("gather_segments" if n3 > span // 2 else "gather_whole_rows"), plan
    seen = _cover(rows, n3, span, plan["kernel"], plan["grid"])
    assert (seen == 1).all()


def test_flat_views_off_16_bytes_take_gather_segments():
    b = torch.zeros(4097)
    add1 = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)), ("r", ("add", "x", "y")), ("o", ("store", "r", 1))]
    plan = E.from_spec(add1).plan(b[1:], b[:4096], torch.zeros(4096))
    # x, y in two entries of four sub-chunks (K = 4): super-chunks of 1024 elements
    assert plan["path"] == "gather" and plan["kernel"] == "gather_segments" and plan["grid"] == 4, plan
    assert plan["elems_per_thread"] == 16 and plan["lds_bytes"] == 2 * 4 * 1024, plan


def test_per_element_kernel_on_request(monkeypatch):
    monkeypatch.setenv("ECMD_GATHER_MODE", "0")
    x = torch.zeros(10, 33)[:, :32]
    plan = E.from_spec(ADD2).plan(x, torch.zeros(10, 32), torch.zeros(10, 32))
    assert plan["kernel"] == "gather_generic" and plan["block"] == 256 and plan["lds_bytes"] == 0, plan


def test_dispatch_limits_lower_the_planned_grid(monkeypatch):
    """ECMD_GATHER_DISPATCH / ECMD_INTERP_DISPATCH cap the work-groups of one
    dispatch; the host issues as many dispatches as the work needs."""
    x = torch.zeros(100, 1001)[:, :1000]
    c = E.from_spec(ADD2)
    whole = c.plan(x, torch.zeros(100, 1000), torch.zeros(100, 1000))["grid"]
    monkeypatch.setenv("ECMD_GATHER_DISPATCH", "7")
    assert c.plan(x, torch.zeros(100, 1000), torch.zeros(100, 1000))["grid"] == min(7, whole)
    add1 = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 1)), ("m", ("max", "x", "y")), ("o", ("store", "m", 1))]
    n = 50 * 1024
    p = E.from_spec(add1).plan(torch.zeros(n), torch.zeros(n), torch.zeros(n))
    assert p["kernel"] == "linear_generic" and p["grid"] == n // (64 * p["elems_per_thread"]), p
    monkeypatch.setenv("ECMD_INTERP_DISPATCH", "5")
    assert E.from_spec(add1).plan(torch.zeros(n), torch.zeros(n), torch.zeros(n))["grid"] == 5


def test_compiled_gather_grid():
    """A compiled gather kernel (Command.jit()): 64 x 8 elements per wavefront,
    four wavefronts per work-group, no LDS."""
    rows, n3 = 37, 2100
    x = torch.zeros(rows, n3 + 1)[:, :n3]
    p = E.from_spec(ADD2).jit().plan(x, torch.zeros(rows, n3), torch.zeros(rows, n3))
    segs = -(-n3 // 512)
    assert p["kernel"] == "jit_gather" and p["compiled"] and p["block"] == 256 and p["lds_bytes"] == 0, p
    assert p["elems_per_thread"] == 8 and p["grid"] == -(-(rows * segs) // 4), p
