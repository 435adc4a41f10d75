"""GPU parity at the largest sizes: views of more than 2^32 elements, byte
offsets past 2^32, and a linear launch whose work exceeds the 2^31 work-items
one dispatch can count (the kernel loops over the rest).

Inputs are synthetic and deterministic: a multiplicative hash of the element
index, written on the GPU in slices.  The outputs are compared with the
oracle at about a million sampled positions (seeded) plus every boundary that
matters: the first and last elements, the elements after 2^29, 2^30, 2^31 and
2^32 (byte offsets 2^31 and 2^32 for binary32), and the elements on both
sides of 2^33, where the capped grid's first pass ends.
"""
import gc

import numpy as np
import pytest
import torch

from gpu_util import compare, dev, run_oracle
from specs import SPECS

pytestmark = pytest.mark.gpu

SLICE = 1 << 26


def _fill_hash(t, mult, add, f32):
    """t[i] = a hash of the global index i, written slice by slice (bounded
    temporaries).  binary32: an exact value k / 1024 - 512 with k < 2^20."""
    flat = t.view(-1)
    for s in range(0, flat.numel(), SLICE):
        e = min(flat.numel(), s + SLICE)
        h = (torch.arange(s, e, device=t.device, dtype=torch.int64) * mult + add) & 0xFFFFFFFF
        if f32:
            flat[s:e] = ((h >> 12).to(torch.float32) / 1024.0) - 512.0
        else:
            flat[s:e] = torch.where(h >= 2**31, h - 2**32, h).to(torch.int32)


def _sample(total, extra=()):
    rng = np.random.default_rng(20261202)
    idx = [rng.integers(0, total, 1 << 20, dtype=np.int64), np.arange(0, 4096), np.arange(total - 8192, total)]
    for b in (1 << 29, 1 << 30, 1 << 31, 1 << 32, 1 << 33, *extra):
        if b - 4096 < total:
            idx.append(np.arange(max(0, b - 4096), min(total, b + 4096)))
    return np.unique(np.concatenate(idx))


def _add2(dt):
    """The rank-1 add of SPECS with rank-2 views (the oracle checks samples
    with the rank-1 Command: the operation is elementwise)."""
    return [("x", ("load", dt, 2)), ("y", ("load", dt, 2)), ("r", ("add", "x", "y")), ("o", ("store", "r", 2))]


def _release():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,specialised", [("add_f32", True), ("add_i32", False)])
def test_linear_past_the_dispatch_limit(name, specialised):
    """2^33 + 4099 elements.  Specialised kernel: 2^25 + 16 wavefront chunks
    of 256 elements, the grid capped at 2^23 work-groups (2^31 work-items), 3
    elements of tail.  Interpreter: 2^23 + 4 super-chunks of 1024 elements
    (four sub-chunks), one work-group each, 3 elements of tail."""
    import elementwise_tensor_commands_amd as ecmd
    n = (1 << 33) + 4099
    f32 = name == "add_f32"
    dt = torch.float32 if f32 else torch.int32
    print("  max size %s n=%d" % (name, n), flush=True)
    x = torch.empty(n, dtype=dt, device=dev())
    y = torch.empty(n, dtype=dt, device=dev())
    z = torch.full((n,), -1 if not f32 else float("nan"), dtype=dt, device=dev())
    try:
        _fill_hash(x, 0x9E3779B1, 12345, f32)
        _fill_hash(y, 0x85EBCA77, 777, f32)
        cmd = ecmd.from_spec(SPECS[name])
        plan = cmd.plan(x, y, z)
        assert plan["path"] == "linear" and plan["specialised"] == specialised, plan
        if specialised:       # the grid is capped at 2^31 work-items and the kernel loops
            assert plan["grid"] * plan["block"] == 1 << 31, plan
        else:                 # the interpreter: one work-group per super-chunk
            assert plan["grid"] == n // (64 * plan["elems_per_thread"]) and plan["block"] == 64, plan
        cmd.launch(x, y, z)
        torch.cuda.synchronize()
        idx = _sample(n)
        it = torch.from_numpy(idx).to(dev())
        xs, ys, zs = (t[it].cpu().numpy() for t in (x, y, z))
    finally:
        del x, y, z
        _release()
    ref = run_oracle(SPECS[name], [xs, ys])[0]
    compare(zs, ref, 0, "%s n=%d (%s), %d sampled elements" % (name, n, plan["kernel"], idx.size))


def test_padded_rows_past_the_rows_limit():
    """A (2^21, 4096) binary32 add with X in rows padded to 4160 elements: 2^31
    vectors of 4, one more than the rows kernel's dispatch can count, so the view
    goes to the tiled kernel; element offsets reach 2^33 + 2^27."""
    import elementwise_tensor_commands_amd as ecmd
    rows, cols, ld = 1 << 21, 4096, 4160
    print("  max size padded rows %dx%d ld=%d" % (rows, cols, ld), flush=True)
    xs_ = torch.empty((rows, ld), dtype=torch.float32, device=dev())
    y = torch.empty((rows, cols), dtype=torch.float32, device=dev())
    z = torch.full((rows, cols), float("nan"), dtype=torch.float32, device=dev())
    x = None
    try:
        _fill_hash(xs_, 0x9E3779B1, 5, True)
        _fill_hash(y, 0x85EBCA77, 9, True)
        x = xs_[:, :cols]
        cmd = ecmd.from_spec(_add2("f32"))
        plan = cmd.plan(x, y, z)
        assert plan["path"] == "tiled", plan
        cmd.launch(x, y, z)
        torch.cuda.synchronize()
        total = rows * cols
        idx = _sample(total)
        it = torch.from_numpy(idx).to(dev())
        r, c = it // cols, it % cols
        xv, yv, zv = x[r, c].cpu().numpy(), y.view(-1)[it].cpu().numpy(), z.view(-1)[it].cpu().numpy()
    finally:
        del xs_, x, y, z
        _release()
    ref = run_oracle(SPECS["add_f32"], [xv, yv])[0]
    compare(zv, ref, 0, "padded rows (%s), %d sampled elements" % (plan["kernel"], idx.size))


@pytest.mark.parametrize("compiled", [False, True])
def test_gather_past_2pow32_elements(compiled, tmp_path, monkeypatch):
    """(2^20 + 1, 4099) int32 add whose rows start every 4101 elements (not a
    multiple of 4: no vector path applies), 2^32 + 3,149,827 elements, so the
    gather kernel's element index and every offset pass 2^32: the gather
    interpreter, and the kernel compiled at run time (its 64-bit offsets)."""
    import elementwise_tensor_commands_amd as ecmd
    monkeypatch.setenv("ECMD_CACHE_DIR", str(tmp_path))
    rows, cols, ld = (1 << 20) + 1, 4099, 4101
    total = rows * cols
    print("  max size gather %dx%d ld=%d (%d elements)" % (rows, cols, ld, total), flush=True)
    xb = torch.empty((rows, ld), dtype=torch.int32, device=dev())
    yb = torch.empty((rows, ld), dtype=torch.int32, device=dev())
    zb = torch.full((rows, ld), -7, dtype=torch.int32, device=dev())
    x = y = z = None
    try:
        _fill_hash(xb, 0x9E3779B1, 1, False)
        _fill_hash(yb, 0x85EBCA77, 2, False)
        x, y, z = xb[:, :cols], yb[:, :cols], zb[:, :cols]
        cmd = ecmd.from_spec(_add2("i32"))
        if compiled:
            cmd.jit(ecmd.JIT_SYNC)
        plan = cmd.plan(x, y, z)
        assert plan["path"] == "gather" and (plan["kernel"] == "jit_gather") == compiled, plan
        cmd.launch(x, y, z)
        torch.cuda.synchronize()
        idx = _sample(total, extra=(total - (1 << 20),))
        it = torch.from_numpy(idx).to(dev())
        r, c = it // cols, it % cols
        xv, yv, zv = x[r, c].cpu().numpy(), y[r, c].cpu().numpy(), z[r, c].cpu().numpy()
        pad_ok = bool(torch.all(zb[:, cols:] == -7).item())
    finally:
        del xb, yb, zb, x, y, z
        _release()
    assert pad_ok, "the gather kernel wrote into the output's row padding"
    ref = run_oracle(SPECS["add_i32"], [xv, yv])[0]
    compare(zv, ref, 0, "gather (%s), %d sampled elements" % (plan["kernel"], idx.size))
