"""Helpers for the GPU parity tests: host<->device copies, running a spec on
the GPU library and on the oracle, and element-by-element comparison."""
import os

import numpy as np
import torch

# bfloat16 has no NumPy type: on the host it is a uint16 array of bit patterns
# (every uint16 array in these tests is one), on the device torch.bfloat16.
TD = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32, "i32": torch.int32}
NPD = {"f16": np.float16, "bf16": np.uint16, "f32": np.float32, "i32": np.int32}
BITS = {2: np.uint16, 4: np.uint32}
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


def dev():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch.device("cuda:0")


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev())


def host(t):
    """A device tensor as a NumPy array (bfloat16: uint16 bit patterns)."""
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _nan_mask(a):
    if a.dtype == np.uint16:                 # bfloat16 bit patterns
        return ((a & 0x7F80) == 0x7F80) & ((a & 0x7F) != 0)
    return np.isnan(a)


def bits(a):
    return np.ascontiguousarray(a).view(BITS[a.itemsize])


def ordered(b, width):
    """Map IEEE bit patterns to integers whose difference counts ulps (+0 and -0 both map to 0)."""
    b = b.astype(np.int64)
    sign = 1 << (width - 1)
    return np.where(b & sign, -(b & (sign - 1)), b)


def compare(got, ref, max_ulp=0, what=""):
    """Bitwise equality (NaN equals any NaN), or at most max_ulp ulps per element."""
    got, ref = np.asarray(got), np.asarray(ref)
    assert got.shape == ref.shape and got.dtype == ref.dtype, (got.shape, ref.shape, got.dtype, ref.dtype)
    gb, rb = bits(got).ravel(), bits(ref).ravel()
    if got.dtype.kind == "f" or got.dtype == np.uint16:
        nan_g, nan_r = _nan_mask(got).ravel(), _nan_mask(ref).ravel()
        assert np.array_equal(nan_g, nan_r), "%s: NaN positions differ" % what
        gb, rb = gb[~nan_g], rb[~nan_r]
        if max_ulp:
            d = np.abs(ordered(gb, got.itemsize * 8) - ordered(rb, got.itemsize * 8))
            worst = int(d.max()) if d.size else 0
            assert worst <= max_ulp, "%s: max %d ulp > %d at %s" % (what, worst, max_ulp, np.flatnonzero(d > max_ulp)[:10])
            return worst
    bad = np.flatnonzero(gb != rb)
    if bad.size:
        show = ", ".join("[%d] gpu %#x oracle %#x" % (i, gb[i], rb[i]) for i in bad[:10])
        raise AssertionError("%s: %d of %d elements differ: %s" % (what, bad.size, gb.size, show))
    return 0


def run_gpu(spec, values, out_shapes_dtypes, outputs=None, stream=None):
    """values: device tensors / scalars in declaration order (inputs only)."""
    import elementwise_tensor_commands_amd as ecmd
    cmd = ecmd.from_spec(spec)
    if outputs is None:
        outputs = [torch.empty(s, dtype=TD[d], device=dev()) for s, d in out_shapes_dtypes]
    cmd.launch(*values, *outputs, stream=stream)
    torch.cuda.synchronize()
    return cmd, outputs


def run_oracle(spec, values, outputs=None):
    from oracle import oracle
    return oracle.from_spec(spec).run(*values, outputs=outputs, nthreads=ORACLE_THREADS)
