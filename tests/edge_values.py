"""Edge-value inputs for binary32 and int32 operations (inputs only: no
arithmetic here).

``pairs32(dt)`` gives two arrays of bit patterns: every ordered pair of the
special values below, then seeded random 32-bit patterns, so that a sweep over
them puts each edge value in the vector body of a kernel as well as its tail.
"""
import numpy as np

# binary32 bit patterns: signed zeros, subnormals, the normal range's ends,
# values around 1 (ties for add and mul), infinities, quiet and signalling
# NaNs of both signs, the int32 range's ends (saturation of binary32 -> int32
# at +-2^31), 2^24 (the last odd integer), binary16's and bfloat16's rounding
# edges (largest finite 65504, overflow threshold 65520, smallest subnormal
# 2^-24 and half of it, a bfloat16 midpoint).
F32_SPECIAL = [
    0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x007FFFFF, 0x807FFFFF, 0x00400000,
    0x00800000, 0x80800000, 0x00800001,
    0x3F800000, 0xBF800000, 0x3F800001, 0x3F7FFFFF, 0xBF800001, 0xBF7FFFFF,
    0x3F000000, 0xBF000000, 0x40000000, 0x40400000, 0x3FC00000, 0xBFC00000, 0x40200000,
    0x3E800000, 0xBE800000, 0x33800000, 0x34000000,
    0x7F7FFFFF, 0xFF7FFFFF, 0x7F000000, 0x7EFFFFFF,
    0x7F800000, 0xFF800000,
    0x7FC00000, 0xFFC00000, 0x7F800001, 0xFF800001, 0x7FFFFFFF,
    0x4F000000, 0xCF000000, 0x4EFFFFFF, 0xCEFFFFFF, 0x4F000001, 0xCF000001,
    0x4B800000, 0x4B800001, 0xCB800001,
    0x477FE000, 0x477FF000, 0x477FEFFF, 0xC77FF000, 0x33800000, 0x33000000, 0x33000001, 0x38800000,
    0x387FC000, 0x3F808000, 0x3F818000, 0x7F7F8000, 0x00008000,
]

# int32 bit patterns: zero, +-1, the range's ends and their neighbours, the
# 16-bit boundaries, 2^24 and its neighbours (exactness of int32 -> binary32),
# binary16's largest finite and overflow threshold as integers, alternating
# bits, and the int32 fused Command's scalar 12345.
I32_SPECIAL = [
    0x00000000, 0x00000001, 0xFFFFFFFF, 0x00000002, 0xFFFFFFFE, 0x00000003,
    0x7FFFFFFF, 0x80000000, 0x80000001, 0x7FFFFFFE,
    0x00008000, 0xFFFF8000, 0x00007FFF, 0x00010000, 0xFFFF0000, 0x0000FFFF,
    0x01000000, 0x01000001, 0xFEFFFFFF, 0x00FFFFFF, 0x01000003,
    0x0000FFE0, 0x0000FFF0, 0xFFFF0010,
    0x40000000, 0xC0000000, 0x55555555, 0xAAAAAAAA,
    0x00003039, 0xFFFFCFC7,
]


def special(dt):
    return np.array(F32_SPECIAL if dt == "f32" else I32_SPECIAL, dtype=np.uint32)


def pairs32(dt, n_random=1 << 20, seed=91, tail=21):
    """Every ordered pair of special values, then n_random + tail random
    32-bit patterns (the tail keeps the length off every power of two)."""
    sp = special(dt)
    a = np.repeat(sp, sp.size)
    b = np.tile(sp, sp.size)
    rng = np.random.default_rng(seed)
    ra = rng.integers(0, 1 << 32, n_random + tail, dtype=np.uint64).astype(np.uint32)
    rb = rng.integers(0, 1 << 32, n_random + tail, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([a, ra]), np.concatenate([b, rb])


def conditions(n, seed=92):
    """int32 select conditions: 0, 1, -1, INT_MIN and random patterns."""
    rng = np.random.default_rng(seed)
    c = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    c[0::4] = 0
    c[1::8] = 1
    c[3::16] = 0x80000000
    return c
