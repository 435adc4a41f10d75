"""Rank-1 to rank-4 views on the host side: binding (right-aligned shapes,
strides, one-to-one stores, aliasing) and the path the library picks after
dropping size-1 dimensions, ordering by the first output and merging
contiguous dimensions.  No GPU is used: cmd_plan only reads pointers, sizes and
strides (the coordinate-transform model of rocRoller "Design Overview",
section "Kernel Graph": a dimension has a size and a stride)."""
import numpy as np
import pytest
import torch

import elementwise_tensor_commands_amd as E


class FakeTensor:
    """Pointer, shape and strides only: enough for cmd_plan, never read."""

    def __init__(self, shape, strides, dtype=torch.float32, ptr=1 << 32):
        self.shape = tuple(shape)
        self._strides = tuple(strides)
        self.dtype = dtype
        self._ptr = ptr

    def stride(self):
        return self._strides

    def data_ptr(self):
        return self._ptr

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n


def contiguous_strides(shape):
    st, acc = [], 1
    for s in reversed(shape):
        st.append(acc)
        acc *= s
    return tuple(reversed(st))


def T(shape, strides=None, dtype=torch.float32, base=0):
    """A fake tensor whose storage starts at a 4 KiB-aligned address + base elements."""
    global _next
    _next += 1 << 44
    esz = torch.empty((), dtype=dtype).element_size()
    return FakeTensor(shape, contiguous_strides(shape) if strides is None else strides, dtype,
                      _next + base * esz)


_next = 1 << 40


def _err(fn, name):
    with pytest.raises(E.Error) as e:
        fn()
    assert e.value.name == name, str(e.value)


def add_spec(rank):
    return [("x", ("load", "f32", rank)), ("y", ("load", "f32", rank)), ("z", ("add", "x", "y")),
            ("out", ("store", "z", rank))]


def scaled_spec(rank):
    """out = X + alpha * Y (the specialised tiled Program)."""
    return [("X", ("load", "f32", rank)), ("Yt", ("load", "f32", rank)), ("alpha", ("scalar", "f32")),
            ("ay", ("mul", "alpha", "Yt")), ("o", ("add", "X", "ay")), ("out", ("store", "o", rank))]


@pytest.mark.parametrize("shape", [(1155,), (35, 33), (3, 5, 77), (3, 5, 7, 11), (1, 1, 1, 1)])
def test_contiguous_views_of_any_rank_are_linear(shape):
    r = len(shape)
    p = E.from_spec(add_spec(r)).plan(T(shape), T(shape), T(shape))
    n = 1
    for s in shape:
        n *= s
    assert p["path"] == "linear" and p["dims"] == 1 and p["size"] == (1, 1, 1, n), p


def test_size_one_dimensions_are_ignored():
    shape = (1, 64, 1, 64)
    odd = (12345, 64, 999, 1)                  # strides of size-1 dimensions do not matter
    p = E.from_spec(add_spec(4)).plan(T(shape, odd), T(shape), T(shape, (7, 64, 3, 1)))
    assert p["path"] == "linear" and p["size"] == (1, 1, 1, 4096), p


def test_contiguous_dimensions_merge_despite_row_padding_elsewhere():
    # rows padded to 80 elements: dimensions 0 and 1 merge (64 * 80 == 5120), 2 stays
    shape = (4, 64, 64)
    pad = (64 * 80, 80, 1)
    p = E.from_spec(add_spec(3)).plan(T(shape, pad), T(shape, pad), T(shape, pad))
    assert p["path"] == "rows" and p["dims"] == 2 and p["size"] == (1, 1, 256, 64), p
    assert p["specialised"] and p["kernel"] == "rows_add_f32" and p["lds_bytes"] == 0


def test_batched_transpose_is_tiled_and_specialised():
    B, R, C = 3, 64, 128
    yt = T((B, R, C), (R * C, 1, R))                 # Y of shape (B, C, R), transposed per batch
    p = E.from_spec(scaled_spec(3)).plan(T((B, R, C)), yt, 2.0, T((B, R, C)))
    assert p["path"] == "tiled" and p["specialised"] and p["dims"] == 3, p
    assert p["size"] == (1, B, R, C)
    assert p["lds_bytes"] > 0


def test_transposed_dimension_pairs_merge_to_a_plane():
    # Y[a, r, c] at a + 8*(r*32 + c): unit stride along a, and (r, c) jointly contiguous
    A_, R, C = 8, 16, 32
    y = T((A_, R, C), (1, C * A_, A_))
    p = E.from_spec(add_spec(3)).plan(T((A_, R, C)), y, T((A_, R, C)))
    assert p["path"] == "tiled" and p["dims"] == 2 and p["size"] == (1, 1, A_, R * C), p


def test_staged_dimension_is_moved_next_to_the_inner_one():
    # Y[a, r, c] at a + 8*r + 128*c: unit stride along a, nothing merges
    A_, R, C = 8, 16, 32
    y = T((A_, R, C), (1, A_, A_ * R))
    p = E.from_spec(add_spec(3)).plan(T((A_, R, C)), y, T((A_, R, C)))
    assert p["path"] == "tiled" and p["dims"] == 3, p
    assert p["size"] == (1, R, A_, C)               # a becomes the plane's row dimension


def test_output_order_decides_the_inner_dimension():
    # the output is the transpose of a row-major (C, R) array; the input is row-major (R, C)
    R, C = 96, 160
    out = T((R, C), (1, R))
    p = E.from_spec(add_spec(2)).plan(T((R, C)), T((R, C)), out)
    assert p["path"] == "tiled" and p["size"] == (1, 1, C, R), p
    assert p["lds_bytes"] > 0                        # both inputs staged


def test_per_channel_broadcast_nchw_is_row_constant():
    N, C, H, W = 2, 8, 4, 16
    bias = T((N, C, H, W), (0, 1, 0, 0))
    p = E.from_spec(add_spec(4)).plan(T((N, C, H, W)), bias, T((N, C, H, W)))
    assert p["path"] == "rows" and p["specialised"], p
    assert p["dims"] == 3 and p["size"] == (1, N, C, H * W)
    assert p["lds_bytes"] == 0
    # with a transposed input as well, the tiled path reads the bias once per row
    yt = T((N, C, H, W), (C * H * W, H * W, 1, H))
    p = E.from_spec(add_spec(4)).plan(yt, bias, T((N, C, H, W)))
    assert p["path"] == "tiled" and not p["specialised"], p


def test_per_channel_broadcast_nhwc_is_direct():
    N, H, W, C = 2, 4, 16, 8
    scale = T((N, H, W, C), (0, 0, 0, 1))
    p = E.from_spec(add_spec(4)).plan(T((N, H, W, C)), scale, T((N, H, W, C)))
    assert p["path"] == "rows" and p["dims"] == 2 and p["size"] == (1, 1, N * H * W, C), p


def test_broadcast_along_every_dimension_is_one_row():
    shape = (4, 8, 17)
    p = E.from_spec(add_spec(3)).plan(T(shape), T(shape, (0, 0, 0)), T(shape))
    assert p["path"] == "rows" and p["size"] == (1, 1, 1, 4 * 8 * 17), p
    assert p["grid"] == (4 * 8 * 17 // 4 + 1 + 255) // 256


def test_no_vector_alignment_gathers():
    shape = (4, 8, 16)
    p = E.from_spec(add_spec(3)).plan(T(shape), T(shape, (0, 0, 0), base=1), T(shape, (8 * 17, 17, 1)))
    assert p["path"] == "gather", p


def test_misaligned_batch_stride_gathers():
    shape = (3, 8, 16)
    out = T(shape, (8 * 16 + 1, 16, 1))            # planes start one element apart from 16-byte lines
    p = E.from_spec(add_spec(3)).plan(T(shape), T(shape), out)
    assert p["path"] == "gather", p
    ok = T(shape, (8 * 16 + 4, 16, 1))
    assert E.from_spec(add_spec(3)).plan(T(shape), T(shape), ok)["path"] == "rows"


def test_misaligned_base_of_a_staged_input_gathers():
    R, C = 64, 64
    y = T((R, C), (1, R), base=1)
    p = E.from_spec(add_spec(2)).plan(T((R, C)), y, T((R, C)))
    assert p["path"] == "gather", p


def test_four_staged_inputs_gather():
    spec = [("a", ("load", "f32", 2)), ("b", ("load", "f32", 2)), ("c", ("load", "f32", 2)),
            ("d", ("load", "f32", 2)), ("s", ("add", "a", "b")), ("t", ("add", "c", "d")),
            ("u", ("add", "s", "t")), ("out", ("store", "u", 2))]
    tr = lambda: T((64, 64), (1, 64))
    p = E.from_spec(spec).plan(tr(), tr(), tr(), T((64, 64)), T((64, 64)))
    # the tiled interpreter: four entries (the four inputs; s, t and u reuse
    # theirs), each a 32 x 64 x 4-byte region holding every wavefront's two
    # 1 KiB sub-chunks; the three staged inputs are staged in their own regions
    assert p["path"] == "tiled" and p["lds_bytes"] == 4 * 32 * 64 * 4, p
    p = E.from_spec(spec).plan(tr(), tr(), tr(), tr(), T((64, 64)))
    assert p["path"] == "gather"


def test_shapes_are_right_aligned():
    mixed = [("x", ("load", "f32", 1)), ("y", ("load", "f32", 2)), ("z", ("add", "x", "y")),
             ("out", ("store", "z", 3))]
    c = E.from_spec(mixed)
    p = c.plan(T((12,)), T((1, 12)), T((1, 1, 12)))
    assert p["path"] == "linear" and p["size"] == (1, 1, 1, 12)
    _err(lambda: E.from_spec(mixed).plan(T((12,)), T((3, 4)), T((1, 3, 4))), "CMD_E_SHAPE")
    _err(lambda: E.from_spec(mixed).plan(T((4,)), T((3, 4)), T((1, 3, 4))), "CMD_E_SHAPE")   # no implicit broadcast


def test_rank_of_a_value_must_match_its_declaration():
    c = E.from_spec(add_spec(3))
    _err(lambda: c.plan(T((2, 3, 4)), T((6, 4)), T((2, 3, 4))), "CMD_E_SHAPE")


def test_store_views_must_be_one_to_one():
    spec = add_spec(2)
    _err(lambda: E.from_spec(spec).plan(T((2, 4)), T((2, 4)), T((2, 4), (0, 1))), "CMD_E_STRIDE")
    _err(lambda: E.from_spec(spec).plan(T((4, 4)), T((4, 4)), T((4, 4), (2, 1))), "CMD_E_STRIDE")
    _err(lambda: E.from_spec(add_spec(4)).plan(T((2, 2, 2, 2)), T((2, 2, 2, 2)), T((2, 2, 2, 2), (8, 4, 2, 2))),
         "CMD_E_STRIDE")
    assert E.from_spec(spec).plan(T((4, 4)), T((4, 4)), T((4, 4), (1, 4)))["path"] == "tiled"
    # interleaved but one-to-one: strides 1 and 3 over sizes 3 and 5 (reach 2 < 3)
    p = E.from_spec(spec).plan(T((5, 3)), T((5, 3)), T((5, 3), (3, 1)))
    assert p["path"] == "linear"
    p = E.from_spec(spec).plan(T((5, 3)), T((5, 3)), T((5, 3), (1, 5)))
    assert p["path"] == "gather"                     # output rows of 5 elements: no 16-byte vectors


def test_aliasing_in_four_dimensions():
    spec = add_spec(4)
    shape = (2, 3, 4, 8)
    st = (4 * 8 * 3 * 2, 8, 3 * 8 * 2, 1)           # a permuted view of one storage
    x = T(shape, st)
    same = FakeTensor(shape, st, ptr=x.data_ptr())
    E.from_spec(spec).plan(x, T(shape), same)        # in place through the identical view
    shifted = FakeTensor(shape, st, ptr=x.data_ptr() + 4)
    _err(lambda: E.from_spec(spec).plan(x, T(shape), shifted), "CMD_E_ALIAS")
    other_order = FakeTensor(shape, contiguous_strides(shape), ptr=x.data_ptr())
    _err(lambda: E.from_spec(spec).plan(x, T(shape), other_order), "CMD_E_ALIAS")


def test_empty_shapes_plan_nothing():
    shape = (3, 0, 5)
    p = E.from_spec(add_spec(3)).plan(T(shape), T(shape), T(shape))
    assert p["path"] == "none" and p["grid"] == 0


def test_huge_linear_grid_is_capped_and_loops():
    n = 1 << 36
    p = E.from_spec(add_spec(1)).plan(T((n,)), T((n,)), T((n,)))
    assert p["path"] == "linear" and p["grid"] * p["block"] <= 1 << 31, p


def test_tiny_planes_beyond_the_dispatch_limit_gather():
    B, R, C = 1 << 24, 8, 8
    yt = T((B, R, C), (R * C, 1, R))
    p = E.from_spec(add_spec(3)).plan(T((B, R, C)), yt, T((B, R, C)))
    assert p["path"] == "gather", p
    B = 1 << 10
    yt = T((B, R, C), (R * C, 1, R))
    p = E.from_spec(add_spec(3)).plan(T((B, R, C)), yt, T((B, R, C)))
    assert p["path"] == "tiled" and p["grid"] == B, p


def test_negative_strides_and_sizes_are_rejected():
    spec = add_spec(3)
    _err(lambda: E.from_spec(spec).plan(T((2, 3, 4)), T((2, 3, 4), (12, -4, 1)), T((2, 3, 4))), "CMD_E_STRIDE")
    _err(lambda: E.from_spec(spec).plan(T((2, -3, 4), (12, 4, 1)), T((2, 3, 4)), T((2, 3, 4))), "CMD_E_SHAPE")


def test_random_view_cases_reach_every_path():
    """The random view cases that the GPU parity tests run cover the linear,
    rows, tiled and gather paths (planned here with the device's alignment: every
    storage at a fresh 4 KiB-aligned address)."""
    import workloads as W
    from random_commands import random_view_case
    seen = {}
    for seed, staged in [(s, False) for s in range(80)] + [(s, True) for s in range(30)]:
        spec, ins, outs = random_view_case(seed, staged)
        vals = []
        for x in list(ins) + list(outs):
            if isinstance(x, tuple):
                view, storage = x
                off, strides = W.layout(view, storage)
                dt = {np.dtype(np.float16): torch.float16, np.dtype(np.uint16): torch.bfloat16,
                      np.dtype(np.float32): torch.float32, np.dtype(np.int32): torch.int32}[view.dtype]
                base = T((1,), dtype=dt).data_ptr()
                vals.append(FakeTensor(view.shape, strides, dt, base + off * view.itemsize))
            else:
                vals.append(x)
        p = E.from_spec(spec).plan(*vals)
        seen[p["path"]] = seen.get(p["path"], 0) + 1
    assert all(seen.get(k, 0) >= 8 for k in ("linear", "rows", "tiled", "gather")), seen
