"""The staggered operand allocation of the Python binding, on the CPU (no
kernel runs): start addresses k * step modulo 32 KiB past a 32 KiB boundary,
no overlap, the requested shapes and dtypes, independent contents."""
import pytest
import torch

import elementwise_tensor_commands_amd as ecmd


@pytest.mark.parametrize("step", [256, 4096, 12288, 32768, 40960])
def test_offsets_modulo_period(step):
    specs = [((1000, 3), torch.float32), ((4097,), torch.float16), ((5, 5, 5), torch.int32),
             ((70000,), torch.bfloat16), ((1,), torch.float32), ((33, 2), torch.float32),
             ((9,), torch.float16), ((10,), torch.int32), ((11,), torch.float32)]
    ts = ecmd.empty_staggered(specs, device="cpu", step=step)
    P = ecmd.STAGGER_PERIOD
    for k, ((shape, dt), t) in enumerate(zip(specs, ts)):
        assert t.shape == torch.Size(shape) and t.dtype == dt and t.is_contiguous()
        assert t.data_ptr() % P == (k * step) % P, (k, t.data_ptr() % P)
    spans = sorted((t.data_ptr(), t.data_ptr() + t.numel() * t.element_size()) for t in ts)
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    for k, t in enumerate(ts):
        t.view(-1)[:] = k + 1
    for k, t in enumerate(ts):
        assert bool((t.view(-1) == k + 1).all())


def test_storage_outlives_the_first_tensor():
    a, b = ecmd.empty_staggered([((64,), torch.float32), ((64,), torch.float32)], device="cpu")
    b.fill_(3.0)
    del a
    assert bool((b == 3.0).all())


@pytest.mark.parametrize("step", [0, -4096, 100])
def test_bad_step(step):
    with pytest.raises(ValueError):
        ecmd.empty_staggered([((4,), torch.float32)], device="cpu", step=step)
