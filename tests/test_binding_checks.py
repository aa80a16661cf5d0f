"""Argument checks of the Python binding that run before any C call (CPU only).

The C entry points see only addresses and sizes: a caller-supplied output or
workspace with the wrong dtype, shape, device or layout would be written past
its end or with the wrong byte layout, so the binding rejects it first.
"""
import pytest
import torch

from exact_attention_22_amd import binding

CPU = torch.device("cpu")


def test_buffer_with_the_right_dtype_shape_device_and_layout_passes():
    binding._check_buffer("out", torch.empty((2, 3, 5, 64), dtype=torch.bfloat16), torch.bfloat16, (2, 3, 5, 64), CPU)
    binding._check_buffer("ws", torch.empty(1000, dtype=torch.uint8), torch.uint8, None, CPU)


@pytest.mark.parametrize("t,dtype,shape,exc", [
    (torch.empty((2, 3, 5, 64), dtype=torch.float32), torch.bfloat16, (2, 3, 5, 64), TypeError),   # out fp32 for bf16
    (torch.empty((2, 3, 4, 64), dtype=torch.bfloat16), torch.bfloat16, (2, 3, 5, 64), ValueError),  # undersized
    (torch.empty((2, 3, 5, 64), dtype=torch.bfloat16).transpose(1, 2), torch.bfloat16, (2, 5, 3, 64), ValueError),
    (torch.empty((2, 3, 5), dtype=torch.float64), torch.float32, (2, 3, 5), TypeError),             # lse dtype
    (torch.empty(100, dtype=torch.int8), torch.uint8, None, TypeError),                            # workspace dtype
    ([0.0] * 4, torch.float32, (4,), TypeError),                                                   # not a tensor
])
def test_buffer_mismatches_are_rejected(t, dtype, shape, exc):
    with pytest.raises(exc):
        binding._check_buffer("buf", t, dtype, shape, CPU)


def test_buffer_on_another_device_is_rejected():
    with pytest.raises(ValueError):
        binding._check_buffer("out", torch.empty(4, dtype=torch.float32), torch.float32, (4,), torch.device("cuda:0"))
