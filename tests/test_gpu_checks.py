"""The GPU parity bars themselves, on the CPU: each accepts what it should
and rejects a result one step outside it."""
import numpy as np
import pytest
import torch

from gpu_checks import assert_near_each_other, assert_parity


def rejects(y, ref, dtype):
    with pytest.raises(AssertionError):
        assert_parity(y, np.asarray(ref, dtype=np.float64), dtype)


def test_fp32_bar():
    ref = np.array([[1.0, -3.0, 0.0]])
    assert_parity(torch.tensor([[1.0 + 9e-6, -3.0 * (1 - 9e-6), 0.0]]), ref, torch.float32)
    rejects(torch.tensor([[1.0 + 2e-5, -3.0, 0.0]]), ref, torch.float32)
    rejects(torch.tensor([[1.0, -3.0, 1e-30]]), ref, torch.float32)  # zero stays zero


def test_bf16_bar_is_one_ulp():
    ref = np.array([[1.0 + 2.0 ** -9]])  # between 1 and 1 + 2^-7
    assert_parity(torch.tensor([[1.0]]).bfloat16(), ref, torch.bfloat16)
    assert_parity(torch.tensor([[1.0 + 2.0 ** -7]]).bfloat16(), ref, torch.bfloat16)
    rejects(torch.tensor([[1.0 + 2.0 ** -6]]).bfloat16(), ref, torch.bfloat16)


def test_e4m3_bar_and_saturation():
    F8 = torch.float8_e4m3fn
    assert_parity(torch.tensor([[448.0, -448.0, 1.0]]).to(F8), np.array([[881.0, -600.0, 1.01]]), F8)
    rejects(torch.tensor([[416.0]]).to(F8), [[881.0]], F8)      # must saturate to 448
    rejects(torch.tensor([[1.25]]).to(F8), [[1.0]], F8)         # two e4m3 ulps away
    assert_parity(torch.tensor([[1.125]]).to(F8), np.array([[1.0]]), F8)  # one ulp
    assert_parity(torch.tensor([[2.0 ** -9]]).to(F8), np.array([[0.0]]), F8)  # subnormal spacing
    rejects(torch.tensor([[float("nan")]]).to(F8), [[1.0]], F8)


def test_near_each_other():
    a = torch.tensor([1.0, 2.0]).bfloat16()
    b = torch.tensor([1.0 + 2.0 ** -7, 2.0]).bfloat16()
    assert assert_near_each_other(a, b, torch.bfloat16) == 0.5
    with pytest.raises(AssertionError):
        assert_near_each_other(a, torch.tensor([1.0 + 2.0 ** -5, 2.0]).bfloat16(), torch.bfloat16)
