"""The parity bar's allowance for a bf16 output store (tests/gpu_common.py):
half a bf16 ulp at the value's magnitude bounds what round-to-nearest adds,
checked against torch's own bf16 rounding (a library routine)."""
import numpy as np
import pytest
import torch

from tests.gpu_common import bf16_half_ulp

pytestmark = pytest.mark.cpu


def test_half_ulp_values():
    assert bf16_half_ulp(np.array([1.0]))[0] == 2.0 ** -8        # [1, 2): ulp 2^-7
    assert bf16_half_ulp(np.array([3.5]))[0] == 2.0 ** -7        # [2, 4): ulp 2^-6
    assert bf16_half_ulp(np.array([0.75]))[0] == 2.0 ** -9
    assert bf16_half_ulp(np.array([0.0]))[0] == 0.0


def test_half_ulp_bounds_torch_rounding():
    g = torch.Generator().manual_seed(3)
    # the kernels round fp32 values to bf16, so the values start in fp32 (a
    # float64 -> fp32 -> bf16 chain rounds twice and may pass the half ulp)
    x = (torch.randn(200000, generator=g, dtype=torch.float32) * 3).double()
    r = x.to(torch.float32).to(torch.bfloat16).to(torch.float64)
    err = (r - x).abs().numpy()
    bound = bf16_half_ulp(np.abs(x.numpy()))
    assert (err <= bound).all()
    assert (err > 0.9 * bound).any()          # the bound is attained, not loose
