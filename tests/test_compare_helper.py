"""The GPU tests' comparison helper on CPU data: the per-head relative RMS bound catches a
proportional error that the absolute bounds cannot see at the small |O| of long rows."""
import pytest
import torch

from gpu_util import BF16_TOL, compare


def _case(scale_err: float):
    g = torch.Generator().manual_seed(0)
    o_ref = 1.6e-3 * torch.randn(1, 64, 4, 128, generator=g, dtype=torch.float64)  # |O| at ~1M keys
    l_ref = torch.full((1, 64, 4), 14.0, dtype=torch.float64)
    return o_ref * (1.0 + scale_err), l_ref.clone(), o_ref, l_ref


def test_small_relative_error_passes():
    compare(*_case(1e-3), BF16_TOL, "0.1% off")


def test_proportional_error_below_absolute_bounds_is_caught():
    o, l, o_ref, l_ref = _case(3e-2)
    assert (o - o_ref).abs().max().item() < BF16_TOL.max_abs  # invisible to the absolute bounds
    with pytest.raises(AssertionError, match="relative RMS"):
        compare(o, l, o_ref, l_ref, BF16_TOL, "3% off")
