"""The gradient tolerance rule of the GPU parity tests, checked against the
element formats themselves: the stated bound (5e-2 bf16, 2e-2 f16, 1e-4
fp32) holds everywhere, and one ulp of |ref| is added only from the
magnitude at which half the spacing of the output format alone exceeds it."""

import numpy as np
import pytest

from tests.gpu_helpers import G_TOL, grad_bound, half_ulp_threshold


def bf16_spacing(x):
    """Distance from the bf16 value x to the next larger bf16 value."""
    bits = np.array([x], np.float32).view(np.uint32)[0]
    assert bits & 0xFFFF == 0, "x must be a bf16 value"
    nxt = np.array([bits + 0x10000], np.uint32).view(np.float32)[0]
    return float(nxt) - x


def spacing(dtype, x):
    if dtype == "bf16":
        return bf16_spacing(x)
    return float(np.spacing({"f16": np.float16, "f32": np.float32}[dtype](x)))


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_threshold_is_where_half_spacing_first_exceeds_the_tolerance(dtype):
    tol = G_TOL[dtype]
    t = half_ulp_threshold(dtype, tol)
    assert t == {"bf16": 16.0, "f16": 64.0, "f32": 2048.0}[dtype]
    assert spacing(dtype, t) / 2 > tol
    # the largest value of the binade below: half its spacing fits the tolerance
    below = t - spacing(dtype, t / 2)
    assert spacing(dtype, below) / 2 <= tol


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_bound_is_the_stated_tolerance_below_the_threshold(dtype):
    tol = G_TOL[dtype]
    t = half_ulp_threshold(dtype, tol)
    ref = np.array([0.0, -1.0, 3.5, t / 2, -(t * 0.999), t, -2 * t])
    b = grad_bound(ref, dtype)
    assert np.all(b[:5] == tol)
    assert np.all(b[5:] > tol)
    # above the threshold the extra term covers one rounding of the output
    for x in (t, 2 * t, 3.75 * t):
        assert grad_bound(np.array([x]), dtype)[0] >= tol + spacing(dtype, x) / 2 * (1 - 1e-12)
