"""Pins of the error metrics every GPU parity test goes through (oracle/metrics.py).

The metrics implement the row-wise reading of "max rel err": for every row (the
last axis) ||y - r||_inf / ||r||_inf, maximised over rows; states per matrix.
Each test below plants an error of known size and checks that the metric
reports exactly that size, on the right axis, and that non-finite results fail.
"""
import numpy as np
import pytest
import torch

from oracle.metrics import mat_rel_err, row_rel_err


def _ref(shape, seed=0):
    return np.random.default_rng(seed).standard_normal(shape)


def test_planted_error_reported_exactly():
    ref = np.zeros((3, 4, 8))
    ref[...] = 4.0              # every row has ||r||_inf = 4
    ref[1, 2, 5] = -16.0        # row (1, 2) has ||r||_inf = 16
    y = ref.copy()
    y[2, 3, 1] += 0.5           # row (2, 3): 0.5 / 4
    assert row_rel_err(y, ref) == 0.125
    y = ref.copy()
    y[1, 2, 0] -= 0.5           # row (1, 2): 0.5 / 16
    assert row_rel_err(y, ref) == 0.03125
    assert row_rel_err(ref, ref) == 0.0


def test_largest_row_error_wins():
    ref = np.ones((5, 6))
    y = ref.copy()
    y[0, 0] += 2.0 ** -10
    y[4, 5] += 2.0 ** -6
    y[2, 3] -= 2.0 ** -8
    assert row_rel_err(y, ref) == 2.0 ** -6


def test_late_small_row_error_is_caught():
    """Gradient-like rows whose magnitude falls by 500x along the sequence: an
    error of twice the size of a late row must show as 2, although it is far
    below 1e-2 of the largest element of the tensor."""
    n = 1000
    scale = np.geomspace(1.0, 1.0 / 500.0, n)[:, None]
    ref = _ref((n, 64)) * scale
    y = ref.copy()
    row = n - 7
    y[row] += 2.0 * ref[row]              # the late row is off by 2x its own size
    assert np.abs(y - ref).max() / np.abs(ref).max() < 1e-2   # the whole-tensor ratio misses it
    assert row_rel_err(y, ref) == pytest.approx(2.0, rel=1e-12)


def test_row_is_the_last_axis():
    """Rows of very different size: the error must be divided by its own row's
    maximum, not by a column's or the tensor's."""
    ref = np.array([[1.0, 2.0, 3.0, 4.0],
                    [100.0, 200.0, 300.0, 400.0]])
    y = ref.copy()
    y[0, 1] += 1.0               # row 0: 1 / 4; column 1: 1 / 200; tensor: 1 / 400
    assert row_rel_err(y, ref) == 0.25
    # the same data transposed puts the error in a row whose maximum is 200
    assert row_rel_err(y.T.copy(), ref.T.copy()) == 1.0 / 200.0


def test_zero_rows_use_absolute_error():
    ref = np.ones((3, 4))
    ref[1] = 0.0
    y = ref.copy()
    y[1, 2] = 0.75
    assert row_rel_err(y, ref) == 0.75
    y[1, 2] = 0.0
    y[0, 0] = 1.5
    assert row_rel_err(y, ref) == 0.5


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_non_finite_results_fail(bad):
    ref = np.ones((4, 4))
    y = ref.copy()
    y[3, 1] = bad
    assert row_rel_err(y, ref) == float("inf")
    assert mat_rel_err(y.reshape(1, 4, 4), ref.reshape(1, 4, 4)) == float("inf")
    # a non-finite reference can never pass a "< tol" check either
    assert row_rel_err(ref, y) == float("inf")


def test_shape_mismatch_raises():
    with pytest.raises(ValueError):
        row_rel_err(np.ones((2, 3)), np.ones((3, 2)))
    with pytest.raises(ValueError):
        mat_rel_err(np.ones((2, 3, 3)), np.ones((2, 3, 4)))


def test_mat_rel_err_per_matrix():
    """States: one ratio per (b, h) matrix over its last two axes."""
    ref = np.ones((2, 3, 4, 5))
    ref[0, 1] *= 1000.0
    y = ref.copy()
    y[0, 1, 3, 4] += 1.0         # matrix (0, 1): 1 / 1000
    y[1, 2, 0, 0] += 0.25        # matrix (1, 2): 0.25 / 1
    assert mat_rel_err(y, ref) == 0.25
    y[1, 2, 0, 0] = 1.0
    assert mat_rel_err(y, ref) == 0.001
    # vectors (z): mat_dims = 1 gives one ratio per row
    zr = np.full((2, 3, 8), 2.0)
    zy = zr.copy()
    zy[1, 0, 7] = 2.5
    assert mat_rel_err(zy, zr, 1) == 0.25


def test_torch_inputs_convert_exactly():
    ref = torch.tensor([[1.0, -2.0, 4.0]], dtype=torch.float64)
    y = torch.tensor([[1.0, -2.0, 4.0 + 2.0 ** -8]], dtype=torch.bfloat16)
    # bf16 holds 4 + 2^-8 only as 4 (8 bits of mantissa): the metric sees the bf16 value
    assert row_rel_err(y, ref) == 0.0
    y32 = torch.tensor([[1.0, -2.0, 4.0 + 2.0 ** -8]], dtype=torch.float32)
    assert row_rel_err(y32, ref) == 2.0 ** -10
    assert row_rel_err(torch.zeros(3, 0), torch.zeros(3, 0)) == 0.0


def test_grad_rel_err_rows_and_zero_rows():
    """Gradient rows: each against its own maximum, except the rows that are
    identically zero by the method, which are measured against the tensor."""
    from oracle.metrics import grad_rel_err

    n = 600
    ref = _ref((2, 3, n, 16), 5) * np.geomspace(1.0, 1.0 / 300.0, n)[:, None]
    zero = np.zeros((2, 3, n), dtype=bool)
    zero[..., 0] = True
    ref[..., 0, :] = 1e-17                 # rounding left where the exact gradient is 0
    y = ref.copy()
    y[..., 0, :] = 0.0
    assert grad_rel_err(y, ref, zero) < 1e-15
    # a late row off by 3x its own size is reported as 3
    y2 = y.copy()
    y2[1, 2, n - 3] += 3.0 * ref[1, 2, n - 3]
    assert grad_rel_err(y2, ref, zero) == pytest.approx(3.0, rel=1e-9)
    # a zero row that is not zero on the other side: measured against the tensor maximum
    y3 = y.copy()
    y3[0, 1, 0, 4] = 0.5 * np.abs(ref).max()
    assert grad_rel_err(y3, ref, zero) == pytest.approx(0.5, rel=1e-12)
    # without the mask the first row's 1e-17 reference makes any rounding there huge
    y4 = y.copy()
    y4[..., 0, :] = 1e-9
    assert grad_rel_err(y4, ref) > 1e6 and grad_rel_err(y4, ref, zero) < 1e-8
    y5 = y.copy()
    y5[0, 0, 7, 0] = np.nan
    assert grad_rel_err(y5, ref, zero) == float("inf")
    # a tensor that vanishes everywhere (dq with one token): only an outside scale works
    r0 = np.full((2, 3, 1, 16), 1e-17)
    g0 = np.full((2, 3, 1, 16), 2e-9)
    allz = np.ones((2, 3, 1), dtype=bool)
    assert grad_rel_err(g0, r0, allz) > 1e6
    assert grad_rel_err(g0, r0, allz, zero_scale=4.0) == pytest.approx(5e-10, rel=1e-12)


def test_grad_rel_err_row_floor():
    """A per-row floor (the size of the terms a row cancels from) replaces the
    row's own maximum only where it is larger."""
    from oracle.metrics import grad_rel_err

    ref = np.ones((1, 2, 4, 8))
    ref[0, 1, 2] = 1e-3                   # a row that nearly cancels
    floor = np.full((1, 2, 4), 0.5)
    floor[0, 1, 2] = 2.0                  # ... from terms of size 2
    y = ref.copy()
    y[0, 1, 2, 3] += 1e-5                 # 1e-2 of the row, 5e-6 of its terms
    assert grad_rel_err(y, ref) == pytest.approx(1e-2, rel=1e-9)
    assert grad_rel_err(y, ref, row_floor=floor) == pytest.approx(5e-6, rel=1e-9)
    y2 = ref.copy()
    y2[0, 0, 1, 0] += 0.25                # a floor below the row's own size changes nothing
    assert grad_rel_err(y2, ref, row_floor=floor) == 0.25
    with pytest.raises(ValueError):
        grad_rel_err(y, ref, row_floor=np.ones((2, 4)))
