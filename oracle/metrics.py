"""Error metrics used to compare results with the oracle (test infrastructure).

Row-wise relative error: for every output row r (the last axis is the row),
    err = ||y - r||_inf / ||r||_inf,
maximised over rows.  Rows whose reference is exactly zero use the absolute
error.  The element-wise ratio is not used: a causal output row is a convex
combination of value rows, so individual components pass through zero and
their relative error is unbounded for any implementation.

A non-finite value in either the result or the reference gives inf, so that a
"< tol" check can never pass on it; callers that expect NaN rows (maps whose
denominator can vanish) compare the NaN pattern first and pass only the
finite rows.  The metrics themselves are pinned in tests/test_metrics_cpu.py.
"""
from __future__ import annotations

import numpy as np


def _np(x):
    if hasattr(x, "detach"):
        import torch
        return x.detach().to("cpu").to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def row_rel_err(y, ref) -> float:
    y, ref = _np(y), _np(ref)
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    if y.size == 0:
        return 0.0
    if not (np.all(np.isfinite(y)) and np.all(np.isfinite(ref))):
        return float("inf")
    diff = np.abs(y - ref).max(axis=-1)
    scale = np.abs(ref).max(axis=-1)
    rel = np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), diff)
    return float(rel.max())


def mat_rel_err(y, ref, mat_dims: int = 2) -> float:
    """Relative error per matrix (the last ``mat_dims`` axes): max |y-r| / max |r|."""
    y, ref = _np(y), _np(ref)
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    if y.size == 0:
        return 0.0
    if not (np.all(np.isfinite(y)) and np.all(np.isfinite(ref))):
        return float("inf")
    axes = tuple(range(y.ndim - mat_dims, y.ndim))
    diff = np.abs(y - ref).max(axis=axes)
    scale = np.abs(ref).max(axis=axes)
    rel = np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), diff)
    return float(np.max(rel))


def grad_rel_err(y, ref, zero_rows=None, zero_scale=None, row_floor=None) -> float:
    """Row-wise error of a gradient (the reading above, per (b, h, token) row).

    ``zero_rows`` marks, over the leading axes, the rows whose exact value is
    identically zero by the method (for example dq of the first token, whose
    output is v_1 whatever q_1 is); the oracle holds only rounding there (about
    1e-17), so those rows are measured against ``zero_scale`` (the caller's
    scale of the problem, for example the largest element of all the
    gradients; default: the largest element of this one, which is itself only
    rounding when every row of the tensor vanishes).  Every other row is
    measured against its own maximum, as row_rel_err does, or against
    ``row_floor`` (per row, over the leading axes) where that is larger: the
    size of the terms a row is the difference of, for rows that cancel (a
    mixed relative error: any float32 evaluation errs by rounding times the
    terms, not times the result).
    """
    y, ref = _np(y), _np(ref)
    if y.shape != ref.shape:
        raise ValueError(f"shape mismatch {y.shape} vs {ref.shape}")
    if y.size == 0:
        return 0.0
    if not (np.all(np.isfinite(y)) and np.all(np.isfinite(ref))):
        return float("inf")
    zero = np.zeros(y.shape[:-1], dtype=bool) if zero_rows is None else np.asarray(zero_rows, dtype=bool)
    if zero.shape != y.shape[:-1]:
        raise ValueError(f"zero_rows shape {zero.shape} vs rows {y.shape[:-1]}")
    keep = ~zero
    if row_floor is None:
        err = row_rel_err(y[keep], ref[keep]) if keep.any() else 0.0
    else:
        floor = np.asarray(row_floor, dtype=np.float64)
        if floor.shape != y.shape[:-1]:
            raise ValueError(f"row_floor shape {floor.shape} vs rows {y.shape[:-1]}")
        diff = np.abs(y - ref).max(axis=-1)
        scale = np.maximum(np.abs(ref).max(axis=-1), floor)
        rel = np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), diff)
        err = float(rel[keep].max()) if keep.any() else 0.0
    if zero.any():
        top = np.abs(ref).max() if zero_scale is None else float(zero_scale)
        z = np.abs(y[zero]).max()
        err = max(err, z / top if top > 0 else z)
    return float(err)
