"""Error metrics used to compare results with the oracle (test infrastructure).

Row-wise relative error: for every output row r (the last axis is the row),
    err = ||y - r||_inf / ||r||_inf,
maximised over rows.  Rows whose reference is exactly zero use the absolute
error.  The element-wise ratio is not used: a causal output row is a convex
combination of value rows, so individual components pass through zero and
their relative error is unbounded for any implementation.
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
    if not np.all(np.isfinite(y)):
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
    if not np.all(np.isfinite(y)):
        return float("inf")
    axes = tuple(range(y.ndim - mat_dims, y.ndim))
    diff = np.abs(y - ref).max(axis=axes)
    scale = np.abs(ref).max(axis=axes)
    rel = np.where(scale > 0, diff / np.where(scale > 0, scale, 1.0), diff)
    return float(np.max(rel))
