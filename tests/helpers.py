"""Comparison helpers for the tests (no arithmetic of the method here)."""
import numpy as np


def max_abs_rel(a, b):
    """max|a - b| / max(max|b|, 1e-30) over the whole tensor (b = reference)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(float(np.max(np.abs(b))) if b.size else 0.0, 1e-30)
    return float(np.max(np.abs(a - b))) / den if a.size else 0.0
