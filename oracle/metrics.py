"""Comparison helpers for parity checks (test infrastructure)."""

import numpy as np


def rel_frob(y, ref):
    """Relative Frobenius error ||y - ref||_F / ||ref||_F in float64."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.linalg.norm((y - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    return float(num / den) if den > 0 else float(num)
