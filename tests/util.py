"""Comparison helpers shared by the tests (no backward arithmetic here)."""
import numpy as np


def relrms(a, b) -> float:
    """Norm-relative error ||a-b|| / ||b|| (the `relerr` metric of the PR #730 harness)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = float(np.linalg.norm(b))
    num = float(np.linalg.norm(a - b))
    return num / den if den else num


def maxabs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b))) if a.size else 0.0
