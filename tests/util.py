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


def bf16_rne_bits(x) -> np.ndarray:
    """bf16 bit patterns of finite fp32 values, rounded to nearest, ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
