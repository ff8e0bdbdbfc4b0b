"""Exact conversions between storage formats and float64 (oracle side)."""
import numpy as np


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Storage values -> float64. bf16 bit patterns widen exactly: the 16 bits
    become the high half of an IEEE float32, which float64 holds exactly."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    raise ValueError(dtype)
