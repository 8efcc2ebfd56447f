"""Exact upcasting of stored tensors to float64 (oracle side; test infrastructure).

bf16 tensors are stored as uint16 bit patterns; a bf16 value is the float32
whose upper 16 bits are those bits, so widening is exact.
"""
import numpy as np


def decode(a, dtype: str) -> np.ndarray:
    """Stored tensor -> float64, exactly."""
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype in ("f32", "f16"):
        return np.asarray(a).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
