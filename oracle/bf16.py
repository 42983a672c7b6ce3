"""Decode bf16 bit patterns to float64 (oracle side; test infrastructure only).

A bf16 value is the upper half of an IEEE-754 binary32: widening is exact.
"""
import numpy as np


def to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)
