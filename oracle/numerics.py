"""Exact conversions of stored inputs to float64 (test infrastructure: only
the tests, the smoke check and the benchmark's CPU baseline use the oracle).

The oracle sees the values exactly as stored on the device: a bf16 value is
the top 16 bits of an IEEE binary32, so widening its bit pattern by 16 zero
bits gives the binary32 with the same value, which float64 holds exactly.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """float64 values of bf16 bit patterns given as uint16/int16 arrays."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_f64(x: np.ndarray) -> np.ndarray:
    """float64 values of a binary32 array (exact)."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)

