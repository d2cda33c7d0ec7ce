"""Exact conversions of stored inputs to float64, and exact column sums
(test infrastructure: only the tests, the smoke check and the benchmark's
CPU baseline use the oracle).

The oracle sees the values exactly as stored on the device: a bf16 value is
the top 16 bits of an IEEE binary32, so widening its bit pattern by 16 zero
bits gives the binary32 with the same value, which float64 holds exactly.
"""

from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """float64 values of bf16 bit patterns given as uint16/int16 arrays."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_to_f64(x: np.ndarray) -> np.ndarray:
    """float64 values of a binary32 array (exact)."""
    return np.asarray(x, dtype=np.float32).astype(np.float64)



def exact_column_sums(x: np.ndarray) -> np.ndarray:
    """Sum of every column of ``x[n][d]`` (float64), computed exactly and then
    rounded once to the nearest float64 (ties to even): what ``math.fsum``
    returns for the column.

    A column goes through numpy's own sum only when no partial sum can round,
    whatever the order: with u the weight of the lowest set significand bit
    of the column's finest value, every value is an integer multiple of u,
    and if sum |x| <= 2^53 u every partial sum is an integer multiple of u of
    magnitude at most 2^53 u, which float64 holds exactly (the bound is taken
    with a factor of 2 to spare for the rounding of the computed sum |x|).
    Every other column goes through ``math.fsum``."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2:
        raise ValueError("x must be 2-D")
    sums = x.sum(axis=0)
    if x.shape[0] == 0:
        return sums
    mant, ex = np.frexp(x)                     # x = mant * 2^ex, 0.5 <= |mant| < 1
    sig = (np.abs(mant) * 2.0 ** 53).astype(np.int64)   # integer significand, exact
    low = sig & -sig                           # its lowest set bit
    unit = np.ldexp(low.astype(np.float64), ex - 53)
    unit = np.where(x != 0.0, unit, np.inf).min(axis=0)
    certified = np.abs(x).sum(axis=0) <= np.ldexp(unit, 52)
    for c in np.nonzero(~certified)[0]:
        sums[c] = math.fsum(x[:, c].tolist())
    return sums
