"""Exact widening of stored element patterns to float64 (oracle; test infrastructure only).

A bf16 value is the upper 16 bits of an IEEE binary32 value, so widening is exact: place the 16-bit
pattern in the high half of a 32-bit word, read that word as binary32, then convert to binary64.
"""

import numpy as np


def bf16_bits_to_f64(bits):
    """Widen raw bf16 patterns (any integer array of 16-bit values) to float64, exactly."""
    u16 = np.asarray(bits).astype(np.uint16, copy=False)
    u32 = u16.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def as_f64(x, dtype):
    """Return the float64 value of an array stored as ``dtype`` ("f32" values or "bf16" raw bits)."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")
