"""Brute-force bfloat16 rounding for the CPU pins: the nearest of all finite
bfloat16 values, ties to the even bit pattern, by search over the whole
grid (independent of the oracle's round_to_bf16).  Not collected by pytest."""
import numpy as np


def bf16_grid():
    """Every finite non-negative bfloat16 value, ascending, with its bit
    pattern."""
    bits = np.arange(0, 0x7f80, dtype=np.uint32)
    vals = (bits << 16).view(np.float32).astype(np.float64)
    return vals, bits


def nearest_bf16(x):
    """Round float64 values to the nearest bfloat16 value, ties to even."""
    vals, bits = bf16_grid()
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a), 1, vals.size - 1)
    lo = hi - 1
    dlo, dhi = a - vals[lo], vals[hi] - a
    pick = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(bits[lo] % 2 == 0, lo, hi)))
    return np.sign(x) * vals[pick]
