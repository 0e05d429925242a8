"""bfloat16 rounding for the oracle's bf16 mode.

bfloat16 is the upper half of an IEEE binary32. Rounding to it is
round-to-nearest, ties-to-even on the low 16 bits. A float64 input is first
rounded to binary32 (also ties-to-even), as the GPU rounds its float32
accumulators; the double rounding is part of the definition used here.
"""
import numpy as np


def identity(x):
    """Exact mode: no rounding."""
    return x


def round_bf16(x):
    """Nearest bfloat16 value of x (float64 in, float64 out). NaN stays NaN."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = r.view(np.float32).astype(np.float64)
    nan = np.isnan(f)
    if np.any(nan):
        out[nan] = np.nan
    return out


def bf16_bits(x):
    """16-bit pattern of round_bf16(x)."""
    v = round_bf16(x).astype(np.float32)
    return (np.ascontiguousarray(v).view(np.uint32) >> 16).astype(np.uint16)


def from_bf16_bits(b):
    """float64 values of 16-bit bfloat16 patterns."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16)).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)
