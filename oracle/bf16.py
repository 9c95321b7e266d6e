"""bfloat16 rounding used by the precision contract of the observation set.

The cache stores bfloat16 keys and values; the observation queries are
rotated in float64 and then rounded, first to float32 and then to bfloat16,
each time to nearest with ties to even.  bfloat16 keeps the upper 16 bits of
an IEEE float32, so rounding to it is integer arithmetic on the float32 bit
pattern: add 0x7FFF plus the lowest kept bit, then drop the low 16 bits.
"""

import numpy as np


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 (RNE); return the 16-bit patterns."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    is_nan = np.isnan(x32)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    # A NaN keeps its sign and becomes a quiet NaN instead of rounding.
    nan_bits = ((u >> np.uint64(16)) | np.uint64(0x0040)) & np.uint64(0xFFFF)
    r = np.where(is_nan, nan_bits, r & np.uint64(0xFFFF))
    return r.astype(np.uint16)


def bf16_bits_to_f64(b):
    """Widen bfloat16 bit patterns exactly to float64."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def round_f64_to_bf16(x):
    """float64 -> float32 (RNE) -> bfloat16 (RNE), returned as float64 values.

    This is the two-step chain named by the precision contract: numpy's
    float64 -> float32 cast rounds to nearest even.
    """
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    return bf16_bits_to_f64(f32_to_bf16_bits(x32))
