"""float32 -> bfloat16 storage rounding, round-to-nearest-even.

bfloat16 keeps the top 16 bits of an IEEE-754 binary32 value (sign, 8-bit
exponent, 7 stored mantissa bits).  Rounding to nearest, ties to even, adds
0x7FFF plus the lowest kept bit to the 32-bit pattern before truncation.
NaN maps to the canonical quiet NaN 0x7FC0.

The pages' own cast (``f32_to_bf16_kernel`` in "DQN Backward-Path NaN Audit",
section "Prior-investigation status") also replaces NaN by 0 and clamps to
+-500; the plain rounding used here agrees with it on every finite input of
magnitude <= 500, which covers all inputs these tests draw.
"""
import numpy as np


def to_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns (RNE)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    out = (rounded & np.uint32(0xFFFF)).astype(np.uint16)
    out[np.isnan(x)] = np.uint16(0x7FC0)
    return out


def from_bits(b):
    """uint16 bfloat16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(x):
    """Round float32 values to the nearest bfloat16 value, returned as float32."""
    return from_bits(to_bits(x))
