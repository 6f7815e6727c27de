"""Non-finite sentinel: CPU reference.  Test infrastructure only -- the
product path never imports it.

Source: "DQN Backward-Path NaN Audit -- SP1 Phase A", section "Phase E -- SP2
fused NaN check kernel": one check over a table of buffers, a flag per slot
that is written 1 when the slot's buffer holds a bad value and is never
cleared, null entries skipped.  Reading: a bad value is any IEEE-754 value
that is not finite (NaN or +-infinity), the condition the same page's Adam
guard tests before it uses a gradient.
"""
import numpy as np


def is_nonfinite_bits(x):
    """float32 values whose exponent field is all ones (NaN or infinity),
    decided on the bit pattern."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32)
    return (b & np.uint32(0x7F800000)) == np.uint32(0x7F800000)


def update_flags(flags, buffers):
    """Sticky per-slot flags: slot s becomes 1 when buffers[s] (None = null
    entry) holds a non-finite value; otherwise it keeps its value."""
    out = np.array(flags, dtype=np.int32, copy=True)
    for s, b in enumerate(buffers):
        if b is not None and np.any(is_nonfinite_bits(b)):
            out[s] = 1
    return out
