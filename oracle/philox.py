"""Philox4x64-10, written from its published definition.

Reference: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3", SC'11 (the Philox-4x64 round function,
its two multipliers and the two Weyl key increments are given there).

The HER "future" and "random" donor strategies of "GPU IQL + HER Porting Plan"
(section "Donor Index Generation") draw a uniform index per relabelled row; the
pages use cuRAND without naming a generator, so both this oracle and the HIP
library implement Philox4x64-10 independently from the paper.

Vectorised over NumPy uint64 arrays; the 64x64->128 bit product is formed
exactly from 32-bit limbs.
"""
import numpy as np

U64 = np.uint64
MASK32 = U64(0xFFFFFFFF)

# Round multipliers and key schedule (Weyl) constants, Philox-4x64.
M0 = U64(0xD2E7470EE14C6C93)
M1 = U64(0xCA5A826395121157)
W0 = U64(0x9E3779B97F4A7C15)
W1 = U64(0xBB67AE8584CAA73B)
ROUNDS = 10


def mulhilo64(a, b):
    """Exact 128-bit product of uint64 arrays; returns (hi, lo)."""
    a = np.asarray(a, dtype=U64)
    b = np.asarray(b, dtype=U64)
    with np.errstate(over="ignore"):
        a_lo, a_hi = a & MASK32, a >> U64(32)
        b_lo, b_hi = b & MASK32, b >> U64(32)
        ll = a_lo * b_lo
        lh = a_lo * b_hi
        hl = a_hi * b_lo
        hh = a_hi * b_hi
        mid = (ll >> U64(32)) + (lh & MASK32) + (hl & MASK32)
        lo = (ll & MASK32) | ((mid & MASK32) << U64(32))
        hi = hh + (lh >> U64(32)) + (hl >> U64(32)) + (mid >> U64(32))
    return hi, lo


def philox4x64(ctr, key, rounds=ROUNDS):
    """Philox4x64-R block function.

    ctr: tuple of 4 uint64 arrays (broadcastable), key: tuple of 2 uint64.
    Returns a tuple of 4 uint64 arrays.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=U64) for c in ctr)
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = U64(key[0])
    k1 = U64(key[1])
    with np.errstate(over="ignore"):
        for r in range(rounds):
            if r > 0:
                k0 = k0 + W0
                k1 = k1 + W1
            hi0, lo0 = mulhilo64(M0, c0)
            hi1, lo1 = mulhilo64(M1, c2)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def uniform_index(r64, lo, span):
    """Map a 64-bit random word to lo + floor(r64 * span / 2**64).

    Exact integer multiply-shift; ``span`` must be >= 1.  Bias is at most
    span / 2**64 per value.
    """
    hi, _ = mulhilo64(np.asarray(r64, dtype=U64), np.asarray(span, dtype=U64))
    return np.asarray(lo, dtype=np.int64) + hi.astype(np.int64)
