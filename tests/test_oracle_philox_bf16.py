"""Pins of the oracle's Philox4x64-10 and bfloat16 rounding.

Philox: NumPy ships an independent Philox4x64-10 bit generator; it increments
its 256-bit counter before producing each block, so the block at counter c is
``Philox(counter=c - 1).random_raw(4)``.
bf16: torch's float32 -> bfloat16 conversion (round to nearest even) and
hand-worked tie cases.
"""
import numpy as np
import torch

from oracle import bf16, philox


def _numpy_block(ctr, key):
    c = np.array(ctr, dtype=np.uint64).copy()
    # numpy pre-increments with carry over the four words
    for i in range(4):
        if c[i] != 0:
            c[i] -= np.uint64(1)
            break
        c[i] = np.uint64(0xFFFFFFFFFFFFFFFF)
    bg = np.random.Philox(counter=c, key=np.array(key, dtype=np.uint64))
    return bg.random_raw(4)


def test_philox_matches_numpy():
    cases = [((1, 0, 0, 0), (0, 0)), ((5, 7, 0, 0), (20261202, 0x484552646F6E6F72)),
             ((123456789, 42, 3, 9), (0xFFFFFFFFFFFFFFFF, 1)), ((0, 1, 0, 0), (9, 9))]
    for ctr, key in cases:
        ref = _numpy_block(ctr, key)
        out = philox.philox4x64(ctr, key)
        assert [int(x) for x in out] == [int(x) for x in ref], (ctr, key)


def test_philox_vectorised_rows():
    rows = np.arange(50, dtype=np.uint64)
    w0, w1, w2, w3 = philox.philox4x64((rows + 1, 77, 0, 0), (5, 6))
    for r in range(0, 50, 7):
        ref = _numpy_block((r + 1, 77, 0, 0), (5, 6))
        assert [int(w0[r]), int(w1[r]), int(w2[r]), int(w3[r])] == [int(x) for x in ref]


def test_mulhilo_exact():
    g = np.random.default_rng(1)
    a = g.integers(0, 2**63, 200, dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    b = g.integers(0, 2**63, 200, dtype=np.uint64)
    hi, lo = philox.mulhilo64(a, b)
    for i in range(200):
        p = int(a[i]) * int(b[i])
        assert int(hi[i]) == p >> 64 and int(lo[i]) == p & ((1 << 64) - 1)


def test_bf16_matches_torch():
    g = np.random.default_rng(2)
    x = np.concatenate([g.standard_normal(10000).astype(np.float32) * 100,
                        np.array([0.0, -0.0, 1e-40, -1e-40, 3.4e38, -3.4e38, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    out = bf16.round_bf16(x)
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))


def test_bf16_ties_to_even():
    one = np.float32(1.0)
    t1 = np.float32(1.0 + 2.0 ** -8)          # halfway between 1 and 1 + 2^-7 -> even (1)
    t2 = np.float32(1.0 + 3 * 2.0 ** -8)      # halfway between 1+2^-7 and 1+2^-6 -> 1+2^-6
    just_above = np.float32(1.0 + 2.0 ** -8 + 2.0 ** -20)
    out = bf16.round_bf16(np.array([t1, t2, just_above], np.float32))
    assert out[0] == one
    assert out[1] == np.float32(1.0 + 2.0 ** -6)
    assert out[2] == np.float32(1.0 + 2.0 ** -7)
    assert bf16.to_bits(np.array([np.nan], np.float32))[0] == 0x7FC0
