"""Pins of the non-finite sentinel oracle: IEEE-754 special values decided
on their bit patterns agree with the definitions (NaN and infinities are
non-finite; the largest finite value, subnormals and negative zero are
finite), and the slot flags are sticky and skip null entries."""
import numpy as np

from oracle import sentinel


def test_special_values():
    f32 = np.float32
    vals = np.array([np.nan, np.inf, -np.inf, np.finfo(f32).max, -np.finfo(f32).max, np.finfo(f32).tiny,
                     f32(1e-45), -0.0, 0.0, 1.0], dtype=np.float32)
    np.testing.assert_array_equal(sentinel.is_nonfinite_bits(vals), [1, 1, 1, 0, 0, 0, 0, 0, 0, 0])
    # every NaN payload, both signs
    bits = np.array([0x7F800001, 0x7FC00000, 0x7FFFFFFF, 0xFF800001, 0xFFFFFFFF], dtype=np.uint32)
    assert np.all(sentinel.is_nonfinite_bits(bits.view(np.float32)))
    # agrees with numpy's isfinite on a sweep of random bit patterns
    r = np.random.default_rng(0).integers(0, 1 << 32, 100000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    np.testing.assert_array_equal(sentinel.is_nonfinite_bits(r), ~np.isfinite(r))


def test_flags_are_sticky_and_skip_null_entries():
    clean = np.ones(10, np.float32)
    dirty = clean.copy()
    dirty[7] = np.nan
    f = sentinel.update_flags([0, 0, 0], [clean, dirty, None])
    np.testing.assert_array_equal(f, [0, 1, 0])
    f = sentinel.update_flags(f, [clean, clean, np.array([np.inf], np.float32)])
    np.testing.assert_array_equal(f, [0, 1, 1])  # slot 1 stays set on clean data
