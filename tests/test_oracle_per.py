"""Pins of the prioritized-replay sampling oracle: the inverse-transform
search against a brute-force scan, the draw frequencies against the
priorities (chi-square), zero-priority rows never drawn, the IS weights
against their definition (N P(i))^-beta / max and hand-worked values, and
the uniform words against numpy's own Philox."""
import numpy as np
import pytest

from oracle import per, philox


def test_search_matches_brute_force_scan():
    g = np.random.default_rng(0)
    p = g.random(37) * (g.random(37) < 0.8)
    idx, w, u, prefix = per.sample(p, 500, seed=5, step=2, beta=0.4)
    for k in range(500):
        acc, want = 0.0, None
        for i, pi in enumerate(p):
            acc += pi
            if acc > u[k]:
                want = i
                break
        assert idx[k] == want
    assert np.all(p[idx] > 0)


def test_frequencies_follow_priorities():
    p = np.array([1.0, 0.0, 2.0, 4.0, 0.5, 0.0, 2.5])
    n = 200000
    idx, _, _, _ = per.sample(p, n, seed=11, step=0, beta=0.0)
    counts = np.bincount(idx, minlength=p.size)
    expect = n * p / p.sum()
    assert counts[1] == 0 and counts[5] == 0
    nz = expect > 0
    chi2 = np.sum((counts[nz] - expect[nz]) ** 2 / expect[nz])
    assert chi2 < 22.5  # 5 degrees of freedom, p ~ 0.0004


def test_importance_weights_definition():
    g = np.random.default_rng(1)
    p = g.random(1000) + 0.01
    beta = 0.6
    idx, w, _, _ = per.sample(p, 256, seed=3, step=7, beta=beta)
    P = p / p.sum()
    raw = (p.size * P[idx]) ** (-beta)
    np.testing.assert_allclose(w, raw / raw.max(), rtol=1e-12)
    assert w.max() == 1.0
    # two rows of priority 1 and 3 drawn: weights 1 and (1/3)^beta
    idx, w, _, _ = per.sample([1.0, 3.0], 64, seed=1, step=0, beta=0.5)
    assert set(idx) == {0, 1}
    np.testing.assert_allclose(w[idx == 0], 1.0)
    np.testing.assert_allclose(w[idx == 1], (1.0 / 3.0) ** 0.5)
    # uniform priorities: every weight 1
    _, w, _, _ = per.sample(np.full(50, 2.5), 100, seed=2, step=1, beta=0.9)
    np.testing.assert_array_equal(w, 1.0)


def test_uniform_words_are_philox_word_zero():
    """Word 0 of numpy's independent Philox4x64-10 at the same counter and
    key (numpy pre-increments its counter: start one block earlier)."""
    n, seed, step = 64, 123, 9
    u = per.uniforms(n, seed, step)
    for k in (0, 1, 17, 63):
        c = np.array([k, step, 0, 0], dtype=np.uint64)
        for i in range(4):  # counter - 1 with borrow
            if c[i] != 0:
                c[i] -= np.uint64(1)
                break
            c[i] = np.uint64(0xFFFFFFFFFFFFFFFF)
        w0 = np.random.Philox(counter=c, key=np.array([seed, per.PER_KEY1], dtype=np.uint64)).random_raw(1)[0]
        assert u[k] == float(w0 >> np.uint64(11)) * 2.0 ** -53


def test_search_takes_the_first_prefix_exceeding_u():
    """The row is the first whose inclusive prefix exceeds u: at u equal to a
    prefix value the next row of positive priority is taken, a leading or
    inner row of priority 0 is never found (brute force over exact values)."""
    p = np.array([0.0, 1.0, 0.0, 0.0, 2.0, 0.5, 0.0])
    prefix = np.cumsum(p)
    us = np.array([0.0, 0.5, 1.0, 2.9, 3.0, 3.25, np.nextafter(3.5, 0)])
    got = per.find_rows(prefix, us)
    brute = [next(i for i in range(len(p)) if prefix[i] > u) for u in us]
    np.testing.assert_array_equal(got, brute)
    np.testing.assert_array_equal(got, [1, 1, 4, 4, 5, 5, 5])
    assert np.all(p[got] > 0)
