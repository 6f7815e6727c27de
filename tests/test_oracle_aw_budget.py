"""Pins of the oracle's advantage-weighted policy and gradient budget.

AW policy: rows sum to 1, beta = 0 gives the uniform policy, shift invariance
without an active clamp, all-clamped rows are uniform, a +1e3 outlier at
beta = 10 is one-hot, no overflow, and ``scipy.special.softmax`` on the clamped
logits (library special case).
Budget: the fractions 0.70/0.15/0.10/0.05 sum to 1 so the total norm is
bounded by max_grad_norm; each clipped contribution has norm
min(n_k, f_k * mgn) and the direction of its source; with every source inside
its budget the result is the plain alpha-weighted sum.
"""
import numpy as np
import pytest
import scipy.special

from oracle import aw, budget, iql


def test_rows_sum_to_one_and_scipy():
    g = np.random.default_rng(0)
    Q, V = g.standard_normal((300, 9)) * 3, g.standard_normal(300)
    pi = aw.aw_policy(Q, V, 3.0)
    np.testing.assert_allclose(pi.sum(1), 1.0, rtol=1e-14)
    ref = scipy.special.softmax(3.0 * np.clip(Q - V[:, None], -10, 10), axis=1)
    np.testing.assert_allclose(pi, ref, rtol=1e-13)


def test_beta_zero_uniform():
    g = np.random.default_rng(1)
    pi = aw.aw_policy(g.standard_normal((50, 7)) * 100, g.standard_normal(50), 0.0)
    np.testing.assert_allclose(pi, 1.0 / 7, rtol=1e-15)


def test_shift_invariance_without_clamp():
    g = np.random.default_rng(2)
    Q, V = g.standard_normal((40, 5)), g.standard_normal(40) * 0.1
    a = aw.aw_policy(Q, V, 2.0)
    b = aw.aw_policy(Q + 1.5, V + 1.5, 2.0)
    np.testing.assert_allclose(a, b, rtol=1e-13)


def test_clamp_before_beta():
    # all gaps >= 10 -> uniform; clamp applies to Q - V, not to beta * (Q - V)
    Q = np.array([[20.0, 11.0, 10.0, 500.0]])
    np.testing.assert_allclose(aw.aw_policy(Q, np.zeros(1), 3.0), 0.25, rtol=1e-15)
    Q = np.array([[4.0, 0.0]])  # gap 4 < 10 but beta * gap = 12 > 10
    pi = aw.aw_policy(Q, np.zeros(1), 3.0)
    assert pi[0, 0] == pytest.approx(1.0 / (1.0 + np.exp(-12.0)), rel=1e-14)


def test_outlier_one_hot_no_overflow():
    Q = np.zeros((2, 16))
    Q[0, 3] = 1e3
    Q[1, 5] = -1e3
    pi = aw.aw_policy(Q, np.zeros(2), 10.0)
    assert np.all(np.isfinite(pi))
    assert pi[0, 3] == pytest.approx(1.0, abs=1e-40)
    assert pi[0, 3] == pytest.approx(1.0 / (1.0 + 15.0 * np.exp(-100.0)), rel=1e-15)
    assert pi[1, 5] == pytest.approx(np.exp(-100.0) / (15.0 + np.exp(-100.0)), rel=1e-12)


# ------------------------------------------------------------------ budget
def _sources(n, scales, seed=0):
    g = np.random.default_rng(seed)
    return [g.standard_normal(n) * s for s in scales]


def test_fractions_sum_to_one():
    assert sum(budget.FRACTIONS) == pytest.approx(1.0, abs=1e-15)


def test_budget_bounds_total_norm():
    for seed in range(5):
        src = _sources(5000, (1, 5, 0.5, 0.2), seed)
        grad, norms, comb, scales = budget.accumulate(src, budget.FRACTIONS, (1, 1, 1, 1), 1.0)
        assert comb <= 1.0 * (1 + 1e-12)
        # Adam's safety clip therefore never fires
        assert iql.clip_coef(comb, 1.0) == 1.0
        for s, n, c, f in zip(src, norms, scales, budget.FRACTIONS):
            assert n == pytest.approx(np.linalg.norm(s), rel=1e-13)
            contrib = c * s
            assert np.linalg.norm(contrib) == pytest.approx(min(n, f * 1.0), rel=1e-12)
            cos = contrib @ s / (np.linalg.norm(contrib) * np.linalg.norm(s))
            assert cos == pytest.approx(1.0, abs=1e-12)


def test_budget_inside_budgets_is_plain_sum():
    src = _sources(300, (1e-4, 1e-4, 1e-4, 1e-4), 3)
    alphas = (1.0, 1.0, 0.5, 2.0)
    grad, _, _, scales = budget.accumulate(src, budget.FRACTIONS, alphas, 1.0)
    assert scales == [1.0, 1.0, 1.0, 1.0]
    np.testing.assert_allclose(grad, sum(a * s for a, s in zip(alphas, src)), rtol=1e-15)


def test_budget_hand_worked():
    # primary (3, 4): norm 5 > 0.7 -> scaled to norm 0.7 -> (0.42, 0.56)
    # second (0, 0.1): norm 0.1 <= 0.15 -> unchanged; alpha 2 -> (0, 0.2)
    # third (0.3, 0): norm 0.3 is below max_grad_norm but above its budget
    #   0.10 -> scaled to (0.1, 0)
    grad, norms, comb, scales = budget.accumulate(
        [np.array([3.0, 4.0]), np.array([0.0, 0.1]), np.array([0.3, 0.0])],
        (0.70, 0.15, 0.10), (1.0, 2.0, 1.0), 1.0)
    np.testing.assert_allclose(grad, [0.52, 0.76], rtol=1e-14)
    assert norms == pytest.approx([5.0, 0.1, 0.3])
    assert comb == pytest.approx(np.hypot(0.52, 0.76), rel=1e-14)


def test_unbudgeted_example_from_pages():
    # each source clipped at the full max_grad_norm and added with weights
    # 1, lambda, s sums to up to (1 + lambda + s) * mgn; 1.35 x mgn -> 26% cut
    bound = 1.0 + 0.25 + 0.10
    assert 1.0 - iql.clip_coef(bound, 1.0) == pytest.approx(0.26, abs=1e-3)
