"""Pins of the oracle's HER relabelling and donor selection.

Each check is independent of the oracle's own code path: hand-worked values,
the pages' printed numbers, brute-force enumeration, range invariants and a
uniformity test of the multiply-shift mapping.
"""
import json
import os

import numpy as np
import pytest

from oracle import her, philox

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "her_hand.json")))


def _buf():
    return dict(states=np.array(GOLD["states"], np.float32),
                next_states=np.array(GOLD["next_states"], np.float32),
                actions=np.array(GOLD["actions"], np.int32),
                dones=np.array(GOLD["dones"], np.float32),
                episode_ends=np.array(GOLD["episode_ends"], np.int32),
                buffer_size=6)


def test_final_hand_worked():
    b, c = _buf(), GOLD["final"]
    out = her.her_step(b, c["source_idx"], GOLD["goal_dim"], her.FINAL, seed=1, step=0)
    assert out["donor_idx"].tolist() == c["donor_idx"]
    np.testing.assert_array_equal(out["states"], np.array(c["out_states"], np.float32))
    np.testing.assert_array_equal(out["next_states"], np.array(c["out_next_states"], np.float32))
    assert out["actions"].tolist() == c["out_actions"]
    np.testing.assert_array_equal(out["dones"], np.array(c["out_dones"], np.float32))
    np.testing.assert_array_equal(out["rewards"], np.array(c["out_rewards"], np.float32))


def test_given_donors_hand_worked():
    b, c = _buf(), GOLD["given_donors"]
    out = her.relabel(b["states"], b["next_states"], b["actions"], b["dones"],
                      c["source_idx"], c["donor_idx"], GOLD["goal_dim"])
    np.testing.assert_array_equal(out["states"], np.array(c["out_states"], np.float32))
    np.testing.assert_array_equal(out["next_states"], np.array(c["out_next_states"], np.float32))
    np.testing.assert_array_equal(out["rewards"], np.array(c["out_rewards"], np.float32))


def test_reward_metric_is_euclidean_strict():
    c = GOLD["metric_cases"]
    r = her.reward_decision(np.array(c["achieved"], np.float32), np.array(c["desired"], np.float32),
                            0.01, 1.0, -0.01)
    np.testing.assert_array_equal(r, np.array(c["rewards"], np.float32))
    # strict '<': a distance exactly at the float32 threshold misses
    thr = np.float32(0.01)
    r = her.reward_decision(np.array([[0.0]], np.float32), np.array([[thr]], np.float32), 0.01, 1.0, -0.01)
    assert r[0] == np.float32(-0.01)


def test_page_numbers():
    p = GOLD["page_numbers"]
    n = her.her_size(p["batch"], p["her_ratio"])
    assert n == p["her_rows"]
    assert 2 * n * p["state_dim"] * 4 == p["staging_bytes"]
    # truncation, not rounding
    assert her.her_size(3, 0.5) == 1
    assert her.her_size(10, 0.33) == 3
    assert her.her_size(4096, 0.25) == 1024
    assert her.her_size(16384, 0.0) == 0


def test_strategy_mapping():
    assert her.strategy_from_name("final") == her.FINAL
    assert her.strategy_from_name("future") == her.FUTURE
    assert her.strategy_from_name("episode") == her.RANDOM
    assert her.strategy_from_name("random") == her.RANDOM


def _episodes(n_ep, L):
    return (np.arange(n_ep) + 1) * L


def test_final_and_future_brute_force_ranges():
    # ragged episode lengths
    lens = np.array([1, 2, 5, 16, 3, 1, 7])
    ends = np.cumsum(lens).astype(np.int32)
    C = int(ends[-1])
    src = np.arange(C)
    fin = her.donors(her.FINAL, src, ends, C, seed=7, step=3)
    fut = her.donors(her.FUTURE, src, ends, C, seed=7, step=3)
    for s in range(C):  # brute force: scan the episode list
        e = next(k for k in range(len(ends)) if ends[k] > s)
        end = int(ends[e])
        assert fin[s] == end - 1
        if s + 1 < end:
            assert s + 1 <= fut[s] < end
        else:
            assert fut[s] == s  # empty future range -> the source itself


def test_random_range_and_step_dependence():
    src = np.zeros(5000, np.int64)
    ends = np.array([5000], np.int32)
    a = her.donors(her.RANDOM, src, ends, 4321, seed=11, step=0)
    b = her.donors(her.RANDOM, src, ends, 4321, seed=11, step=1)
    assert a.min() >= 0 and a.max() < 4321
    assert np.mean(a == b) < 0.01


def test_multiply_shift_mapping():
    # r = 2^63 maps to floor(span / 2); r = 2^64 - 1 maps to span - 1; r = 0 to lo
    r = np.array([1 << 63, (1 << 64) - 1, 0], dtype=np.uint64)
    idx = philox.uniform_index(r, 10, np.uint64(7))
    assert idx.tolist() == [10 + 3, 10 + 6, 10]
    big = np.uint64((1 << 40) + 3)
    idx = philox.uniform_index(np.array([1 << 62], np.uint64), 0, big)
    assert int(idx[0]) == ((1 << 40) + 3) // 4


def test_future_uniformity_chi_square():
    # one long episode, a fixed source: donors should be uniform over the range
    n = 60000
    span = 50
    src = np.zeros(n, np.int64)
    ends = np.array([span + 1], np.int32)
    d = her.donors(her.FUTURE, src, ends, span + 1, seed=3, step=9)
    counts = np.bincount(d - 1, minlength=span)
    exp = n / span
    chi2 = float(np.sum((counts - exp) ** 2 / exp))
    # 49 dof: P(chi2 > 90) < 1e-3
    assert chi2 < 90.0


def test_non_goal_columns_bitwise_and_goal_from_donor_next_state():
    g = np.random.default_rng(0)
    C, S, G = 64, 9, 3
    st = g.standard_normal((C, S)).astype(np.float32)
    ns = g.standard_normal((C, S)).astype(np.float32)
    src = g.integers(0, C, 40)
    don = g.integers(0, C, 40)
    out = her.relabel(st, ns, np.zeros(C, np.int32), np.zeros(C, np.float32), src, don, G)
    assert np.array_equal(out["states"][:, G:].view(np.uint32), st[src, G:].view(np.uint32))
    assert np.array_equal(out["next_states"][:, G:].view(np.uint32), ns[src, G:].view(np.uint32))
    assert np.array_equal(out["states"][:, :G].view(np.uint32), ns[don, :G].view(np.uint32))
    assert np.array_equal(out["next_states"][:, :G].view(np.uint32), ns[don, :G].view(np.uint32))
    assert set(np.unique(out["rewards"]).tolist()) <= {np.float32(1.0), np.float32(-0.01)}
    same = her.relabel(st, ns, np.zeros(C, np.int32), np.zeros(C, np.float32), src, src, G)
    assert np.all(same["rewards"] == np.float32(1.0))  # own achieved goal -> +1


def test_episode_lookup_rejects_out_of_range():
    with pytest.raises(ValueError):
        her.episode_bounds(np.array([10]), np.array([5, 10]))


def test_merged_importance_weights():
    """HER rows enter the merged batch with importance weight 1 after the
    prioritized rows, which keep their own weights ("How HER Interacts with
    GPU PER"); at the pages' batch 256 and ratio 0.5 that is 128 ones after
    128 prioritized weights."""
    p = GOLD["page_numbers"]
    n = her.her_size(p["batch"], p["her_ratio"])
    w_normal = np.linspace(0.1, 1.0, p["batch"] - n).astype(np.float32)
    w = her.merged_is_weights(w_normal, n)
    assert w.shape == (p["batch"],) and w.dtype == np.float32
    assert np.array_equal(w[: p["batch"] - n], w_normal)
    assert np.all(w[p["batch"] - n:] == np.float32(1.0))
    # relabel returns one weight of exactly 1 per relabelled row
    g = np.random.default_rng(0)
    s = g.standard_normal((10, 4)).astype(np.float32)
    out = her.relabel(s, s, np.zeros(10, np.int32), np.zeros(10, np.float32), [1, 2, 3], [4, 5, 6], 2)
    assert np.array_equal(out["is_weights"], np.ones(3, np.float32))
