"""GPU parity of her_relabel against the oracle: bit-exact donors, relabelled
states (f32 and bf16), next states, actions, dones and rewards."""
import numpy as np
import pytest

import synth
from oracle import her
from tests.gpu_util import dev, host, sync, to_dev

pytestmark = pytest.mark.gpu

STRATS = {"final": 0, "future": 1, "random": 2}


def _run(m, buf, src, G, strategy, seed, step, out_bf16, ld=None, merged_rows=0, flags=None):
    import torch
    S = buf["states"].shape[1]
    n = len(src)
    ld = S if ld is None else ld
    d = dev()
    t_states = to_dev(buf["states"])
    t_next = to_dev(buf["next_states"])
    t_act = to_dev(buf["actions"])
    t_done = to_dev(buf["dones"])
    t_ends = to_dev(buf["episode_ends"].astype(np.int32))
    t_src = to_dev(np.asarray(src, np.int32))
    t_step = torch.tensor([step], dtype=torch.int64, device=d)
    odt = torch.bfloat16 if out_bf16 else torch.float32
    X = torch.full((merged_rows + n, ld), 7.0, dtype=odt, device=d)  # sentinel outside the written block
    o_next = torch.zeros((n, S), dtype=torch.float32, device=d)
    o_act = torch.zeros(n, dtype=torch.int32, device=d)
    o_rew = torch.zeros(n, dtype=torch.float32, device=d)
    o_done = torch.zeros(n, dtype=torch.float32, device=d)
    o_don = torch.zeros(n, dtype=torch.int32, device=d)
    W = torch.full((merged_rows + n,), 7.0, dtype=torch.float32, device=d)  # the merged batch's IS weights
    cfg = m.her_config(S, G, strategy)
    hb = m.her_buffer(t_states, t_next, t_act, t_done, t_ends, buffer_size=buf["buffer_size"])
    tail = X.data_ptr() + merged_rows * ld * X.element_size()
    ho = m.her_out(tail, m.BF16 if out_bf16 else m.F32, ld, o_rew, next_states=o_next, actions=o_act,
                   dones=o_done, donor_idx=o_don, d_flags=flags,
                   is_weights=W.data_ptr() + merged_rows * W.element_size())
    m.her_relabel(cfg, hb, t_src, n, seed, t_step, ho)
    sync()
    return dict(X=X, states=X[merged_rows:, :S], next_states=o_next, actions=o_act, rewards=o_rew,
                dones=o_done, donor_idx=o_don, W=W, is_weights=W[merged_rows:])


def _compare(got, ref, out_bf16):
    assert np.array_equal(host(got["donor_idx"]), ref["donor_idx"])
    gs = host(got["states"]).astype(np.float32)
    assert np.array_equal(gs.view(np.uint32), ref["states"].view(np.uint32))
    assert np.array_equal(host(got["next_states"]).view(np.uint32), ref["next_states"].view(np.uint32))
    assert np.array_equal(host(got["actions"]), ref["actions"])
    assert np.array_equal(host(got["dones"]), ref["dones"])
    assert np.array_equal(host(got["rewards"]).view(np.uint32), ref["rewards"].view(np.uint32))
    assert np.array_equal(host(got["is_weights"]).view(np.uint32), ref["is_weights"].view(np.uint32))


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


@pytest.mark.parametrize("strategy", ["final", "future", "random"])
@pytest.mark.parametrize("out_bf16", [False, True])
def test_her_tiny(m, strategy, out_bf16):
    w = synth.WORKLOADS["tiny_b256_s16_h32"]
    buf = synth.replay_buffer(w)
    src = synth.her_sources(w, buf)
    for step in (0, 1, 57):
        ref = her.her_step(buf, src, w.G, STRATS[strategy], seed=123, step=step, out_bf16=out_bf16)
        got = _run(m, buf, src, w.G, STRATS[strategy], 123, step, out_bf16)
        _compare(got, ref, out_bf16)


@pytest.mark.parametrize("strategy", ["final", "future", "random"])
def test_her_ragged_episodes_and_merged_batch(m, strategy):
    g = np.random.default_rng(4)
    lens = g.integers(1, 40, size=300)
    ends = np.cumsum(lens).astype(np.int32)
    C, S, G = int(ends[-1]), 42, 8
    buf = dict(states=g.standard_normal((C, S), dtype=np.float32),
               next_states=g.standard_normal((C, S), dtype=np.float32),
               actions=g.integers(0, 9, C, dtype=np.int32), dones=np.zeros(C, np.float32),
               episode_ends=ends, buffer_size=C)
    buf["dones"][ends - 1] = 1.0
    # every last step of an episode plus random rows: exercises the empty future range
    src = np.concatenate([ends - 1, g.integers(0, C, 1500)]).astype(np.int32)
    ref = her.her_step(buf, src, G, STRATS[strategy], seed=99, step=3, out_bf16=True)
    got = _run(m, buf, src, G, STRATS[strategy], 99, 3, True, ld=48, merged_rows=777)
    _compare(got, ref, True)
    # rows before the HER block and the padding columns are untouched
    X = host(got["X"])
    assert np.all(X[:777] == 7.0) and np.all(X[777:, S:] == 7.0)
    # the merged weights: the prioritized rows' own weights (here the 7.0
    # sentinel), then 1 for every HER row
    Wm = host(got["W"])
    assert np.array_equal(Wm, her.merged_is_weights(np.full(777, 7.0, np.float32), len(src)))


# float32 bit patterns at the edges of round-to-nearest-even to bfloat16
EDGE_BITS = np.array([0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0xBF818000, 0x00000001, 0x00008000,
                      0x00018000, 0x007FFFFF, 0x807FFFFF, 0x7F7FFFFF, 0x7F7F7FFF, 0xFF7FFFFF, 0x7F800000,
                      0xFF800000, 0x80000000, 0x7FC00000, 0x7F800001, 0xFFC12345, 0x7FFFFFFF], np.uint32)


@pytest.mark.parametrize("S", [48, 45])
def test_her_bf16_rounding_edges(m, S):
    """Relabelled states stored as bfloat16 round to nearest even exactly as
    the oracle does at ties (even and odd), near ties, denormals, overflow to
    infinity, infinities, signed zero and NaN (quiet, signalling, negative,
    with payloads: all 0x7FC0); S = 48 takes the paired stores, 45 the
    element stores."""
    g = np.random.default_rng(8)
    C, G = 512, 6
    ends = np.arange(16, C + 1, 16, dtype=np.int32)
    states = g.standard_normal((C, S), dtype=np.float32)
    cols = np.arange(G, S)
    edge = EDGE_BITS[(np.arange(C)[:, None] + cols[None, :]) % EDGE_BITS.size].view(np.float32)
    states[:, G:] = edge
    buf = dict(states=states, next_states=g.standard_normal((C, S), dtype=np.float32),
               actions=g.integers(0, 4, C, dtype=np.int32), dones=np.zeros(C, np.float32),
               episode_ends=ends, buffer_size=C)
    src = g.integers(0, C, 700).astype(np.int32)
    ref = her.her_step(buf, src, G, her.FUTURE, seed=31, step=2, out_bf16=True)
    got = _run(m, buf, src, G, her.FUTURE, 31, 2, True)
    _compare(got, ref, True)


def test_her_equal_goals_reward_hit(m):
    w = synth.shrink(synth.WORKLOADS["stress_b65536_s256_h512_bf16"], B=4096, C=1 << 14)
    buf = synth.replay_buffer(w)
    src = synth.her_sources(w, buf)
    ref = her.her_step(buf, src, w.G, her.FUTURE, seed=5, step=0, out_bf16=True)
    got = _run(m, buf, src, w.G, her.FUTURE, 5, 0, True)
    _compare(got, ref, True)
    # at least the constant-goal share of sources (and the empty-range ones) hit
    assert np.mean(ref["rewards"] == np.float32(1.0)) >= 0.09


def test_her_full_size_bf16_future(m):
    w = synth.WORKLOADS["b16384_s128_h128_bf16_g2"]
    buf = synth.replay_buffer(w)
    src = synth.her_sources(w, buf)
    ref = her.her_step(buf, src, w.G, her.FUTURE, seed=synth.DEFAULT_SEED, step=11, out_bf16=True)
    got = _run(m, buf, src, w.G, her.FUTURE, synth.DEFAULT_SEED, 11, True, merged_rows=w.B - w.n_her)
    _compare(got, ref, True)


def test_her_bad_index_flag(m):
    import torch
    w = synth.WORKLOADS["tiny_b256_s16_h32"]
    buf = synth.replay_buffer(w)
    src = np.array([3, -1, 10, 256, 5], np.int32)  # -1 and 256 are outside the buffer
    flags = torch.zeros(1, dtype=torch.int32, device=dev())
    got = _run(m, buf, src, w.G, her.FUTURE, 1, 0, False, flags=flags)
    assert int(flags.item()) & m.FLAG_BAD_INDEX
    don = host(got["donor_idx"])
    assert don[1] == -1 and don[3] == -1
    assert np.all(host(got["states"])[[1, 3]] == 0.0) and np.all(host(got["rewards"])[[1, 3]] == 0.0)
    assert np.array_equal(host(got["is_weights"]), np.array([1, 0, 1, 0, 1], np.float32))
    ok = np.array([0, 2, 4])
    safe = np.where((src >= 0) & (src < w.C), src, 0)
    ref = her.her_step(buf, safe, w.G, her.FUTURE, seed=1, step=0)
    assert np.array_equal(don[ok], ref["donor_idx"][ok])
    assert np.array_equal(host(got["rewards"])[ok], ref["rewards"][ok])
    assert np.array_equal(host(got["states"])[ok], ref["states"][ok])


@pytest.mark.parametrize("S,G", [(96, 40), (80, 72), (20, 0), (12, 12)])
@pytest.mark.parametrize("strategy", ["final", "future"])
def test_her_goal_widths_ragged(m, S, G, strategy):
    """Goals wider than the 16 entries loaded with the episode probe, wider
    than the 64 staged per row, empty, and rows narrower than 16 entries; the
    episodes are ragged, so many guessed donors miss and are reloaded."""
    g = np.random.default_rng(S * 100 + G)
    lens = g.integers(1, 30, size=200)
    ends = np.cumsum(lens).astype(np.int32)
    C = int(ends[-1])
    buf = dict(states=g.standard_normal((C, S), dtype=np.float32),
               next_states=g.standard_normal((C, S), dtype=np.float32),
               actions=g.integers(0, 9, C, dtype=np.int32), dones=np.zeros(C, np.float32),
               episode_ends=ends, buffer_size=C)
    buf["dones"][ends - 1] = 1.0
    src = g.integers(0, C, 700).astype(np.int32)
    ref = her.her_step(buf, src, G, STRATS[strategy], seed=7, step=2, out_bf16=False)
    got = _run(m, buf, src, G, STRATS[strategy], 7, 2, False)
    _compare(got, ref, False)
