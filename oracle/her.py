"""Hindsight Experience Replay relabelling, CPU reference.

Source: "GPU IQL + HER Porting Plan"
  * section "Current State / HER (CPU)": the goal is the first ``goal_dim``
    entries of the state; a relabelled transition gets the achieved goal of
    another experience; sparse reward +1.0 when the goal distance is below
    0.01, -0.01 otherwise; ``her_ratio`` of the batch is relabelled.
  * section "CUDA Kernel: her_relabel_kernel.cu": per relabelled row, copy
    state and next_state of the source, overwrite the goal entries of BOTH with
    the donor's next_state goal, copy action and done, and recompute the
    reward from the Euclidean distance between the source's own next_state
    goal and the donor's next_state goal.
  * section "Donor Index Generation": final = last experience of the source's
    episode; future = uniform in [source + 1, episode_end); random = uniform
    over the whole buffer.
  * section "How HER Interacts with GPU PER": her_size = batch * her_ratio
    (float multiply then truncation), normal rows first, HER rows appended,
    importance weights 1 for HER rows.

Readings where the page is silent:
  * ``episode_ends`` are exclusive and ascending; the episode of ``src`` is the
    first e with episode_ends[e] > src; episode e starts at episode_ends[e-1].
  * future with an empty range (src is the episode's last step) uses the
    source itself as donor.
  * the random draw is word 0 of Philox4x64-10 with key (seed, HER_KEY1) and
    counter (row, step, 0, 0), mapped by floor(r * span / 2**64).
  * the reward decision is taken in float32 exactly as the page's kernel
    spells it: sequential float32 sum of squared differences (no fused
    multiply-add), float32 square root, strict ``<`` against the float32
    threshold.
"""
import numpy as np

from . import philox
from . import bf16 as _bf16

FINAL, FUTURE, RANDOM = 0, 1, 2
HER_KEY1 = 0x484552646F6E6F72  # second key word of the donor stream ("HERdonor")


def strategy_from_name(name):
    """'final' -> FINAL, 'future' -> FUTURE, anything else -> RANDOM
    (section "Config Wiring" of the HER part)."""
    if name == "final":
        return FINAL
    if name == "future":
        return FUTURE
    return RANDOM


def her_size(batch_size, her_ratio):
    """Number of relabelled rows: float multiply, truncation."""
    return int(float(batch_size) * float(her_ratio))


def episode_bounds(src, episode_ends):
    """(start, end) of the episode holding each source index."""
    ends = np.asarray(episode_ends, dtype=np.int64)
    src = np.asarray(src, dtype=np.int64)
    e = np.searchsorted(ends, src, side="right")
    if np.any(e >= len(ends)):
        raise ValueError("source index beyond the last episode end")
    end = ends[e]
    start = np.where(e > 0, ends[np.maximum(e - 1, 0)], 0)
    return start, end


def random_words(n, seed, step):
    """Word 0 of Philox4x64-10 for rows 0..n-1 at the given step."""
    rows = np.arange(n, dtype=np.uint64)
    w0, _, _, _ = philox.philox4x64((rows, np.uint64(step), 0, 0),
                                    (np.uint64(seed), np.uint64(HER_KEY1)))
    return w0


def donors(strategy, source_idx, episode_ends, buffer_size, seed, step):
    """Donor index per relabelled row (int64 array)."""
    src = np.asarray(source_idx, dtype=np.int64)
    n = src.shape[0]
    if strategy == RANDOM:
        r = random_words(n, seed, step)
        return philox.uniform_index(r, 0, np.uint64(buffer_size))
    _, end = episode_bounds(src, episode_ends)
    if strategy == FINAL:
        return end - 1
    if strategy == FUTURE:
        r = random_words(n, seed, step)
        span = end - src - 1
        pick = philox.uniform_index(r, src + 1, np.maximum(span, 1).astype(np.uint64))
        return np.where(span > 0, pick, src)
    raise ValueError("unknown strategy")


def reward_decision(achieved, desired, threshold, reward_hit, reward_miss):
    """Sparse reward in float32, summing squared differences in goal order."""
    a = np.asarray(achieved, dtype=np.float32)
    d = np.asarray(desired, dtype=np.float32)
    acc = np.zeros(a.shape[0], dtype=np.float32)
    for k in range(a.shape[1]):
        diff = (a[:, k] - d[:, k]).astype(np.float32)
        sq = (diff * diff).astype(np.float32)
        acc = (acc + sq).astype(np.float32)
    dist = np.sqrt(acc).astype(np.float32)
    hit = dist < np.float32(threshold)
    return np.where(hit, np.float32(reward_hit), np.float32(reward_miss)).astype(np.float32)


def relabel(states, next_states, actions, dones, source_idx, donor_idx, goal_dim,
            threshold=0.01, reward_hit=1.0, reward_miss=-0.01, out_bf16=False):
    """Relabel the rows named by source_idx with the goals of donor_idx.

    Returns dict(states, next_states, actions, rewards, dones, is_weights).
    ``is_weights`` is 1 per row (relabelled rows are not sampled by
    priority, section "How HER Interacts with GPU PER").  ``states`` is
    float32, or float32 holding bfloat16-rounded values when ``out_bf16``.
    """
    src = np.asarray(source_idx, dtype=np.int64)
    don = np.asarray(donor_idx, dtype=np.int64)
    G = int(goal_dim)
    out_s = np.array(states[src], dtype=np.float32, copy=True)
    out_ns = np.array(next_states[src], dtype=np.float32, copy=True)
    goal = np.asarray(next_states[don, :G], dtype=np.float32)
    out_s[:, :G] = goal
    out_ns[:, :G] = goal
    rew = reward_decision(next_states[src, :G], goal, threshold, reward_hit, reward_miss)
    if out_bf16:
        out_s = _bf16.round_bf16(out_s)
    return dict(states=out_s, next_states=out_ns,
                actions=np.asarray(actions[src], dtype=np.int32),
                rewards=rew,
                dones=np.asarray(dones[src], dtype=np.float32),
                is_weights=np.ones(src.shape[0], dtype=np.float32))


def merged_is_weights(normal_is_weights, n_her):
    """Importance-sampling weights of the merged batch ("How HER Interacts
    with GPU PER"): the prioritized rows keep their own weights and come
    first; the relabelled rows are not drawn by priority and weigh 1 each."""
    w = np.asarray(normal_is_weights, dtype=np.float32)
    return np.concatenate([w, np.ones(int(n_her), dtype=np.float32)])


def her_step(buffer, source_idx, goal_dim, strategy, seed, step, **kw):
    """Donor selection followed by relabelling (one HER pass)."""
    don = donors(strategy, source_idx, buffer["episode_ends"], buffer["buffer_size"], seed, step)
    out = relabel(buffer["states"], buffer["next_states"], buffer["actions"], buffer["dones"],
                  source_idx, don, goal_dim, **kw)
    out["donor_idx"] = don.astype(np.int32)
    return out
