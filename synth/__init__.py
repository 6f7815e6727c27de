"""Seeded synthetic inputs for the IQL + HER step.

Shared by the tests, ``bench.py`` and the oracle's CPU timing.  This module
only draws numbers and lays them out; it contains none of the method's
arithmetic (no relabelling, no network, no loss, no clipping).

All draws use NumPy ``Generator(PCG64(seed))``.  The workloads mirror the
shapes of the pages' production setting (batch 16384, value-MLP hidden 128,
grouped high/low trainers) and smaller / larger cases around it; the market
data the pages train on is proprietary and replaced by Gaussian draws.
"""
from dataclasses import dataclass, field, replace

import numpy as np

DEFAULT_SEED = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    B: int                 # merged batch (normal + HER rows)
    S: int                 # state_dim
    G: int                 # goal_dim (first G state entries)
    H: int                 # value-MLP first hidden width (and second when H2 is 0)
    A: int                 # number of actions
    dtype: str             # "f32" or "bf16" GEMM operand type
    groups: int            # independent IQL trainers sharing the batch
    taus: tuple            # expectile tau per group
    beta: float            # advantage temperature
    her_ratio: float
    strategy: str          # "final" | "future" | "random"
    L: int                 # episode length in the replay buffer
    C: int                 # replay buffer rows (consecutive episodes)
    q_sd: float = 1.0
    q_outlier_frac: float = 0.0
    q_outlier_mag: float = 0.0
    const_goal_frac: float = 0.0   # share of HER sources from constant-goal episodes
    lr: float = 3e-4
    max_grad_norm: float = 1.0
    steps: int = 1
    budget: bool = False
    budget_scales: tuple = (1.0, 5.0, 0.5, 0.2)
    budget_fractions: tuple = (0.70, 0.15, 0.10, 0.05)
    H2: int = 0            # second hidden width, 0 = H

    @property
    def n_her(self):
        return int(float(self.B) * float(self.her_ratio))

    @property
    def hidden2(self):
        return self.H2 or self.H

    @property
    def n_params(self):
        S, H1, H2 = self.S, self.H, self.hidden2
        return S * H1 + H1 + H2 * H1 + H2 + H2 + 1

    @property
    def n_budget(self):
        # parameter count of the network the budgeted gradient belongs to
        return 4 * self.n_params


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_b256_s16_h32", B=256, S=16, G=4, H=32, A=4, dtype="f32", groups=1,
                 taus=(0.7,), beta=3.0, her_ratio=0.5, strategy="future", L=16, C=256,
                 q_sd=1.0, steps=1),
        Workload("b4096_s42_h128_f32", B=4096, S=42, G=8, H=128, A=9, dtype="f32", groups=1,
                 taus=(0.7,), beta=3.0, her_ratio=0.25, strategy="final", L=64, C=4096,
                 q_sd=2.0, steps=100),
        Workload("b16384_s128_h128_bf16_g2", B=16384, S=128, G=8, H=128, A=9, dtype="bf16",
                 groups=2, taus=(0.7, 0.7), beta=3.0, her_ratio=0.5, strategy="future",
                 L=64, C=1 << 20, q_sd=1.0, steps=200),
        Workload("b16384_s128_h128_bf16_g2_budget", B=16384, S=128, G=8, H=128, A=9,
                 dtype="bf16", groups=2, taus=(0.7, 0.7), beta=3.0, her_ratio=0.5,
                 strategy="future", L=64, C=1 << 20, q_sd=1.0, steps=1000, budget=True),
        Workload("stress_b65536_s256_h512_bf16", B=65536, S=256, G=16, H=512, A=16,
                 dtype="bf16", groups=1, taus=(0.9,), beta=10.0, her_ratio=0.5,
                 strategy="future", L=64, C=1 << 20, q_sd=1.0, q_outlier_frac=0.05,
                 q_outlier_mag=1e3, const_goal_frac=0.10, steps=200),
    ]
}

BENCH_WORKLOAD = "b16384_s128_h128_bf16_g2_budget"


def shrink(w, **kw):
    """Same workload recipe at other sizes (for oracle-speed parity cases)."""
    return replace(w, **kw)


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _bf16_values(x32):
    """Round float32 draws to bfloat16-representable float32 values (storage)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def replay_buffer(w, seed=DEFAULT_SEED):
    """C rows of consecutive length-L episodes; s, s' ~ N(0, 1) float32."""
    g = rng(seed)
    C, S = w.C, w.S
    states = g.standard_normal((C, S), dtype=np.float32)
    next_states = g.standard_normal((C, S), dtype=np.float32)
    actions = g.integers(0, w.A, size=C, dtype=np.int32)
    n_ep = (C + w.L - 1) // w.L
    episode_ends = np.minimum((np.arange(n_ep, dtype=np.int64) + 1) * w.L, C).astype(np.int32)
    dones = np.zeros(C, dtype=np.float32)
    dones[episode_ends - 1] = 1.0
    rewards = g.standard_normal(C, dtype=np.float32)  # never read by the method
    const_eps = np.zeros(0, dtype=np.int64)
    if w.const_goal_frac > 0.0:
        # constant-goal episodes: every next_state of the episode shares one goal
        n_const = max(1, int(round(n_ep * w.const_goal_frac)))
        const_eps = np.sort(g.choice(n_ep, size=n_const, replace=False))
        for e in const_eps:
            lo = 0 if e == 0 else int(episode_ends[e - 1])
            hi = int(episode_ends[e])
            next_states[lo:hi, :w.G] = next_states[lo, :w.G]
    return dict(states=states, next_states=next_states, actions=actions, rewards=rewards,
                dones=dones, episode_ends=episode_ends, buffer_size=C, capacity=C,
                const_episodes=const_eps)


def her_sources(w, buf, seed=DEFAULT_SEED + 1):
    """HER source indices ~ U[0, C); a share from constant-goal episodes."""
    g = rng(seed)
    n = w.n_her
    src = g.integers(0, w.C, size=n, dtype=np.int64)
    ce = buf["const_episodes"]
    if w.const_goal_frac > 0.0 and len(ce) > 0:
        k = int(round(n * w.const_goal_frac))
        pick = g.choice(n, size=k, replace=False)
        ends = buf["episode_ends"].astype(np.int64)
        e = ce[g.integers(0, len(ce), size=k)]
        lo = np.where(e > 0, ends[np.maximum(e - 1, 0)], 0)
        src[pick] = lo + g.integers(0, w.L, size=k) % (ends[e] - lo)
    return src.astype(np.int32)


def batch_states(w, seed=DEFAULT_SEED + 2, ld=None):
    """Normal (non-HER) rows of the merged batch, N(0,1), in the compute dtype's
    value set.  Returns float32 [B - n_her, S] (bf16-representable when bf16)."""
    g = rng(seed)
    x = g.standard_normal((w.B - w.n_her, w.S), dtype=np.float32)
    if w.dtype == "bf16":
        x = _bf16_values(x)
    return x


def q_values(w, buf, src, seed=DEFAULT_SEED + 3):
    """Q[B, A] (Gaussian, optional +-outliers), batch actions and q_taken.

    Actions of HER rows are those of their source transitions, so
    q_taken[b] = Q[b, action_b] matches the relabelled batch."""
    g = rng(seed)
    Q = (g.standard_normal((w.B, w.A)) * w.q_sd).astype(np.float32)
    if w.q_outlier_frac > 0.0:
        mask = g.random((w.B, w.A)) < w.q_outlier_frac
        sign = np.where(g.random((w.B, w.A)) < 0.5, -1.0, 1.0)
        Q = np.where(mask, (sign * w.q_outlier_mag).astype(np.float32), Q)
    a_norm = g.integers(0, w.A, size=w.B - w.n_her, dtype=np.int32)
    a_her = buf["actions"][np.asarray(src, dtype=np.int64)]
    acts = np.concatenate([a_norm, a_her]).astype(np.int32)
    q_taken = Q[np.arange(w.B), acts].astype(np.float32)
    return Q, acts, q_taken


def kaiming_uniform(w, seed=DEFAULT_SEED + 10):
    """He-uniform float32 weights U(+-sqrt(6/fan_in)), zero biases, flat in the
    order w1, b1, w2, b2, w3, b3."""
    g = rng(seed)
    S, H1, H2 = w.S, w.H, w.hidden2
    parts = [
        g.uniform(-1, 1, size=H1 * S) * np.sqrt(6.0 / S),
        np.zeros(H1),
        g.uniform(-1, 1, size=H2 * H1) * np.sqrt(6.0 / H1),
        np.zeros(H2),
        g.uniform(-1, 1, size=H2) * np.sqrt(6.0 / H2),
        np.zeros(1),
    ]
    return np.concatenate(parts).astype(np.float32)


def group_inits(w, seed=DEFAULT_SEED + 10):
    return [kaiming_uniform(w, seed + gi) for gi in range(w.groups)]


def budget_sources(w, seed=DEFAULT_SEED + 20, n=None):
    """Four gradient sources ~ N(0,1) scaled x {1, 5, 0.5, 0.2}."""
    g = rng(seed)
    n = w.n_budget if n is None else n
    return [(g.standard_normal(n) * s).astype(np.float32) for s in w.budget_scales]


def budget_params(w, seed=DEFAULT_SEED + 30, n=None):
    g = rng(seed)
    n = w.n_budget if n is None else n
    return (g.standard_normal(n) * 0.05).astype(np.float32)
