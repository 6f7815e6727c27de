"""GPU parity of iql_aux_step, the whole step in four launches.

The whole-step call must give, bit for bit, what her_relabel +
iql_train_step_aw + grad_budget_accumulate give when called one after the
other (the same block functions run in both), on every output and on the
state it leaves behind, over several steps; and one step of it must match
the oracle directly.  Optional parts (no HER, no policy, no budget, budget
without Adam) are covered the same way.
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import adam_update_close, assert_rel, assert_scalar_rel, dev, host, sync, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


class Inputs:
    """Read-only inputs shared by the two rigs."""

    def __init__(self, w, B, n_budget, bad_sources=False):
        import torch
        self.w, self.B = w, B
        self.n = int(B * w.her_ratio)
        self.buf = buf = synth.replay_buffer(w)
        self.src = synth.her_sources(synth.shrink(w, B=B), buf)
        assert len(self.src) == self.n
        self.Xn = synth.batch_states(synth.shrink(w, B=B))
        self.Q, _, self.q = synth.q_values(synth.shrink(w, B=B), buf, self.src)
        if bad_sources:  # indices outside the buffer: flagged, zero rows
            self.src = self.src.copy()
            self.src[::97] = -1
            self.src[5::101] = w.C + 3
        self.inits = synth.group_inits(w)
        self.sources = synth.budget_sources(w, n=n_budget)
        self.theta = synth.budget_params(w, n=n_budget)
        self.n_budget = n_budget
        self.bf16 = w.dtype == "bf16"
        self.sdt = torch.bfloat16 if self.bf16 else torch.float32
        self.t_states, self.t_next = to_dev(buf["states"]), to_dev(buf["next_states"])
        self.t_actions, self.t_dones = to_dev(buf["actions"]), to_dev(buf["dones"])
        self.t_ends = to_dev(buf["episode_ends"].astype(np.int32))
        self.t_src = to_dev(self.src.astype(np.int32))
        self.t_Q, self.t_q = to_dev(self.Q), to_dev(self.q)
        self.t_sources = [to_dev(s) for s in self.sources]


class Rig:
    """Outputs and trainer state of one way of running the step."""

    def __init__(self, m, inp, her=True, policy=True, budget=True, adam=True, norms=True, strategy=None,
                 minimal_out=False, alias=True):
        import torch
        w, B, n, d = inp.w, inp.B, inp.n, dev()
        self.m, self.inp = m, inp
        self.use_her, self.use_pi, self.use_budget = her, policy, budget
        S = w.S
        self.X = torch.zeros((B, S), dtype=inp.sdt, device=d)
        self.X[: B - n] = to_dev(inp.Xn, inp.sdt)
        if not her or not alias:  # rows the relabelling does not write: fixed values
            self.X[B - n:] = to_dev(inp.buf["states"][np.clip(inp.src, 0, w.C - 1)], inp.sdt)
        # relabelled rows outside the batch when not aliased
        self.Xh = torch.zeros((n, S), dtype=inp.sdt, device=d)
        cfg = m.make_config(S, w.H, B, num_groups=w.groups, compute_dtype=m.BF16 if inp.bf16 else m.F32,
                            states_ld=S, tau=w.taus, lr=w.lr, max_grad_norm=w.max_grad_norm, hidden2=w.H2)
        self.tr = m.IqlTrainer(cfg, np.concatenate(inp.inits))
        self.out_v = torch.zeros((w.groups, B), dtype=torch.float32, device=d)
        self.out_loss = torch.zeros(w.groups, dtype=torch.float32, device=d)
        self.out_gn = torch.zeros(w.groups, dtype=torch.float32, device=d)
        self.pi = torch.zeros((w.groups, B, w.A), dtype=torch.float32, device=d)
        self.rew = torch.zeros(n, dtype=torch.float32, device=d)
        self.nxt = torch.zeros((n, S), dtype=torch.float32, device=d)
        self.act = torch.zeros(n, dtype=torch.int32, device=d)
        self.done = torch.zeros(n, dtype=torch.float32, device=d)
        self.donor = torch.zeros(n, dtype=torch.int32, device=d)
        # the merged batch's importance-sampling weights: the caller's for the
        # normal rows (0.5 here), the relabelling's for the HER tail
        self.isw = torch.full((B,), 0.5, dtype=torch.float32, device=d)
        self.hcfg = m.her_config(S, w.G, m.HER_FUTURE if strategy is None else strategy)
        self.hbuf = m.her_buffer(inp.t_states, inp.t_next, inp.t_actions, inp.t_dones, inp.t_ends)
        tail = (self.X.data_ptr() + (B - n) * S * self.X.element_size()) if alias else self.Xh.data_ptr()
        if minimal_out:
            self.hout = m.her_out(tail, m.BF16 if inp.bf16 else m.F32, S, self.rew, d_flags=self.tr.flags)
        else:
            self.hout = m.her_out(tail, m.BF16 if inp.bf16 else m.F32, S, self.rew, next_states=self.nxt,
                                  actions=self.act, dones=self.done, donor_idx=self.donor, d_flags=self.tr.flags,
                                  is_weights=self.isw.data_ptr() + (B - n) * self.isw.element_size())
        P = inp.n_budget
        self.theta = to_dev(inp.theta)
        self.tm = torch.zeros(P, dtype=torch.float32, device=d)
        self.tv = torch.zeros(P, dtype=torch.float32, device=d)
        self.tt = torch.zeros(1, dtype=torch.int32, device=d)
        self.grad = torch.zeros(P, dtype=torch.float32, device=d)
        self.norms = torch.zeros(len(inp.sources) + 1, dtype=torch.float32, device=d) if norms else None
        self.ws = torch.zeros(m.grad_budget_workspace_bytes(P, len(inp.sources)) // 4, dtype=torch.float32,
                              device=d)
        self.adam = m.make_adam(self.theta, self.tm, self.tv, self.tt, lr=w.lr, max_grad_norm=w.max_grad_norm,
                                d_flags=self.tr.flags) if adam else None
        self.seed = 20261202

    def separate(self):
        m, inp, w = self.m, self.inp, self.inp.w
        if self.use_her:
            m.her_relabel(self.hcfg, self.hbuf, inp.t_src, inp.n, self.seed, self.tr.step_counter, self.hout)
        if self.use_pi:
            self.tr.train_step_aw(self.X, inp.t_q, inp.B, inp.t_Q, w.A, w.beta, self.pi, self.out_v,
                                  self.out_loss, self.out_gn)
        else:
            self.tr.train_step(self.X, inp.t_q, inp.B, self.out_v, self.out_loss, self.out_gn)
        if self.use_budget:
            m.grad_budget_accumulate(self.grad, inp.t_sources, w.budget_fractions, (1.0, 1.0, 1.0, 1.0),
                                     inp.n_budget, w.max_grad_norm, self.norms, self.adam, self.ws)

    def whole(self):
        m, inp, w = self.m, self.inp, self.inp.w
        her = m.her_step(self.hcfg, self.hbuf, inp.t_src, inp.n, self.seed, self.hout) if self.use_her else None
        bud = (m.budget_step(self.grad, inp.t_sources, w.budget_fractions, (1.0, 1.0, 1.0, 1.0), inp.n_budget,
                             w.max_grad_norm, self.norms, self.adam, self.ws) if self.use_budget else None)
        if self.use_pi:
            self.tr.aux_step(her, self.X, inp.t_q, inp.B, inp.t_Q, w.A, w.beta, self.pi, self.out_v,
                             self.out_loss, self.out_gn, bud)
        else:
            self.tr.aux_step(her, self.X, inp.t_q, inp.B, out_v=self.out_v, out_loss=self.out_loss,
                             out_grad_norm=self.out_gn, budget=bud)

    def tensors(self):
        import torch
        out = {"X": self.X, "Xh": self.Xh, "rew": self.rew, "next": self.nxt, "act": self.act, "done": self.done,
               "donor": self.donor, "v": self.out_v, "loss": self.out_loss, "gn": self.out_gn, "pi": self.pi,
               "theta": self.theta, "theta_m": self.tm, "theta_v": self.tv, "theta_t": self.tt,
               "grad": self.grad, "isw": self.isw}
        if self.norms is not None:
            out["norms"] = self.norms
        P = self.tr.n_params
        for g in range(self.inp.w.groups):
            p = torch.zeros(P, dtype=torch.float32, device=dev())
            mm, vv = torch.zeros_like(p), torch.zeros_like(p)
            t = torch.zeros(1, dtype=torch.int32, device=dev())
            self.tr.get_state(g, p, mm, vv, t)
            out.update({f"params{g}": p, f"m{g}": mm, f"v{g}": vv, f"t{g}": t})
        return out


def _bitwise_equal(a, b, what):
    import torch
    ta, tb = a.tensors(), b.tensors()
    sync()
    for k in ta:
        x, y = ta[k], tb[k]
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        elif x.dtype == torch.float32:
            x, y = x.view(torch.int32), y.view(torch.int32)
        assert torch.equal(x, y), f"{what}: {k} differs"


def _run_pair(m, inp, steps=3, expect_flags=0, **kw):
    a, b = Rig(m, inp, **kw), Rig(m, inp, **kw)
    for s in range(steps):
        a.separate()
        b.whole()
        _bitwise_equal(a, b, f"step {s + 1} {kw}")
    for r in (a, b):
        rc, flags = r.tr.status()
        assert flags == expect_flags and (rc == m.OK) == (expect_flags == 0)
        r.tr.close()
    return a, b


@pytest.fixture(scope="module")
def bench_inputs():
    w = synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"]
    return Inputs(w, w.B, w.n_budget)


def test_whole_step_equals_separate_calls_b16384(m, bench_inputs):
    """The production shape (batch 16384, two bf16 groups, policy fused,
    budget over 132612 parameters), three steps: the step counter drives the
    relabelling draws, Adam's t and the budget's t advance."""
    _run_pair(m, bench_inputs, steps=3)


@pytest.mark.parametrize("kw", [dict(her=False), dict(policy=False), dict(budget=False),
                                dict(adam=False), dict(adam=False, norms=False),
                                dict(her=False, policy=False, budget=False)])
def test_whole_step_optional_parts(m, kw):
    w = synth.shrink(synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"], C=1 << 14)
    _run_pair(m, Inputs(w, 3000, 70001), steps=2, **kw)


@pytest.mark.parametrize("strategy", ["final", "future", "random"])
def test_whole_step_relabelling_strategies(m, strategy):
    """Every donor strategy inside the whole step, the HER rows starting
    inside a 128-row tile of the forward/backward launch, two groups."""
    w = synth.shrink(synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"], C=1 << 15)
    code = {"final": m.HER_FINAL, "future": m.HER_FUTURE, "random": m.HER_RANDOM}[strategy]
    _run_pair(m, Inputs(w, 4000, 3001), steps=2, strategy=code)


@pytest.mark.parametrize("S,G,minimal", [(61, 20, False), (100, 8, True), (64, 3, False)])
def test_whole_step_relabelling_ragged_rows(m, S, G, minimal):
    """State widths that are not a multiple of the operand tile (scalar
    loads, padded features), goals longer than 16 entries, and HER without
    its optional outputs."""
    w = synth.shrink(synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"], S=S, G=G, C=1 << 14)
    _run_pair(m, Inputs(w, 1111, 2048), steps=2, minimal_out=minimal)


def test_whole_step_relabelling_bad_sources(m):
    """Source indices outside the buffer: zero rows, reward 0, donor -1 and
    the bad-index flag, the same in both ways of running the step."""
    w = synth.shrink(synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"], C=1 << 14)
    a, _ = _run_pair(m, Inputs(w, 2048, 1000, bad_sources=True), steps=1, expect_flags=m.FLAG_BAD_INDEX)
    assert np.all(host(a.donor)[::97] == -1) and np.all(host(a.rew)[5::101] == 0.0)


def test_whole_step_relabelled_rows_outside_the_batch(m):
    """HER output rows that are not the tail of the batch: the batch keeps
    its rows and the relabelled rows land where the caller asked."""
    w = synth.shrink(synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"], C=1 << 14)
    a, _ = _run_pair(m, Inputs(w, 2048, 1000), steps=2, alias=False)
    assert np.any(host(a.Xh) != 0)


@pytest.mark.parametrize("B", [3000, 2048])
def test_whole_step_relabelling_matches_oracle(m, B):
    """One whole step with bf16 operands against the oracle's HER pass
    (donors, rewards, the bf16 rows in the batch, s' with the new goal,
    actions, dones), and V against the oracle's step on that batch; at
    batch 2048 the HER rows start at a tile boundary and are relabelled by
    the forward/backward launch."""
    from oracle import her, iql
    w = synth.shrink(synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"], C=1 << 14)
    inp = Inputs(w, B, 1000)
    r = Rig(m, inp)
    r.whole()
    sync()
    ref = her.her_step(inp.buf, inp.src, w.G, her.FUTURE, r.seed, 0, out_bf16=True)
    assert np.array_equal(host(r.donor), ref["donor_idx"])
    assert np.array_equal(host(r.rew), ref["rewards"])
    assert np.array_equal(host(r.X)[inp.B - inp.n:], ref["states"])
    assert np.array_equal(host(r.nxt), ref["next_states"])
    assert np.array_equal(host(r.act), ref["actions"]) and np.array_equal(host(r.done), ref["dones"])
    assert np.array_equal(host(r.isw), her.merged_is_weights(np.full(inp.B - inp.n, 0.5, np.float32), inp.n))
    X = host(r.X).astype(np.float64)
    for g in range(w.groups):
        st = iql.AdamState.fresh(inp.inits[g])
        res = iql.train_step(st, X, inp.q, w.S, w.H, w.H, w.taus[g], iql.AdamHP(lr=w.lr))
        assert_rel(host(r.out_v[g]), res.v, 2e-2, f"V g{g}")
    r.tr.close()


@pytest.mark.parametrize("A", [9, 20])
def test_whole_step_fp32_policy(m, A):
    """fp32 operands: the policy fused into the forward/backward launch
    (A <= 16) or run as its own kernel after it (A = 20); ragged batch and
    budget lengths."""
    w = synth.shrink(synth.WORKLOADS["b4096_s42_h128_f32"], A=A, budget=True)
    _run_pair(m, Inputs(w, 1001, 5003), steps=2)


@pytest.mark.parametrize("H,H2", [(256, 0), (128, 96)])
def test_whole_step_layered_shape(m, H, H2):
    """Shapes beyond the fused tile kernel (hidden 256; two hidden widths)
    go through the layered GEMM path inside the whole step."""
    w = synth.shrink(synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"], S=100, H=H, H2=H2, C=1 << 14)
    _run_pair(m, Inputs(w, 2500, 4096), steps=2)


def test_whole_step_matches_oracle(m):
    """One whole step on the small fp32 workload against the oracle: HER
    rows exact, V / loss / parameters within 1e-4, policy within 1e-5, the
    budgeted gradient's clip bound and the budget parameters' Adam update."""
    from oracle import aw, budget, her, iql
    w = synth.shrink(synth.WORKLOADS["tiny_b256_s16_h32"], budget=True)
    inp = Inputs(w, w.B, 4099)
    r = Rig(m, inp, adam=True)
    r.whole()
    sync()
    ref_h = her.her_step(inp.buf, inp.src, w.G, her.FUTURE, r.seed, 0)
    assert np.array_equal(host(r.donor), ref_h["donor_idx"])
    assert np.array_equal(host(r.rew), ref_h["rewards"])
    assert np.array_equal(host(r.X)[w.B - inp.n:], ref_h["states"])
    X = host(r.X).astype(np.float64)
    hp = iql.AdamHP(lr=w.lr, max_grad_norm=w.max_grad_norm)
    st = iql.AdamState.fresh(inp.inits[0])
    ref = iql.train_step(st, X, inp.q, w.S, w.H, w.H, w.taus[0], hp)
    assert_rel(host(r.out_v[0]), ref.v, 1e-4, "V")
    assert_scalar_rel(host(r.out_loss)[0], ref.loss, 1e-4, "loss")
    assert_scalar_rel(host(r.out_gn)[0], ref.grad_norm, 1e-4, "grad norm")
    p = r.tensors()["params0"]
    sync()
    adam_update_close(host(p), st.params, None, w.lr, 1, 1e-4, "params")
    ref_pi = aw.aw_policy(inp.Q, host(r.out_v[0]), w.beta)
    assert np.max(np.abs(host(r.pi[0]) - ref_pi)) <= 1e-5
    g_ref, n_ref, comb_ref, _ = budget.accumulate(inp.sources, w.budget_fractions, (1, 1, 1, 1), w.max_grad_norm)
    got_norms = host(r.norms)
    assert_rel(got_norms[:4], n_ref, 1e-5, "source norms")
    assert_scalar_rel(got_norms[4], comb_ref, 1e-5, "combined norm")
    th = iql.AdamState.fresh(inp.theta)
    iql.adam_step(th, g_ref, hp)
    adam_update_close(host(r.theta), th.params, None, w.lr, 1, 1e-5, "budget params")
    assert int(host(r.tt)[0]) == 1
    assert np.all(host(r.grad) == 0)  # consumed by Adam
    r.tr.close()


@pytest.mark.parametrize("B,n_budget,first_launch", [(2048, 5000, False), (3000, 5000, True), (1024, 300000, True)])
def test_time_aux_step_reports_every_launch(m, B, n_budget, first_launch):
    """The measurement entry point runs real steps (Adam's t advances) and
    reports a positive kernel time for every launch it makes, and 0 for the
    first when the forward/backward launch hosts both of its passes (HER
    rows at a 128-row boundary of the batch tail, budget norms small enough
    to ride along)."""
    w = synth.shrink(synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"], C=1 << 14)
    inp = Inputs(w, B, n_budget)
    r = Rig(m, inp)
    her = m.her_step(r.hcfg, r.hbuf, inp.t_src, inp.n, r.seed, r.hout)
    bud = m.budget_step(r.grad, inp.t_sources, w.budget_fractions, (1.0, 1.0, 1.0, 1.0), inp.n_budget,
                        w.max_grad_norm, r.norms, r.adam, r.ws)
    us = r.tr.time_aux_step(her, r.X, inp.t_q, inp.B, inp.t_Q, w.A, w.beta, r.pi, r.out_v, r.out_loss, r.out_gn,
                            bud, reps=5)
    assert len(us) == 4 and all(np.isfinite(us)) and min(us[1:]) > 0.0, us
    assert (us[0] > 0.0) if first_launch else (us[0] == 0.0), us
    t = r.tensors()
    sync()
    assert int(host(t["t0"])[0]) == 5 and int(host(r.tt)[0]) == 5
    rc, flags = r.tr.status()
    assert rc == m.OK and flags == 0
    r.tr.close()


@pytest.mark.parametrize("B,n,S,G,strategy,minimal,n_budget", [
    (2048, 1024, 128, 8, "future", False, 3001),
    (2000, 976, 128, 8, "final", False, 3001),     # last tile of 80 rows
    (1536, 1024, 128, 8, "random", True, 3001),    # HER rows from row 512, no optional outputs
    (1280, 768, 104, 20, "future", False, 2048),   # state of 13 chunks (SP 128), goal past 16 entries
    (1280, 768, 100, 20, "future", False, 2048),   # state not a multiple of 8: relabelled by its own launch
    (1280, 640, 56, 56, "final", False, 2048),     # 64-wide operand tile, goal = whole state
    (1408, 640, 96, 64, "future", True, 2048),     # goal of 64 entries, all staged in LDS
    (1408, 640, 96, 70, "future", False, 2048),    # longer goal: relabelled by its own launch
    (1024, 512, 128, 8, "future", False, 300000),  # budget norms too many to ride along
])
def test_whole_step_relabelling_inside_forward_backward(m, B, n, S, G, strategy, minimal, n_budget):
    """HER rows that form the batch tail from a 128-row boundary on are
    relabelled by the forward/backward launch itself (group 0 writes the HER
    outputs, every group builds its tile from the replay buffer), and the
    budget's pass 1 rides on the workgroups without HER rows: bit for bit
    what the separate calls give, over two steps."""
    w = synth.shrink(synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"], S=S, G=G, C=1 << 14, her_ratio=n / B)
    inp = Inputs(w, B, n_budget)
    assert inp.n == n
    code = {"final": m.HER_FINAL, "future": m.HER_FUTURE, "random": m.HER_RANDOM}[strategy]
    _run_pair(m, inp, steps=2, strategy=code, minimal_out=minimal)


@pytest.mark.parametrize("wname,B,n,G,strategy,minimal,budget", [
    ("b4096_s42_h128_f32", 4096, 1024, 8, "final", False, False),   # the workload's own shape
    ("b4096_s42_h128_f32", 1000, 488, 8, "future", False, True),    # last tile of 8 rows; budget norms in A
    ("b4096_s42_h128_f32", 2048, 1024, 20, "random", True, False),  # goal past 16 entries, no optional outputs
    ("b4096_s42_h128_f32", 2000, 1000, 8, "future", False, False),  # HER rows from row 1000
    ("tiny_b256_s16_h32", 256, 128, 4, "future", False, False),     # hidden 32, one wave per tile
    ("tiny_b256_s16_h32", 200, 104, 16, "final", False, False),     # goal = whole state, ragged last tile
])
def test_whole_step_relabelling_fp32(m, wname, B, n, G, strategy, minimal, budget):
    """fp32 trainers (the four-wave hidden-128 kernel and the hidden-32 one):
    the step's first launch relabels the HER rows into the batch tail (rows of
    any width and alignment), and the whole step equals the separate calls
    bit for bit over two steps, for every strategy, ragged last tiles, goals
    past 16 entries and with or without the budget's norms in that launch."""
    w = synth.shrink(synth.WORKLOADS[wname], G=G, her_ratio=n / B)
    inp = Inputs(w, B, 4099)
    assert inp.n == n
    code = {"final": m.HER_FINAL, "future": m.HER_FUTURE, "random": m.HER_RANDOM}[strategy]
    _run_pair(m, inp, steps=2, strategy=code, minimal_out=minimal, budget=budget)


@pytest.mark.parametrize("name,batch,rows", [("b16384_s128_h128_bf16_g2_budget", 16384, 128),
                                             ("b16384_s128_h128_bf16_g2_budget", 1000, 8),
                                             ("stress_b65536_s256_h512_bf16", 65536, 40),
                                             ("stress_b65536_s256_h512_bf16", 1000, 8)])
def test_partial_layout_query(m, name, batch, rows):
    """The partial-buffer query the byte counts of bench.py rest on: one row
    per 128-sample workgroup on the fused path; on the wide-hidden path one
    per sample chunk (at most 42 chunks for six 256 x 256 weight-gradient
    tiles, each a multiple of 128 samples: 1664 at batch 65536, 128 at 1000);
    each row the parameter count rounded up to 128 floats."""
    w = synth.WORKLOADS[name]
    cfg = m.make_config(w.S, w.H, batch, num_groups=w.groups, compute_dtype=m.BF16, states_ld=w.S, tau=w.taus)
    tr = m.IqlTrainer(cfg, np.concatenate(synth.group_inits(w)))
    n, floats = tr.partial_layout(batch)
    assert n == rows and floats == (w.n_params + 127) // 128 * 128
    with pytest.raises(m.IqlhError):
        tr.partial_layout(batch + 1)
    tr.close()
