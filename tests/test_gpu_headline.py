"""The headline workload end to end against the oracle: batch 16384, state
128, two bf16 trainers of hidden 128, 9 actions, HER over half the batch
("future" donors from a replay buffer of 2^20 rows, relabelled inside the
forward/backward launch), the advantage-weighted policy fused into it, and
the budgeted accumulation over 132612 parameters with its Adam update -- one
iql_aux_step call, the step bench.py times.

Bars: HER donors, rewards, relabelled rows (bf16 bit patterns), s', actions,
dones and importance weights bit-exact; V, loss, pre-clip norm, Adam m, v and
the parameters of each trainer within 2e-2 (bf16 operands, fp32 accumulate;
v, a square of the gradient, within twice that); the policy within 1e-5
relative (+1e-7) of the definition evaluated on the step's own V; budget
norms within 1e-5 and the budgeted network's Adam state within 1e-4.

The 1000-step replay (the budget workload's "1000 steps replayed") checks
the trainers teacher-forced at steps 1, 10, 100 and 1000 (each from the
state the GPU itself reached), the relabelling at those steps (the device
step counter advances the donor draws), and the budgeted network's Adam
state free-running against the oracle's own 1000-step replay.  At step 1000
the raw gradient (pre-clip norm, Adam m and v) is compared with the oracle
that stores the same GEMM operands in bf16 as the kernel (pinned against
torch autograd), at 2e-3: near convergence the gradient is a small
difference of large terms and bf16 operand storage alone moves it beyond
2e-2 (tests/test_oracle_conditioning.py); V, the loss, the parameters and
the policy are still held to the plain definition there.
"""
import numpy as np
import pytest

import synth
from oracle import aw, budget, her, iql
from tests.gpu_util import adam_update_close, assert_rel, assert_scalar_rel, host, sync
from tests.test_gpu_step import Inputs, Rig

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


@pytest.fixture(scope="module")
def inp():
    w = synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"]
    return Inputs(w, w.B, w.n_budget)


def _state(r, g):
    t = r.tensors()
    sync()
    return iql.AdamState(host(t[f"params{g}"]).astype(np.float64), host(t[f"m{g}"]).astype(np.float64),
                         host(t[f"v{g}"]).astype(np.float64), int(host(t[f"t{g}"])[0]))


def _check_her(r, inp, step):
    w = inp.w
    ref = her.her_step(inp.buf, inp.src, w.G, her.FUTURE, r.seed, step, out_bf16=True)
    assert np.array_equal(host(r.donor), ref["donor_idx"]), f"donors, step word {step}"
    assert np.array_equal(host(r.rew).view(np.uint32), ref["rewards"].view(np.uint32)), "rewards"
    assert np.array_equal(host(r.X)[inp.B - inp.n:].view(np.uint32), ref["states"].view(np.uint32)), "rows"
    assert np.array_equal(host(r.nxt).view(np.uint32), ref["next_states"].view(np.uint32)), "s'"
    assert np.array_equal(host(r.act), ref["actions"]) and np.array_equal(host(r.done), ref["dones"])
    assert np.array_equal(host(r.isw), her.merged_is_weights(np.full(inp.B - inp.n, 0.5, np.float32), inp.n))


def _check_trainers(r, inp, before, what, rnd=None, rtol=2e-2, grad_checks=True):
    """One step of each trainer from `before` (the state the GPU started the
    step from) on the GPU's merged batch, against what the GPU reported and
    the state it left.  rnd=iql.bf16_operands: the oracle with the kernel's
    bf16 operand storage (W1, W2, h1, dz2, dz1); grad_checks=False leaves out
    the quantities that carry the raw gradient (pre-clip norm, m, v)."""
    w = inp.w
    X = host(r.X).astype(np.float64)
    hp = iql.AdamHP(lr=w.lr, max_grad_norm=w.max_grad_norm)
    for g in range(w.groups):
        st = before[g].copy()
        ref = iql.train_step(st, X, inp.q, w.S, w.H, w.H, w.taus[g], hp, rnd)
        assert_rel(host(r.out_v[g]), ref.v, rtol, f"{what} V g{g}")
        assert_scalar_rel(host(r.out_loss)[g], ref.loss, rtol, f"{what} loss g{g}")
        got = _state(r, g)
        assert got.t == st.t
        adam_update_close(got.params, st.params, None, hp.lr, 1, rtol, f"{what} params g{g}")
        gn = float(host(r.out_gn)[g])
        print(f"  {what} g{g}: grad norm {gn:.6g} vs {ref.grad_norm:.6g} "
              f"(rel {abs(gn - ref.grad_norm) / ref.grad_norm:.2e})", flush=True)
        if grad_checks:
            assert_scalar_rel(gn, ref.grad_norm, rtol, f"{what} grad norm g{g}")
            assert_rel(got.m, st.m, rtol, f"{what} Adam m g{g}")
            assert_rel(got.v, st.v, 2 * rtol, f"{what} Adam v g{g}")
        # the policy of this step, from this step's V
        pi_ref = aw.aw_policy(inp.Q, host(r.out_v[g]), w.beta)
        d = np.abs(host(r.pi[g]) - pi_ref)
        assert np.all(d <= 1e-5 * np.abs(pi_ref) + 1e-7), f"{what} policy g{g}: {d.max():.3e}"


def test_headline_step_matches_oracle(m, inp):
    w = inp.w
    r = Rig(m, inp)
    before = [_state(r, g) for g in range(w.groups)]
    r.whole()
    sync()
    _check_her(r, inp, 0)
    _check_trainers(r, inp, before, "headline step 1")
    g_ref, n_ref, comb_ref, _ = budget.accumulate(inp.sources, w.budget_fractions, (1, 1, 1, 1), w.max_grad_norm)
    got_norms = host(r.norms)
    assert_rel(got_norms[:4], n_ref, 1e-5, "source norms")
    assert_scalar_rel(got_norms[4], comb_ref, 1e-5, "combined norm")
    assert comb_ref <= w.max_grad_norm * (1 + 1e-6)
    th = iql.AdamState.fresh(inp.theta)
    iql.adam_step(th, g_ref, iql.AdamHP(lr=w.lr, max_grad_norm=w.max_grad_norm))
    assert_rel(host(r.tm), th.m, 1e-4, "budget Adam m")
    assert_rel(host(r.tv), th.v, 1e-4, "budget Adam v")
    adam_update_close(host(r.theta), th.params, None, w.lr, 1, 1e-4, "budget params")
    assert np.all(host(r.grad) == 0.0)
    rc, flags = r.tr.status()
    assert rc == m.OK and flags == 0
    r.tr.close()


def test_thousand_step_replay(m, inp):
    w = inp.w
    hp = iql.AdamHP(lr=w.lr, max_grad_norm=w.max_grad_norm)
    r = Rig(m, inp)
    g_ref, _, comb_ref, _ = budget.accumulate(inp.sources, w.budget_fractions, (1, 1, 1, 1), w.max_grad_norm)
    th = iql.AdamState.fresh(inp.theta)
    checkpoints = (1, 10, 100, 1000)
    for k in range(1, 1001):
        forced = k in checkpoints
        if forced:
            before = [_state(r, g) for g in range(w.groups)]
        r.whole()
        iql.adam_step(th, g_ref, hp)  # the budgeted network: same sources every step
        if forced:
            sync()
            print(f"replay step {k}", flush=True)
            _check_her(r, inp, k - 1)
            late = k == 1000
            # near convergence the gradient is a small difference of large
            # terms, and bf16 operand storage alone moves it by more than the
            # bf16 bar (the conditioning test of the oracle shows it): there
            # the raw gradient is held to the oracle with the kernel's operand
            # storage, ten times tighter than the bar, and everything else to
            # the plain definition
            _check_trainers(r, inp, before, f"replay step {k} (teacher-forced)", grad_checks=not late)
            if late:
                _check_trainers(r, inp, before, f"replay step {k} (bf16 operands)", rnd=iql.bf16_operands,
                                rtol=2e-3)
            assert int(host(r.tt)[0]) == k
            assert_scalar_rel(host(r.norms)[4], comb_ref, 1e-5, f"combined norm step {k}")
            assert_rel(host(r.tm), th.m, 1e-4, f"budget Adam m step {k}")
            assert_rel(host(r.tv), th.v, 1e-4, f"budget Adam v step {k}")
            adam_update_close(host(r.theta), th.params, inp.theta, hp.lr, k, 1e-4, f"budget params step {k}")
    rc, flags = r.tr.status()
    assert rc == m.OK and flags == 0
    r.tr.close()
