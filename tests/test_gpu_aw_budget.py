"""GPU parity of iql_aw_policy and grad_budget_accumulate against the oracle."""
import numpy as np
import pytest

import synth
from oracle import aw, budget, iql
from tests.gpu_util import adam_update_close, assert_rel, dev, host, sync, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


def _aw(m, Q, V, beta):
    import torch
    G, B = V.shape
    A = Q.shape[1]
    pi = torch.empty((G, B, A), dtype=torch.float32, device=dev())
    m.iql_aw_policy(to_dev(Q), to_dev(V), G, B, A, beta, pi)
    sync()
    return host(pi)


def _check_pi(got, Q, V, beta, rtol=1e-5, atol=1e-7):
    for g in range(V.shape[0]):
        ref = aw.aw_policy(Q, V[g], beta)
        d = np.abs(got[g] - ref)
        assert np.all(d <= rtol * np.abs(ref) + atol), f"group {g}: max err {d.max():.3e}"
        np.testing.assert_allclose(got[g].sum(1), 1.0, rtol=1e-5)


@pytest.mark.parametrize("B,A,G", [(256, 4, 1), (1000, 9, 2), (257, 16, 2), (513, 64, 1), (1, 1, 1)])
def test_aw_parity(m, B, A, G):
    g = np.random.default_rng(B * A)
    Q = (g.standard_normal((B, A)) * 2).astype(np.float32)
    V = g.standard_normal((G, B)).astype(np.float32)
    _check_pi(_aw(m, Q, V, 3.0), Q, V, 3.0)


def test_aw_outliers_beta_ten(m):
    w = synth.WORKLOADS["stress_b65536_s256_h512_bf16"]
    buf = {"actions": np.zeros(w.C, np.int32)}
    src = np.zeros(w.n_her, np.int64)
    Q, _, _ = synth.q_values(w, buf, src)
    V = np.random.default_rng(1).standard_normal((1, w.B)).astype(np.float32)
    got = _aw(m, Q, V, w.beta)
    assert np.all(np.isfinite(got))
    _check_pi(got, Q, V, w.beta, rtol=2e-5, atol=1e-7)


def test_aw_beta_zero_uniform(m):
    g = np.random.default_rng(3)
    Q = (g.standard_normal((300, 9)) * 50).astype(np.float32)
    V = g.standard_normal((2, 300)).astype(np.float32)
    got = _aw(m, Q, V, 0.0)
    np.testing.assert_allclose(got, 1.0 / 9, rtol=1e-6)


def _budget(m, sources, fracs, alphas, mgn, adam_state=None, hp=None, grad_init=None):
    import torch
    n = sources[0].shape[0]
    ts = [to_dev(s) for s in sources]
    grad = torch.zeros(n, dtype=torch.float32, device=dev()) if grad_init is None else grad_init
    norms = torch.zeros(len(sources) + 1, dtype=torch.float32, device=dev())
    ws = torch.zeros(m.grad_budget_workspace_bytes(n, len(sources)) // 4, dtype=torch.float32, device=dev())
    adam = None
    if adam_state is not None:
        p, mm, vv, t = adam_state
        adam = m.make_adam(p, mm, vv, t, lr=hp.lr, beta1=hp.beta1, beta2=hp.beta2, eps=hp.eps,
                           max_grad_norm=hp.max_grad_norm)
    m.grad_budget_accumulate(grad, ts, fracs, alphas, n, mgn, norms, adam, ws)
    sync()
    return grad, host(norms)


@pytest.mark.parametrize("n", [1, 1000, 132612, 3_000_001])
def test_budget_accumulate_parity(m, n):
    w = synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"]
    src = synth.budget_sources(w, n=n)
    alphas = (1.0, 1.0, 0.5, 2.0)
    grad, norms = _budget(m, src, w.budget_fractions, alphas, 1.0)
    ref, rn, rc, _ = budget.accumulate(src, w.budget_fractions, alphas, 1.0)
    assert_rel(host(grad), ref, 1e-5, "grad")
    assert_rel(norms[:4], rn, 1e-5, "source norms")
    assert_rel(norms[4:], [rc], 1e-5, "combined norm")


def test_budget_in_place_primary(m):
    w = synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"]
    src = synth.budget_sources(w, n=5000)
    g0 = to_dev(src[0])
    import torch
    ts = [g0] + [to_dev(s) for s in src[1:]]
    norms = torch.zeros(5, dtype=torch.float32, device=dev())
    ws = torch.zeros(m.grad_budget_workspace_bytes(5000, 4) // 4, dtype=torch.float32, device=dev())
    m.grad_budget_accumulate(g0, ts, w.budget_fractions, (1, 1, 1, 1), 5000, 1.0, norms, None, ws)
    sync()
    ref, _, rc, _ = budget.accumulate(src, w.budget_fractions, (1, 1, 1, 1), 1.0)
    assert_rel(host(g0), ref, 1e-5, "in-place grad")
    assert host(norms)[4] <= 1.0 * (1 + 1e-5)


def test_budget_adam_replay_parity(m):
    import torch
    w = synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"]
    n = w.n_budget
    src = synth.budget_sources(w)
    p0 = synth.budget_params(w)
    hp = iql.AdamHP(lr=w.lr, max_grad_norm=w.max_grad_norm)
    p = to_dev(p0)
    mm = torch.zeros(n, dtype=torch.float32, device=dev())
    vv = torch.zeros(n, dtype=torch.float32, device=dev())
    t = torch.zeros(1, dtype=torch.int32, device=dev())
    st = iql.AdamState.fresh(p0)
    grad = torch.zeros(n, dtype=torch.float32, device=dev())
    checkpoints = {1, 10, 100}
    for k in range(1, 101):
        g_gpu, norms = _budget(m, src, w.budget_fractions, (1, 1, 1, 1), w.max_grad_norm, (p, mm, vv, t), hp, grad)
        ref, _, rc, _ = budget.accumulate(src, w.budget_fractions, (1, 1, 1, 1), w.max_grad_norm)
        iql.adam_step(st, ref, hp)
        if k in checkpoints:
            assert int(t.item()) == k
            assert np.all(host(grad) == 0.0)  # Adam consumes the gradient
            assert_rel(norms[4:], [rc], 1e-5, "combined norm")
            assert_rel(host(mm), st.m, 1e-4, f"m at step {k}")
            assert_rel(host(vv), st.v, 1e-4, f"v at step {k}")
            adam_update_close(host(p), st.params, p0, hp.lr, k, 1e-4, f"params at step {k}")


def test_budget_nonfinite_source_skips_adam(m):
    import torch
    n = 4096
    g = np.random.default_rng(0)
    src = [g.standard_normal(n).astype(np.float32) for _ in range(4)]
    src[2][17] = np.nan
    p0 = g.standard_normal(n).astype(np.float32)
    p = to_dev(p0)
    mm = torch.zeros(n, dtype=torch.float32, device=dev())
    vv = torch.zeros(n, dtype=torch.float32, device=dev())
    t = torch.zeros(1, dtype=torch.int32, device=dev())
    flags = torch.zeros(1, dtype=torch.int32, device=dev())
    ts = [to_dev(s) for s in src]
    grad = torch.zeros(n, dtype=torch.float32, device=dev())
    ws = torch.zeros(m.grad_budget_workspace_bytes(n, 4) // 4, dtype=torch.float32, device=dev())
    adam = m.make_adam(p, mm, vv, t, d_flags=flags)
    m.grad_budget_accumulate(grad, ts, (0.7, 0.15, 0.1, 0.05), (1, 1, 1, 1), n, 1.0, None, adam, ws)
    sync()
    assert np.array_equal(host(p), p0)
    assert int(flags.item()) & m.FLAG_NONFINITE_GRAD
    assert int(t.item()) == 1
    assert np.all(host(grad) == 0.0)
