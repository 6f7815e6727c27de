"""Pins of the oracle's value network, expectile loss and clipped Adam.

Independent checks: closed forms of the expectile loss, PyTorch CPU fp64
autograd of the same network (library special case), central finite
differences, ``torch.optim.Adam`` / ``AdamW`` in fp64, the t = 1 closed form
of Adam, and the clip arithmetic of the pages' worked example.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import iql

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "iql_hand.json")))


def _net(S, H, seed, H2=None):
    H2 = H if H2 is None else H2
    g = np.random.default_rng(seed)
    flat = np.concatenate([g.uniform(-1, 1, S * H) * np.sqrt(6 / S), g.standard_normal(H) * 0.1,
                           g.uniform(-1, 1, H2 * H) * np.sqrt(6 / H), g.standard_normal(H2) * 0.1,
                           g.uniform(-1, 1, H2) * np.sqrt(6 / H2), g.standard_normal(1) * 0.1])
    return flat


# ---------------------------------------------------------------- expectile
def test_expectile_tau_half_is_half_mse():
    g = np.random.default_rng(0)
    q, v = g.standard_normal(1000), g.standard_normal(1000)
    loss, dv = iql.expectile(q, v, 0.5)
    assert loss == pytest.approx(0.5 * np.mean((q - v) ** 2), rel=1e-14)
    np.testing.assert_allclose(dv, -(q - v) / 1000, rtol=1e-14)


def test_expectile_tau_one_keeps_only_underestimation():
    g = np.random.default_rng(1)
    q, v = g.standard_normal(500), g.standard_normal(500)
    d = q - v
    loss, _ = iql.expectile(q, v, 1.0)
    assert loss == pytest.approx(np.mean(d * d * (d >= 0)), rel=1e-14)


def test_expectile_hand_worked():
    c = GOLD["expectile"]
    loss, dv = iql.expectile(np.array(c["q"]), np.array(c["v"]), c["tau"])
    assert loss == pytest.approx(c["loss"], rel=1e-14)
    np.testing.assert_allclose(dv, c["dv"], rtol=1e-14)


def test_expectile_zero_diff_has_zero_gradient():
    loss, dv = iql.expectile(np.array([1.5]), np.array([1.5]), 0.7)
    assert loss == 0.0 and dv[0] == 0.0


# ------------------------------------------------------- network + autograd
def _torch_loss(flat, X, q, tau, S, H, H2=None):
    H2 = H if H2 is None else H2
    t = torch.tensor(flat, dtype=torch.float64, requires_grad=True)
    o = 0
    w1 = t[o:o + H * S].view(H, S); o += H * S
    b1 = t[o:o + H]; o += H
    w2 = t[o:o + H2 * H].view(H2, H); o += H2 * H
    b2 = t[o:o + H2]; o += H2
    w3 = t[o:o + H2]; o += H2
    b3 = t[o]
    Xt = torch.tensor(X, dtype=torch.float64)
    h1 = torch.relu(torch.nn.functional.linear(Xt, w1, b1))
    h2 = torch.relu(torch.nn.functional.linear(h1, w2, b2))
    v = h2 @ w3 + b3
    d = torch.tensor(q, dtype=torch.float64) - v
    w = torch.where(d >= 0, torch.tensor(tau, dtype=torch.float64), torch.tensor(1 - tau, dtype=torch.float64))
    loss = torch.mean(w * d * d)
    loss.backward()
    return loss.item(), v.detach().numpy(), t.grad.numpy()


@pytest.mark.parametrize("S,H,H2,B,tau", [(5, 4, 4, 8, 0.7), (16, 32, 32, 64, 0.7), (42, 16, 16, 33, 0.9),
                                           (7, 8, 8, 1, 0.3), (6, 9, 4, 17, 0.7), (5, 3, 11, 12, 0.2)])
def test_forward_backward_match_torch_autograd(S, H, H2, B, tau):
    """The network with two hidden widths (W2 [H2, H1]) included: a
    transposed W2 or a swapped width fails the second pair of shapes."""
    flat = _net(S, H, seed=S * 100 + H, H2=H2)
    g = np.random.default_rng(B)
    X, q = g.standard_normal((B, S)), g.standard_normal(B) * 2
    p = iql.unflatten(flat, S, H, H2)
    v, cache = iql.forward(p, X)
    loss, dv = iql.expectile(q, v, tau)
    grad = iql.flatten(iql.backward(p, cache, dv))
    tl, tv, tg = _torch_loss(flat, X, q, tau, S, H, H2)
    assert loss == pytest.approx(tl, rel=1e-12)
    np.testing.assert_allclose(v, tv, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(grad, tg, rtol=1e-10, atol=1e-14)


def _torch_rounded(flat, X, q, tau, S, H):
    """The same network with bf16 operand storage modelled in torch autograd:
    weights and h1 take their bf16 values in the forward (straight-through,
    fp64 identity in the backward), and hooks round the gradients arriving at
    z2 and z1 (dz2, dz1) before they feed the weight and bias gradients and
    dh1."""
    import torch

    def bf(a):
        return a.to(torch.float32).to(torch.bfloat16).to(torch.float64)

    def st(a):  # bf16 value forward, identity backward (fp64 gradient)
        return a + (bf(a) - a).detach()

    t = torch.tensor(flat, dtype=torch.float64, requires_grad=True)
    o = 0
    w1 = t[o:o + H * S].view(H, S); o += H * S
    b1 = t[o:o + H]; o += H
    w2 = t[o:o + H * H].view(H, H); o += H * H
    b2 = t[o:o + H]; o += H
    w3 = t[o:o + H]; o += H
    b3 = t[o]
    Xt = torch.tensor(X, dtype=torch.float64)
    z1 = Xt @ st(w1).T + b1
    z1.register_hook(lambda g: bf(g))
    z2 = st(torch.relu(z1)) @ st(w2).T + b2
    z2.register_hook(lambda g: bf(g))
    v = torch.relu(z2) @ w3 + b3
    d = torch.tensor(q, dtype=torch.float64) - v
    w = torch.where(d >= 0, torch.tensor(tau, dtype=torch.float64), torch.tensor(1 - tau, dtype=torch.float64))
    loss = torch.mean(w * d * d)
    loss.backward()
    return loss.item(), v.detach().numpy(), t.grad.numpy()


@pytest.mark.parametrize("S,H,B,tau", [(5, 4, 8, 0.7), (16, 32, 64, 0.3), (42, 16, 33, 0.9)])
def test_bf16_operand_variant_matches_torch(S, H, B, tau):
    """Pin of the rounded-operand variant against an independent autograd
    model of the same storage; it also differs from the plain definition, so
    every rounding point is exercised."""
    flat = _net(S, H, seed=S * 100 + H + 1)
    g = np.random.default_rng(B + 7)
    X, q = g.standard_normal((B, S)), g.standard_normal(B) * 2
    p = iql.unflatten(flat, S, H, H)
    v, cache = iql.forward(p, X, iql.bf16_operands)
    loss, dv = iql.expectile(q, v, tau)
    grad = iql.flatten(iql.backward(p, cache, dv, iql.bf16_operands))
    tl, tv, tg = _torch_rounded(flat, X, q, tau, S, H)
    assert loss == pytest.approx(tl, rel=1e-10)
    np.testing.assert_allclose(v, tv, rtol=1e-10, atol=1e-13)
    np.testing.assert_allclose(grad, tg, rtol=1e-9, atol=1e-13)
    plain = iql.flatten(iql.backward(p, iql.forward(p, X)[1], iql.expectile(q, iql.forward(p, X)[0], tau)[1]))
    o = 0
    for name, n in (("w1", S * H), ("b1", H), ("w2", H * H), ("b2", H)):
        assert not np.allclose(grad[o:o + n], plain[o:o + n], rtol=1e-6, atol=0), name
        o += n


def test_gradient_finite_differences():
    S, H, B, tau = 5, 4, 8, 0.7
    g = np.random.default_rng(5)
    # resample until no pre-activation or diff sits near a kink
    for _ in range(100):
        flat = _net(S, H, int(g.integers(1 << 30)))
        X, q = g.standard_normal((B, S)), g.standard_normal(B)
        p = iql.unflatten(flat, S, H, H)
        v, cache = iql.forward(p, X)
        if (np.min(np.abs(cache["z1"])) > 1e-3 and np.min(np.abs(cache["z2"])) > 1e-3
                and np.min(np.abs(q - v)) > 1e-3 and np.mean(cache["z2"] > 0) > 0.3):
            break
    loss, dv = iql.expectile(q, v, tau)
    grad = iql.flatten(iql.backward(p, cache, dv))
    h = 1e-6
    fd = np.zeros_like(flat)
    for i in range(flat.size):
        e = np.zeros_like(flat)
        e[i] = h
        lp, _ = iql.expectile(q, iql.forward(iql.unflatten(flat + e, S, H, H), X)[0], tau)
        lm, _ = iql.expectile(q, iql.forward(iql.unflatten(flat - e, S, H, H), X)[0], tau)
        fd[i] = (lp - lm) / (2 * h)
    np.testing.assert_allclose(grad, fd, rtol=1e-5, atol=1e-9)


def test_param_count_and_layout():
    assert iql.num_params(16, 32, 32) == 1633
    assert iql.num_params(42, 128, 128) == 22145
    assert iql.num_params(128, 128, 128) == 33153
    assert iql.num_params(256, 512, 512) == 394753
    flat = np.arange(iql.num_params(3, 2, 2), dtype=np.float64)
    p = iql.unflatten(flat, 3, 2, 2)
    assert p["w1"][1, 0] == 3 and p["b1"][0] == 6 and p["w2"][0, 1] == 9
    assert p["b2"][1] == 13 and p["w3"][0] == 14 and p["b3"][0] == 16
    np.testing.assert_array_equal(iql.flatten(p), flat)
    # two widths: S H1 + H1 + H2 H1 + H2 + H2 + 1, W2 stored [H2][H1] ([out, in])
    assert iql.num_params(3, 2, 4) == 6 + 2 + 8 + 4 + 4 + 1
    flat = np.arange(iql.num_params(3, 2, 4), dtype=np.float64)
    p = iql.unflatten(flat, 3, 2, 4)
    assert p["w2"].shape == (4, 2) and p["w2"][1, 0] == 10 and p["b2"][0] == 16 and p["w3"][3] == 23
    assert p["b3"][0] == 24
    np.testing.assert_array_equal(iql.flatten(p), flat)


# --------------------------------------------------------------------- Adam
def test_adam_matches_torch_without_clip():
    g = np.random.default_rng(3)
    n = 257
    p0 = g.standard_normal(n)
    hp = iql.AdamHP(lr=3e-4, max_grad_norm=np.inf)
    st = iql.AdamState.fresh(p0)
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([tp], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps)
    for k in range(6):
        grad = g.standard_normal(n) * (10.0 ** (k - 3))
        iql.adam_step(st, grad, hp)
        tp.grad = torch.tensor(grad, dtype=torch.float64)
        opt.step()
    np.testing.assert_allclose(st.params, tp.detach().numpy(), rtol=1e-13, atol=1e-15)
    assert st.t == 6


def test_adamw_weight_decay_matches_torch():
    g = np.random.default_rng(4)
    n = 64
    p0 = g.standard_normal(n)
    hp = iql.AdamHP(lr=1e-3, weight_decay=0.1, max_grad_norm=np.inf)
    st = iql.AdamState.fresh(p0)
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps, weight_decay=0.1)
    for _ in range(4):
        grad = g.standard_normal(n)
        iql.adam_step(st, grad, hp)
        tp.grad = torch.tensor(grad, dtype=torch.float64)
        opt.step()
    np.testing.assert_allclose(st.params, tp.detach().numpy(), rtol=1e-13)


def test_adam_first_step_closed_form():
    g = np.random.default_rng(6)
    grad = g.standard_normal(100) * 1e-3
    p0 = g.standard_normal(100)
    hp = iql.AdamHP(lr=3e-4, max_grad_norm=1e9)
    st = iql.AdamState.fresh(p0)
    iql.adam_step(st, grad, hp)
    np.testing.assert_allclose(st.params - p0, -hp.lr * grad / (np.abs(grad) + hp.eps), rtol=1e-9)


def test_clip_worked_example():
    c = GOLD["clip"]
    # a combined norm of 1.35 x max_grad_norm is scaled by 1/1.35: 26% shrink
    coef = iql.clip_coef(c["norm_over_max"] * c["max_grad_norm"], c["max_grad_norm"])
    assert 1.0 - coef == pytest.approx(c["shrink"], abs=1e-3)
    assert iql.clip_coef(0.5, 1.0) == 1.0
    assert iql.clip_coef(0.0, 0.0) == 1.0
    assert np.isnan(iql.clip_coef(float("nan"), 1.0))


def test_adam_clip_scales_gradient():
    g = np.random.default_rng(7)
    grad = g.standard_normal(50)
    grad *= 3.0 / np.linalg.norm(grad)
    hp = iql.AdamHP(lr=1e-2, max_grad_norm=1.0)
    a = iql.AdamState.fresh(np.zeros(50))
    b = iql.AdamState.fresh(np.zeros(50))
    n, _ = iql.adam_step(a, grad, hp)
    assert n == pytest.approx(3.0, rel=1e-14)
    iql.adam_step(b, grad / 3.0, iql.AdamHP(lr=1e-2, max_grad_norm=np.inf))
    np.testing.assert_allclose(a.m, b.m, rtol=1e-14)
    np.testing.assert_allclose(a.v, b.v, rtol=1e-14)


def test_adam_nonfinite_skips_update():
    hp = iql.AdamHP()
    st = iql.AdamState.fresh(np.ones(10))
    grad = np.ones(10)
    grad[3] = np.nan
    n, skipped = iql.adam_step(st, grad, hp)
    assert np.isnan(n) and skipped.all()
    np.testing.assert_array_equal(st.params, np.ones(10))
    assert st.t == 1 and np.all(st.m == 0)


def test_weight_clamp():
    hp = iql.AdamHP(lr=1.0, max_grad_norm=np.inf, weight_clamp_max_abs=0.5)
    st = iql.AdamState.fresh(np.array([0.45, -0.45, 0.0]))
    iql.adam_step(st, np.array([-1.0, 1.0, 1.0]), hp)
    np.testing.assert_allclose(st.params, [0.5, -0.5, -0.5])


# ---------------------------------------------------------- whole train step
def test_train_step_matches_torch_composition():
    S, H, B, tau = 16, 32, 96, 0.7
    flat = _net(S, H, seed=11)
    g = np.random.default_rng(12)
    hp = iql.AdamHP(lr=1e-3, max_grad_norm=0.05)
    st = iql.AdamState.fresh(flat)
    tp = torch.tensor(flat, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Adam([tp], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps)
    for _ in range(3):
        X, q = g.standard_normal((B, S)), g.standard_normal(B)
        r = iql.train_step(st, X, q, S, H, H, tau, hp)
        tl, tv, tg = _torch_loss(tp.detach().numpy(), X, q, tau, S, H)
        n = np.linalg.norm(tg)
        assert r.grad_norm == pytest.approx(n, rel=1e-12)
        assert r.loss == pytest.approx(tl, rel=1e-12)
        c = hp.max_grad_norm / n if n > hp.max_grad_norm else 1.0
        tp.grad = torch.tensor(tg * c, dtype=torch.float64)
        opt.step()
    np.testing.assert_allclose(st.params, tp.detach().numpy(), rtol=1e-11, atol=1e-14)


# ------------------------------------------------------------ target EMA
def test_target_ema_hand_worked_and_limits():
    """Polyak averaging: weight tau on the online value, 1 - tau on the
    target; tau = 0 keeps the target, tau = 1 copies the online network."""
    t, o = np.array([1.0, -2.0, 0.5]), np.array([3.0, 2.0, 0.5])
    np.testing.assert_array_equal(iql.target_ema(t, o, 0.25), [1.5, -1.0, 0.5])
    np.testing.assert_array_equal(iql.target_ema(t, o, 0.0), t)
    np.testing.assert_array_equal(iql.target_ema(t, o, 1.0), o)


def test_target_ema_geometric_convergence():
    """k updates toward a fixed online vector leave (1 - tau)^k of the
    initial gap: target_k = online + (1 - tau)^k (target_0 - online)."""
    g = np.random.default_rng(3)
    t0, o = g.standard_normal(50), g.standard_normal(50)
    tau, t = 0.05, t0.copy()
    for k in range(1, 41):
        t = iql.target_ema(t, o, tau)
        np.testing.assert_allclose(t, o + (1 - tau) ** k * (t0 - o), rtol=1e-12, atol=1e-14)


# ------------------------------------------------------ bootstrap target
def test_bootstrap_target_hand_worked():
    """r + gamma (1 - done) V(s'): gamma 0 leaves the reward, a terminal row
    leaves the reward, otherwise the discounted value is added."""
    r, d, v = np.array([1.0, -0.01, 0.5]), np.array([0.0, 0.0, 1.0]), np.array([2.0, -4.0, 100.0])
    np.testing.assert_array_equal(iql.bootstrap_target(r, d, v, 0.5), [2.0, -2.01, 0.5])
    np.testing.assert_array_equal(iql.bootstrap_target(r, d, v, 0.0), r)
    np.testing.assert_array_equal(iql.bootstrap_target(r, None, v, 0.5), r + 0.5 * v)
