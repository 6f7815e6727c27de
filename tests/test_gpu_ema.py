"""GPU parity of the Polyak (EMA) target copy of the value network against
the oracle's target_ema: the standalone update, the update folded into the
Adam launch of every step (checked per step from the GPU's own parameters),
and the bit-for-bit equality of the two forms, also through the whole-step
entry point.  fp32 elementwise: 1e-6 relative (one fma rounding per step)."""
import numpy as np
import pytest

import synth
from oracle import iql
from tests.gpu_util import dev, host, sync, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


def _trainer(m, w, B, seed=0):
    import torch
    g = np.random.default_rng(seed)
    X = g.standard_normal((B, w.S)).astype(np.float32)
    if w.dtype == "bf16":
        X = synth._bf16_values(X)
    q = (g.standard_normal(B) * w.q_sd).astype(np.float32)
    cfg = m.make_config(w.S, w.H, B, num_groups=w.groups, compute_dtype=m.BF16 if w.dtype == "bf16" else m.F32,
                        states_ld=w.S, tau=w.taus, lr=w.lr, max_grad_norm=w.max_grad_norm)
    tr = m.IqlTrainer(cfg, np.concatenate(synth.group_inits(w)))
    tX = to_dev(X, torch.bfloat16 if w.dtype == "bf16" else torch.float32)
    return tr, tX, to_dev(q)


def _get(tr, g, which):
    import torch
    P = iql.num_params(tr.cfg.state_dim, tr.cfg.hidden, tr.cfg.hidden)
    p = torch.zeros(P, dtype=torch.float32, device=dev())
    if which == "target":
        tr.get_target(g, p)
    else:
        tr.get_state(g, p, None, None, None)
    sync()
    return host(p).astype(np.float64)


def _close(got, ref, scale, what):
    """fp32 update vs fp64 definition: two roundings of quantities bounded by
    |target| + |params| (the difference and the fused multiply-add)."""
    d = np.abs(got - ref)
    bound = 2.5e-7 * scale + 1e-30
    assert np.all(d <= bound), f"{what}: max err {d.max():.3e} (ratio {np.max(d / bound):.2f})"


@pytest.mark.parametrize("wname", ["b16384_s128_h128_bf16_g2", "tiny_b256_s16_h32"])
def test_standalone_update_matches_oracle(m, wname):
    import torch
    w = synth.WORKLOADS[wname]
    tr, tX, tq = _trainer(m, w, 512)
    P = iql.num_params(w.S, w.H, w.hidden2)
    assert np.array_equal(_get(tr, 0, "target"), _get(tr, 0, "params"))  # starts at the initial weights
    tr.train_step(tX, tq, 512)
    g = np.random.default_rng(5)
    t0 = [g.standard_normal(P).astype(np.float32) for _ in range(w.groups)]
    for gi in range(w.groups):
        tr.set_target(gi, to_dev(t0[gi]))
    tr.target_ema_update(0.3)
    sync()
    tau = float(np.float32(0.3))  # the value the device uses
    for gi in range(w.groups):
        p = _get(tr, gi, "params")
        ref = iql.target_ema(t0[gi], p, tau)
        _close(_get(tr, gi, "target"), ref, np.abs(t0[gi]) + np.abs(p), f"{wname} g{gi}")
    tr.close()


def test_fused_update_each_step_matches_oracle(m):
    """With the EMA folded into Adam, after every step the target is the
    oracle's update of the previous target toward that step's parameters."""
    w = synth.WORKLOADS["b16384_s128_h128_bf16_g2"]
    tr, tX, tq = _trainer(m, w, 2048)
    tr.set_target_ema(0.1)
    prev = [_get(tr, g, "target") for g in range(w.groups)]
    for step in range(3):
        tr.train_step(tX, tq, 2048)
        sync()
        for g in range(w.groups):
            now, p = _get(tr, g, "target"), _get(tr, g, "params")
            _close(now, iql.target_ema(prev[g], p, float(np.float32(0.1))), np.abs(prev[g]) + np.abs(p),
                   f"step {step} g{g}")
            prev[g] = now
    rc, flags = tr.status()
    assert rc == m.OK and flags == 0
    tr.close()


@pytest.mark.parametrize("wname", ["b16384_s128_h128_bf16_g2", "stress_b65536_s256_h512_bf16"])
def test_fused_equals_step_then_standalone_bitwise(m, wname):
    w = synth.WORKLOADS[wname]
    B = 4096
    a, aX, aq = _trainer(m, w, B)
    b, bX, bq = _trainer(m, w, B)
    a.set_target_ema(0.05)
    for _ in range(3):
        a.train_step(aX, aq, B)
        b.train_step(bX, bq, B)
        b.target_ema_update(0.05)
    sync()
    for g in range(w.groups):
        assert np.array_equal(_get(a, g, "target"), _get(b, g, "target")), g
        assert np.array_equal(_get(a, g, "params"), _get(b, g, "params")), g
    a.close()
    b.close()


def test_whole_step_folds_the_update(m):
    """iql_aux_step with the EMA set equals the same step followed by the
    standalone update, bit for bit."""
    import torch
    w = synth.WORKLOADS["b16384_s128_h128_bf16_g2"]
    B = 2048
    a, aX, aq = _trainer(m, w, B)
    b, bX, bq = _trainer(m, w, B)
    a.set_target_ema(0.2)
    out = [torch.zeros((w.groups, B), dtype=torch.float32, device=dev()) for _ in range(2)]
    for _ in range(2):
        a.aux_step(None, aX, aq, B, out_v=out[0])
        b.aux_step(None, bX, bq, B, out_v=out[1])
        b.target_ema_update(0.2)
    sync()
    for g in range(w.groups):
        assert np.array_equal(_get(a, g, "target"), _get(b, g, "target")), g
    a.close()
    b.close()


def test_rejects_tau_outside_unit_interval(m):
    w = synth.WORKLOADS["tiny_b256_s16_h32"]
    tr, _, _ = _trainer(m, w, 64)
    for bad in (-0.1, 1.5, float("nan")):
        with pytest.raises(m.IqlhError, match="tau"):
            tr.set_target_ema(bad)
        with pytest.raises(m.IqlhError, match="tau"):
            tr.target_ema_update(bad)
    tr.close()
