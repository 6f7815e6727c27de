"""GPU parity of the forward-only value pass V(s') and of the bootstrap
target r + gamma (1 - done) V(s') against the oracle, on every kernel
family (16-wave bf16 hidden 128, the fp32 tile kernel, the wide-hidden
kernels, the layered kernels); V(s') equals the V(s) of a train step on the
same rows bit for bit; f32 input to a bf16 trainer equals its bf16-rounded
input; the pass changes no trainer state; the HER outputs feed it directly."""
import numpy as np
import pytest

import synth
from oracle import iql
from tests.gpu_util import assert_rel, dev, host, sync, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


CASES = [("b16384_s128_h128_bf16_g2", {}, 3000, 2e-2), ("tiny_b256_s16_h32", {}, 200, 1e-4),
         ("b4096_s42_h128_f32", {}, 1000, 1e-4), ("stress_b65536_s256_h512_bf16", {}, 2000, 2e-2),
         ("b16384_s128_h128_bf16_g2", {"S": 100, "H": 256}, 700, 2e-2),
         ("b16384_s128_h128_bf16_g2", {"S": 64, "H": 96, "H2": 160}, 900, 2e-2)]


def _setup(m, wname, kw, B, seed=0):
    import torch
    w = synth.shrink(synth.WORKLOADS[wname], **kw)
    bf = w.dtype == "bf16"
    g = np.random.default_rng(seed)
    Xn = g.standard_normal((B, w.S)).astype(np.float32)
    if bf:
        Xn = synth._bf16_values(Xn)
    r = np.where(g.random(B) < 0.3, 1.0, -0.01).astype(np.float32)
    d = (g.random(B) < 0.2).astype(np.float32)
    cfg = m.make_config(w.S, w.H, B, num_groups=w.groups, compute_dtype=m.BF16 if bf else m.F32, states_ld=w.S,
                        tau=w.taus, hidden2=w.H2)
    inits = synth.group_inits(w)
    tr = m.IqlTrainer(cfg, np.concatenate(inits))
    tX = to_dev(Xn, torch.bfloat16 if bf else torch.float32)
    return w, tr, Xn, tX, r, d, inits


@pytest.mark.parametrize("wname,kw,B,rtol", CASES)
def test_values_and_target_match_oracle(m, wname, kw, B, rtol):
    import torch
    w, tr, Xn, tX, r, d, inits = _setup(m, wname, kw, B)
    v = torch.zeros((w.groups, B), dtype=torch.float32, device=dev())
    tg = torch.zeros_like(v)
    tr.forward_values(tX, B, v, rewards=to_dev(r), dones=to_dev(d), gamma=0.97, out_target=tg)
    sync()
    for g in range(w.groups):
        ref_v = iql.forward(iql.unflatten(inits[g].astype(np.float64), w.S, w.H, w.hidden2), Xn)[0]
        assert_rel(host(v[g]), ref_v, rtol, f"{wname} V(s') g{g}")
        ref_t = iql.bootstrap_target(r, d, ref_v, 0.97)
        assert_rel(host(tg[g]), ref_t, rtol, f"{wname} target g{g}")
        # the target is formed from this V exactly as the definition says
        np.testing.assert_allclose(host(tg[g]), iql.bootstrap_target(r, d, host(v[g]), np.float32(0.97)),
                                   rtol=1e-6, atol=1e-6)
    tr.close()


@pytest.mark.parametrize("wname,kw,B,rtol", CASES)
def test_values_equal_train_step_v_and_change_nothing(m, wname, kw, B, rtol):
    import torch
    w, tr, Xn, tX, r, d, inits = _setup(m, wname, kw, B, seed=1)
    P = iql.num_params(w.S, w.H, w.hidden2)
    before = torch.zeros(P, device=dev())
    tr.get_state(0, before)
    v = torch.zeros((w.groups, B), dtype=torch.float32, device=dev())
    tr.forward_values(tX, B, v)
    after = torch.zeros(P, device=dev())
    tr.get_state(0, after)
    vs = torch.zeros_like(v)
    q = to_dev(np.zeros(B, np.float32))
    tr.train_step(tX, q, B, out_v=vs)
    sync()
    assert torch.equal(before, after)
    assert torch.equal(v, vs), f"{wname}: forward-only V differs from the train step's V"
    tr.close()


def test_f32_input_to_bf16_trainer(m):
    import torch
    w, tr, Xn, tX, r, d, inits = _setup(m, "b16384_s128_h128_bf16_g2", {}, 1500, seed=2)
    g = np.random.default_rng(9)
    X32 = g.standard_normal((1500, w.S)).astype(np.float32)
    v32 = torch.zeros((w.groups, 1500), device=dev())
    vbf = torch.zeros_like(v32)
    tr.forward_values(to_dev(X32), 1500, v32)
    tr.forward_values(to_dev(synth._bf16_values(X32), torch.bfloat16), 1500, vbf)
    sync()
    assert torch.equal(v32, vbf)
    tr.close()


def test_her_outputs_feed_the_target(m):
    """Relabelled next states (f32), rewards and dones straight from
    her_relabel give the oracle's target on the oracle's relabelled rows."""
    import torch
    from oracle import her
    w = synth.shrink(synth.WORKLOADS["b16384_s128_h128_bf16_g2"], B=2048, C=1 << 14)
    buf = synth.replay_buffer(w)
    src = synth.her_sources(w, buf)
    n = w.n_her
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev())  # noqa: E731
    hb = m.her_buffer(t(buf["states"]), t(buf["next_states"]), t(buf["actions"]), t(buf["dones"]),
                      t(buf["episode_ends"].astype(np.int32)))
    nxt = torch.zeros((n, w.S), device=dev())
    rew, don = torch.zeros(n, device=dev()), torch.zeros(n, device=dev())
    sts = torch.zeros((n, w.S), dtype=torch.bfloat16, device=dev())
    out = m.her_out(sts.data_ptr(), m.BF16, w.S, rew, next_states=nxt, dones=don)
    m.her_relabel(m.her_config(w.S, w.G, m.HER_FUTURE), hb, t(src.astype(np.int32)), n, 11, None, out)
    cfg = m.make_config(w.S, w.H, n, num_groups=w.groups, compute_dtype=m.BF16, states_ld=w.S, tau=w.taus)
    inits = synth.group_inits(w)
    tr = m.IqlTrainer(cfg, np.concatenate(inits))
    v = torch.zeros((w.groups, n), device=dev())
    tg = torch.zeros_like(v)
    tr.forward_values(nxt, n, v, rewards=rew, dones=don, gamma=0.99, out_target=tg)
    sync()
    ref = her.her_step(buf, src, w.G, her.FUTURE, 11, 0, out_bf16=True)
    Xs = synth._bf16_values(ref["next_states"].astype(np.float32))
    for g in range(w.groups):
        rv = iql.forward(iql.unflatten(inits[g].astype(np.float64), w.S, w.H, w.H), Xs)[0]
        assert_rel(host(tg[g]), iql.bootstrap_target(ref["rewards"], ref["dones"], rv, 0.99), 2e-2, f"target g{g}")
    tr.close()


def test_rejects_bad_arguments(m):
    import torch
    w, tr, Xn, tX, r, d, inits = _setup(m, "tiny_b256_s16_h32", {}, 64)
    v = torch.zeros((1, 64), device=dev())
    with pytest.raises(m.IqlhError, match="go together"):
        tr.forward_values(tX, 64, v, rewards=to_dev(r))
    with pytest.raises(m.IqlhError, match="batch"):
        tr.forward_values(tX, 65, v)
    with pytest.raises(m.IqlhError, match="gamma"):
        tr.forward_values(tX, 64, v, rewards=to_dev(r), out_target=v, gamma=float("inf"))
    tr.close()
