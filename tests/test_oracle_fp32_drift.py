"""How far an exact float32 implementation of the step drifts from the fp64
oracle over 100 free-running steps of the 4096-batch / state-42 workload (CPU
only): the basis of the free-running bounds in the GPU test of that workload
(parameters within 1e-3 norm-wise and 10 lr element-wise, the loss within
1e-4, after 100 steps).

The float32 side is written independently of the oracle: torch float32
autograd of the same network and expectile loss, the same clip and Adam
update in float32 arithmetic.  Adam divides by sqrt(v), so an element whose
gradient is near zero amplifies rounding; the drift is real but bounded.
"""
import numpy as np
import torch

import synth
from oracle import iql


def test_float32_drift_over_hundred_steps_is_inside_the_free_running_bounds():
    w = synth.WORKLOADS["b4096_s42_h128_f32"]
    S, H, B, tau, lr = w.S, w.H, w.B, w.taus[0], w.lr
    g = np.random.default_rng(0)
    X = g.standard_normal((B, S)).astype(np.float32)
    q = (g.standard_normal(B) * w.q_sd).astype(np.float32)
    p0 = synth.kaiming_uniform(w)
    hp = iql.AdamHP(lr=lr, max_grad_norm=w.max_grad_norm)
    st = iql.AdamState.fresh(p0)
    P = iql.num_params(S, H, H)
    p = torch.tensor(p0, dtype=torch.float32)
    m, v = torch.zeros(P), torch.zeros(P)
    Xt, qt = torch.tensor(X), torch.tensor(q)
    drift = {}
    for t in range(1, 101):
        ref = iql.train_step(st, X, q, S, H, H, tau, hp)
        pp = p.clone().requires_grad_(True)
        o = 0
        w1 = pp[o:o + H * S].view(H, S); o += H * S
        b1 = pp[o:o + H]; o += H
        w2 = pp[o:o + H * H].view(H, H); o += H * H
        b2 = pp[o:o + H]; o += H
        w3 = pp[o:o + H]; o += H
        b3 = pp[o]
        vv = torch.relu(torch.relu(Xt @ w1.T + b1) @ w2.T + b2) @ w3 + b3
        d = qt - vv
        loss = (torch.where(d >= 0, tau, 1.0 - tau) * d * d).mean()
        loss.backward()
        gr = pp.grad.detach()
        n = gr.norm()
        if n > hp.max_grad_norm:
            gr = gr * (hp.max_grad_norm / n)
        m = hp.beta1 * m + (1 - hp.beta1) * gr
        v = hp.beta2 * v + (1 - hp.beta2) * gr * gr
        p = p - lr * (m / (1 - hp.beta1 ** t)) / (torch.sqrt(v / (1 - hp.beta2 ** t)) + hp.eps)
        if t in (1, 10, 100):
            pn = p.numpy().astype(np.float64)
            drift[t] = (np.linalg.norm(pn - st.params) / np.linalg.norm(st.params), np.max(np.abs(pn - st.params)),
                        abs(float(loss) - ref.loss) / ref.loss)
    # one step: float32 rounding only
    assert drift[1][0] < 1e-5
    # after 100 free-running steps: well past one step's rounding, inside the
    # bounds the GPU test uses, with room to spare
    rel, mx, loss_rel = drift[100]
    assert 1e-6 < rel < 1e-3 / 2
    assert mx < 10 * lr / 2
    assert loss_rel < 1e-4
