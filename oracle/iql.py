"""IQL value network V(s), expectile loss and Adam step: fp64 CPU reference.

Sources:
  * "GPU IQL + HER Porting Plan", section "Current State / IQL (CPU)":
    V(s) is Linear -> ReLU -> Linear -> ReLU -> Linear, state_dim -> hidden ->
    hidden -> 1; expectile loss on diff = Q(s,a) - V(s) with weight tau where
    diff >= 0 and 1 - tau where diff < 0, loss = mean(weight * diff^2); Q is a
    stop-gradient target (section "IQL GPU Porting / What Needs to Happen").
  * same page, section "CUDA Kernel: iql_value_kernel.cu": the six parameter
    tensors w_v1, b_v1, w_v2, b_v2, w_vout, b_vout live in one flat buffer, with
    separate Adam moments; the existing Adam kernel is reused on them with the
    arguments (lr, beta1, beta2, eps, weight_decay, max_grad_norm).
  * "DQN Backward-Path NaN Audit -- SP1 Phase A", section on
    ``iqn_adam_kernel``: norm = sqrt(max(sum g^2, 0)); clip factor
    max_grad_norm / norm when norm > max_grad_norm and norm > 0, else 1;
    non-finite gradients are zeroed and skip the update; bias-corrected moments
    m / (1 - beta1^t), v / (1 - beta2^t); denominator sqrt(v_hat) + eps; the step
    counter is incremented before use; gradients are zeroed after use.
  * same page, "Mech 9": optional post-update clamp |p| <= weight_clamp_max_abs
    (0 disables).

Weights are [out, in] row-major; flat order w1, b1, w2, b2, w3, b3.

``rnd`` (optional, e.g. ``bf16_operands``): the same definition with every
matrix-product operand rounded as a bf16-operand implementation stores it --
W1, W2, h1, dz2 (also in the b2 sum) and dz1 (also in the b1 sum); V, the
loss, dv and dw3 stay unrounded.  It separates the effect of bf16 operand
storage from that of the arithmetic order; the plain fp64 definition is the
parity reference.
Readings: ReLU'(0) = 0; weight tau at diff == 0; the
finite-check is applied after clipping, so a non-finite norm skips the whole
update; decoupled weight decay (AdamW order) when weight_decay != 0.
"""
from dataclasses import dataclass, field

import numpy as np

from oracle.bf16 import round_bf16


def bf16_operands(a):
    """fp64 values -> nearest bfloat16 (through binary32, as stored), fp64."""
    return round_bf16(np.asarray(a, dtype=np.float64).astype(np.float32)).astype(np.float64)


def _same(a):
    return a


def num_params(S, H1, H2):
    return S * H1 + H1 + H1 * H2 + H2 + H2 + 1


def unflatten(flat, S, H1, H2):
    """Views of the six tensors inside the flat parameter vector."""
    flat = np.asarray(flat)
    o = 0
    w1 = flat[o:o + H1 * S].reshape(H1, S); o += H1 * S
    b1 = flat[o:o + H1]; o += H1
    w2 = flat[o:o + H2 * H1].reshape(H2, H1); o += H2 * H1
    b2 = flat[o:o + H2]; o += H2
    w3 = flat[o:o + H2]; o += H2
    b3 = flat[o:o + 1]; o += 1
    assert o == flat.shape[0]
    return dict(w1=w1, b1=b1, w2=w2, b2=b2, w3=w3, b3=b3)


def flatten(t):
    return np.concatenate([t["w1"].ravel(), t["b1"], t["w2"].ravel(), t["b2"],
                           t["w3"].ravel(), np.atleast_1d(t["b3"])])


def forward(p, X, rnd=None):
    """V(s) for each row of X; returns (v, cache)."""
    R = rnd or _same
    X = np.asarray(X, dtype=np.float64)
    z1 = X @ R(p["w1"]).T + p["b1"]
    h1 = np.maximum(z1, 0.0)
    z2 = R(h1) @ R(p["w2"]).T + p["b2"]
    h2 = np.maximum(z2, 0.0)
    v = h2 @ p["w3"] + p["b3"][0]
    return v, dict(X=X, z1=z1, h1=h1, z2=z2, h2=h2)


def expectile(q, v, tau):
    """Expectile loss and its gradient with respect to v (q is stop-grad)."""
    q = np.asarray(q, dtype=np.float64)
    diff = q - v
    w = np.where(diff >= 0.0, tau, 1.0 - tau)
    B = diff.shape[0]
    loss = np.sum(w * diff * diff) / B
    dv = -2.0 * w * diff / B
    return loss, dv


def backward(p, cache, dv, rnd=None):
    """Gradients of sum(dv * v) with respect to the six tensors."""
    R = rnd or _same
    X, z1, h1, z2, h2 = cache["X"], cache["z1"], cache["h1"], cache["z2"], cache["h2"]
    g = {}
    g["w3"] = h2.T @ dv
    g["b3"] = np.array([np.sum(dv)])
    dz2 = R(np.outer(dv, p["w3"]) * (z2 > 0.0))
    g["w2"] = dz2.T @ R(h1)
    g["b2"] = dz2.sum(axis=0)
    dh1 = dz2 @ R(p["w2"])
    dz1 = R(dh1 * (z1 > 0.0))
    g["w1"] = dz1.T @ X
    g["b1"] = dz1.sum(axis=0)
    return g


def l2norm(g):
    g = np.asarray(g, dtype=np.float64)
    return float(np.sqrt(max(float(np.sum(g * g)), 0.0)))


def clip_coef(norm, max_norm):
    """Clip factor of the pages' Adam: only when norm > max and norm > 0.

    A non-finite norm yields NaN, so every clipped gradient is non-finite and
    the finite-guard skips the whole update."""
    if not np.isfinite(norm):
        return float("nan")
    if norm > max_norm and norm > 0.0:
        return max_norm / norm
    return 1.0


@dataclass
class AdamHP:
    lr: float = 3e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    max_grad_norm: float = 1.0
    weight_clamp_max_abs: float = 0.0


@dataclass
class AdamState:
    params: np.ndarray
    m: np.ndarray
    v: np.ndarray
    t: int = 0

    @staticmethod
    def fresh(params):
        p = np.array(params, dtype=np.float64, copy=True)
        return AdamState(p, np.zeros_like(p), np.zeros_like(p), 0)

    def copy(self):
        return AdamState(self.params.copy(), self.m.copy(), self.v.copy(), self.t)


def adam_step(st, grad, hp):
    """One clipped Adam update in place on ``st``; returns (norm, skipped_mask).

    ``norm`` is the pre-clip global L2 norm of ``grad``."""
    g = np.asarray(grad, dtype=np.float64)
    norm = l2norm(g) if np.all(np.isfinite(g)) else float("nan")
    c = clip_coef(norm, hp.max_grad_norm)
    st.t += 1
    t = st.t
    with np.errstate(invalid="ignore", over="ignore"):
        gc = c * g
    ok = np.isfinite(gc)
    gc = np.where(ok, gc, 0.0)
    m_new = hp.beta1 * st.m + (1.0 - hp.beta1) * gc
    v_new = hp.beta2 * st.v + (1.0 - hp.beta2) * gc * gc
    m_hat = m_new / (1.0 - hp.beta1 ** t)
    v_hat = v_new / (1.0 - hp.beta2 ** t)
    p = st.params
    if hp.weight_decay != 0.0:
        p_new = p * (1.0 - hp.lr * hp.weight_decay)
    else:
        p_new = p
    p_new = p_new - hp.lr * m_hat / (np.sqrt(v_hat) + hp.eps)
    if hp.weight_clamp_max_abs > 0.0:
        b = hp.weight_clamp_max_abs
        p_new = np.clip(p_new, -b, b)
    st.params = np.where(ok, p_new, p)
    st.m = np.where(ok, m_new, st.m)
    st.v = np.where(ok, v_new, st.v)
    return norm, ~ok


def bootstrap_target(rewards, dones, v_next, gamma):
    """IQL's bootstrap target with V(s') in place of the target network's
    maximum ("GPU IQL + HER Porting Plan", section "Phase 2 Integration",
    IQL modifies the target computation): r + gamma V(s').  Reading: terminal
    rows (done = 1) drop the bootstrap term, r + gamma (1 - done) V(s'), the
    usual DQN convention the pages' train step takes dones for; dones None
    means no terminal rows."""
    r = np.asarray(rewards, dtype=np.float64)
    d = np.zeros_like(r) if dones is None else np.asarray(dones, dtype=np.float64)
    return r + gamma * (1.0 - d) * np.asarray(v_next, dtype=np.float64)


def target_ema(target, online, tau):
    """Polyak averaging of the target copy ("GPU IQL + HER Porting Plan",
    section "Rust Integration: gpu_iql_trainer.rs", target_ema_update; applied
    after the IQL step, section "Where in the Training Loop IQL Gets
    Called"): (1 - tau) target + tau online, elementwise."""
    return (1.0 - tau) * np.asarray(target, dtype=np.float64) + tau * np.asarray(online, dtype=np.float64)


@dataclass
class StepResult:
    loss: float
    v: np.ndarray
    grad: np.ndarray
    grad_norm: float
    skipped: np.ndarray = field(default=None)


def train_step(st, X, q, S, H1, H2, tau, hp, rnd=None):
    """V forward, expectile loss, backward and clipped Adam, in place on st.

    Returns the loss, V(s) before the update, the flat gradient and its
    pre-clip norm."""
    p = unflatten(st.params, S, H1, H2)
    v, cache = forward(p, X, rnd)
    loss, dv = expectile(q, v, tau)
    g = flatten(backward(p, cache, dv, rnd))
    norm, skipped = adam_step(st, g, hp)
    return StepResult(loss=loss, v=v, grad=g, grad_norm=norm, skipped=skipped)
