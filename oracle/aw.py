"""Advantage-weighted policy, fp64 CPU reference.

Source: "GPU IQL + HER Porting Plan", section "Current State / IQL (CPU)",
item "Advantage-weighted action selection": A(s,a) = Q(s,a) - V(s) per action;
pi(a|s) = softmax(beta * clamp(A, -10, 10)) with the maximum subtracted before
exponentiation; output [batch, num_actions].

Reading: the clamp is applied to A before the multiplication by beta, as the
formula is written.
"""
import numpy as np

CLAMP = 10.0


def aw_policy(Q, V, beta):
    Q = np.asarray(Q, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    x = beta * np.clip(Q - V[:, None], -CLAMP, CLAMP)
    x = x - np.max(x, axis=1, keepdims=True)
    e = np.exp(x)
    return e / np.sum(e, axis=1, keepdims=True)
