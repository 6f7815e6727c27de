"""Budgeted clipped-SAXPY gradient accumulation, fp64 CPU reference.

Source: "Gradient Stability -- Proper Multi-Task Gradient Isolation + Full
Spectral Norm", section "Design -- Why the current per-component clipping is
wrong", subsection "Proper design": each gradient source k owns a fraction f_k
of max_grad_norm (0.70 / 0.15 / 0.10 / 0.05, summing to 1); the primary is
clipped in place to its budget, every further source is clipped to its own
budget in isolation and added with a scale (CQL 1, IQN lambda, ensemble s);
Adam then applies its usual safety clip at max_grad_norm.  Section "Task 1"
gives the clipped SAXPY as grad += alpha * clip(scratch, budget), where the
clip uses the norm of the scratch buffer alone.

Clip rule (same as the Adam clip of "DQN Backward-Path NaN Audit"): scale by
budget / norm when norm > budget and norm > 0, else leave unchanged.

Readings: alpha_0 multiplies the primary too (the page's primary has none,
i.e. alpha_0 = 1); lambda = s = 1 unless the caller passes others.
"""
import numpy as np

FRACTIONS = (0.70, 0.15, 0.10, 0.05)


def clip_scale(norm, budget):
    if norm > budget and norm > 0.0:
        return budget / norm
    return 1.0


def accumulate(sources, fractions, alphas, max_grad_norm):
    """Returns (grad, source_norms, combined_norm, scales)."""
    norms, scales = [], []
    grad = None
    for s, f, a in zip(sources, fractions, alphas):
        s = np.asarray(s, dtype=np.float64)
        n = float(np.sqrt(np.sum(s * s)))
        c = clip_scale(n, f * max_grad_norm)
        norms.append(n)
        scales.append(c)
        contrib = (a * c) * s
        grad = contrib if grad is None else grad + contrib
    combined = float(np.sqrt(np.sum(grad * grad)))
    return grad, norms, combined, scales
