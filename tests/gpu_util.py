"""Helpers for the GPU parity tests (device tensors, tolerance checks)."""
import numpy as np


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev())


def host(t):
    import torch
    if t.dtype == torch.bfloat16:
        t = t.to(torch.float32)
    return t.detach().cpu().numpy()


def sync():
    import torch
    torch.cuda.synchronize()


def assert_rel(gpu, ref, rtol, what=""):
    """Norm-wise and max-wise relative agreement of one tensor:
    ||x - y|| <= rtol ||y||  and  max|x - y| <= rtol max|y|."""
    x = np.asarray(gpu, dtype=np.float64).ravel()
    y = np.asarray(ref, dtype=np.float64).ravel()
    assert x.shape == y.shape, (what, x.shape, y.shape)
    assert np.all(np.isfinite(x)), f"{what}: non-finite GPU values"
    d = x - y
    ny, my = np.linalg.norm(y), np.max(np.abs(y)) if y.size else 0.0
    nd, md = np.linalg.norm(d), np.max(np.abs(d)) if d.size else 0.0
    assert nd <= rtol * ny + 1e-30, f"{what}: norm-wise rel err {nd / max(ny, 1e-300):.3e} > {rtol}"
    assert md <= rtol * my + 1e-30, f"{what}: max-wise rel err {md / max(my, 1e-300):.3e} > {rtol}"


def assert_scalar_rel(gpu, ref, rtol, what=""):
    g, r = float(gpu), float(ref)
    assert np.isfinite(g), what
    assert abs(g - r) <= rtol * abs(r) + 1e-30, f"{what}: {g} vs {r} (rel {abs(g - r) / max(abs(r), 1e-300):.3e})"


def adam_update_close(p_gpu, p_ref, p0, lr, steps, rtol, what=""):
    """Adam updates are bounded by about lr per step and element, and an element
    whose gradient is within rounding of zero may take either sign at t = 1.
    Compare the parameters norm-wise and max-wise at rtol, with the max-wise
    bound relaxed to the update bound 2 * lr * steps for at most 0.1 % of the
    elements."""
    x = np.asarray(p_gpu, np.float64)
    y = np.asarray(p_ref, np.float64)
    d = np.abs(x - y)
    assert np.all(np.isfinite(x)), what
    assert np.linalg.norm(x - y) <= rtol * np.linalg.norm(y), \
        f"{what}: norm-wise rel err {np.linalg.norm(x - y) / np.linalg.norm(y):.3e}"
    big = d > rtol * np.max(np.abs(y))
    assert np.mean(big) <= 1e-3, f"{what}: {int(big.sum())} elements beyond rtol"
    assert np.all(d <= 2.0 * lr * steps + rtol * np.max(np.abs(y))), f"{what}: beyond the Adam step bound"
