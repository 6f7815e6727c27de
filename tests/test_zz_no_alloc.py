"""grad_budget_accumulate_noalloc (the library's static device scratch in place
of a caller workspace) against grad_budget_accumulate: the same passes on the
same inputs, so every output must agree bit for bit.  Two calls in a row, the
second on fewer elements, so that the second call runs on scratch contents the
first one left behind."""
import numpy as np
import pytest

from tests.gpu_util import dev, host, sync, to_dev

pytestmark = pytest.mark.gpu

FRACS = (0.70, 0.15, 0.10, 0.05)
SCALES = (1.0, 5.0, 0.5, 0.2)


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


def _inputs(n, seed):
    g = np.random.default_rng(seed)
    src = [(g.standard_normal(n) * s).astype(np.float32) for s in SCALES]
    theta = (g.standard_normal(n) * 0.05).astype(np.float32)
    return src, theta


def _run(m, n, src, theta, noalloc, steps):
    """`steps` budgeted accumulations + Adam updates; returns every output."""
    import torch
    k = len(src)
    ts = [to_dev(s) for s in src]
    grad = torch.zeros(n, dtype=torch.float32, device=dev())
    norms = torch.zeros(k + 1, dtype=torch.float32, device=dev())
    p = to_dev(theta)
    mm = torch.zeros(n, dtype=torch.float32, device=dev())
    vv = torch.zeros(n, dtype=torch.float32, device=dev())
    t = torch.zeros(1, dtype=torch.int32, device=dev())
    adam = m.make_adam(p, mm, vv, t, lr=3e-4, max_grad_norm=1.0)
    ws = None
    if not noalloc:
        ws = torch.zeros(m.grad_budget_workspace_bytes(n, k) // 4, dtype=torch.float32, device=dev())
    for _ in range(steps):
        if noalloc:
            m.grad_budget_accumulate_noalloc(grad, ts, FRACS, (1.0,) * k, n, 1.0, norms, adam)
        else:
            m.grad_budget_accumulate(grad, ts, FRACS, (1.0,) * k, n, 1.0, norms, adam, ws)
    # accumulation only (no Adam): grad keeps the clipped sum
    g2 = torch.zeros(n, dtype=torch.float32, device=dev())
    n2 = torch.zeros(k + 1, dtype=torch.float32, device=dev())
    if noalloc:
        m.grad_budget_accumulate_noalloc(g2, ts, FRACS, (1.0,) * k, n, 1.0, n2, None)
    else:
        m.grad_budget_accumulate(g2, ts, FRACS, (1.0,) * k, n, 1.0, n2, None, ws)
    sync()
    return {name: host(x) for name, x in
            dict(params=p, m=mm, v=vv, t=t, norms=norms, grad=g2, norms_acc=n2, grad_zeroed=grad).items()}


def test_noalloc_matches_workspace_entry_point_on_two_calls(m):
    # first call: the budgeted network of the whole step (132,612 parameters,
    # 518 blocks of partials); second: a smaller n with a ragged last quad
    for n, seed, steps in ((132612, 1, 3), (1001, 2, 2)):
        print(f"noalloc parity n={n} steps={steps}", flush=True)
        src, theta = _inputs(n, seed)
        ref = _run(m, n, src, theta, noalloc=False, steps=steps)
        got = _run(m, n, src, theta, noalloc=True, steps=steps)
        for key in ref:
            assert np.array_equal(got[key].view(np.uint32) if got[key].dtype == np.float32 else got[key],
                                  ref[key].view(np.uint32) if ref[key].dtype == np.float32 else ref[key]), (n, key)
        assert int(got["t"][0]) == steps
        assert np.all(got["grad_zeroed"] == 0.0)


def test_noalloc_rejects_bad_arguments_on_the_host(m):
    import ctypes
    srcs = (ctypes.c_void_p * 9)(*([16] * 9))
    fr = (ctypes.c_float * 9)(*([0.1] * 9))
    assert m._lib_budget_noalloc(ctypes.c_void_p(16), srcs, fr, fr, 9, 100, 1.0, None, None, None) == m.EINVAL
    assert m._lib_budget_noalloc(ctypes.c_void_p(16), srcs, fr, fr, 4, 0, 1.0, None, None, None) == m.EINVAL
    assert m._lib_budget_noalloc(None, srcs, fr, fr, 4, 100, 1.0, None, None, None) == m.EINVAL
