"""GPU parity of prioritized-replay source sampling against the oracle.

Indices are compared element by element; a draw may differ only where its u
lies within rounding of a prefix-sum boundary (the GPU's binary64 prefix sums
add in another order), and then the GPU's row must be one of the two rows at
that boundary.  The block sums the GPU leaves in the workspace are checked
against the plain binary64 sums.  Weights: 1e-6 relative against the definition evaluated on the
GPU's own rows (one binary64 pow, one rounding to f32)."""
import numpy as np
import pytest

from oracle import per
from tests.gpu_util import dev, host, sync, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


def _run(m, p, n, seed, beta, step=None):
    import torch
    size = p.size
    ws = torch.zeros((m.per_workspace_bytes(size) + 7) // 8, dtype=torch.float64, device=dev())
    idx = torch.full((max(n, 1),), -7, dtype=torch.int32, device=dev())
    w = torch.full((max(n, 1),), -7.0, dtype=torch.float32, device=dev())
    flags = torch.zeros(1, dtype=torch.int32, device=dev())
    d_step = None if step is None else to_dev(np.array([step], np.int64))
    m.per_sample_indices(to_dev(p), n, seed, beta, idx, w, ws, d_step=d_step, d_flags=flags)
    sync()
    nb = (size + 2047) // 2048
    return host(idx)[:n], host(w)[:n], host(ws)[:nb], int(host(flags)[0])


@pytest.mark.parametrize("size,n,zero_frac", [(1, 5, 0.0), (1000, 4096, 0.2), (2049, 777, 0.5),
                                              ((1 << 20) + 7, 8192, 0.2), (5000, 1, 0.9),
                                              # both sides of the switch at 8192 blocks (2^24 rows): the
                                              # last table that fits in LDS (8192 and 8191 blocks), then
                                              # the table of block ends in global memory
                                              (1 << 24, 4096, 0.2), ((1 << 24) - 2048, 4096, 0.2),
                                              ((1 << 24) + 3001, 4096, 0.2)])
def test_draws_match_oracle(m, size, n, zero_frac):
    g = np.random.default_rng(size)
    p = (g.random(size) * 3).astype(np.float32)
    p[g.random(size) < zero_frac] = 0.0
    p[g.integers(size)] = 1.5  # at least one positive row
    seed, step, beta = 20261202, 3, 0.4
    gi, gw, gbs, flags = _run(m, p, n, seed, beta, step)
    oi, ow, ou, opre = per.sample(p, n, seed, step, beta)
    assert flags == 0
    # the workspace starts with the binary64 sum of every 2048-row block
    nb = gbs.size
    padded = np.zeros(nb * 2048, np.float64)
    padded[:size] = p
    np.testing.assert_allclose(gbs, padded.reshape(nb, 2048).sum(axis=1), rtol=1e-12, atol=1e-300)
    total = opre[-1]
    diff = np.nonzero(gi != oi)[0]
    for k in diff:  # only at a boundary, and only to its neighbour row
        lo, hi = sorted((int(gi[k]), int(oi[k])))
        assert abs(ou[k] - opre[lo]) <= 1e-12 * total, (k, gi[k], oi[k])
        assert np.all(p[lo + 1:hi] == 0.0)
    assert diff.size <= 2
    assert np.all(p[gi] > 0)
    ref_w = (p[gi].astype(np.float64).min() / p[gi].astype(np.float64)) ** beta
    np.testing.assert_allclose(gw, ref_w, rtol=1e-6)
    assert gw.max() == 1.0


def test_uniform_priorities_give_unit_weights_and_steps_differ(m):
    p = np.full(3000, 0.25, np.float32)
    i0, w0, _, _ = _run(m, p, 2000, 7, 0.9, step=0)
    i1, w1, _, _ = _run(m, p, 2000, 7, 0.9, step=1)
    assert np.all(w0 == 1.0) and np.all(w1 == 1.0)
    assert np.mean(i0 != i1) > 0.9
    np.testing.assert_array_equal(i0, per.sample(p, 2000, 7, 0, 0.9)[0])
    np.testing.assert_array_equal(_run(m, p, 2000, 7, 0.9)[0], i0)  # no step counter = step 0


def test_bad_priorities_raise_the_flag(m):
    p = np.ones(100, np.float32)
    p[40] = -1.0
    _, _, _, flags = _run(m, p, 10, 1, 0.5)
    assert flags & m.FLAG_BAD_INDEX
    z = np.zeros(100, np.float32)
    idx, w, _, flags = _run(m, z, 10, 1, 0.5)
    assert flags & m.FLAG_BAD_INDEX and np.all(idx == -1) and np.all(w == 0.0)


def test_rejects_bad_arguments(m):
    import torch
    p = to_dev(np.ones(10, np.float32))
    ws = torch.zeros(1, dtype=torch.float64, device=dev())
    idx = torch.zeros(4, dtype=torch.int32, device=dev())
    w = torch.zeros(4, device=dev())
    with pytest.raises(m.IqlhError, match="workspace"):
        m.per_sample_indices(p, 4, 1, 0.5, idx, w, ws)
    big = torch.zeros(64, dtype=torch.float64, device=dev())
    with pytest.raises(m.IqlhError, match="beta"):
        m.per_sample_indices(p, 4, 1, -1.0, idx, w, big)
