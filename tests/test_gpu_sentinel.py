"""GPU parity of the fused non-finite sentinel against the oracle
(bit-exact flags): special values at the first, last and middle positions
of aligned and unaligned buffers, empty and null slots, sticky flags, random
bit patterns; and the state check folded into the Adam launches."""
import numpy as np
import pytest

import synth
from oracle import sentinel
from tests.gpu_util import dev, host, sync, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


def _flags(m, bufs, init):
    import torch
    f = to_dev(np.array(init, np.int32))
    m.nonfinite_check(bufs, f)
    sync()
    return host(f)


def test_slots_match_oracle(m):
    import torch
    g = np.random.default_rng(1)
    a = g.standard_normal(1000).astype(np.float32)                 # clean
    b = g.standard_normal(5000).astype(np.float32); b[0] = np.nan  # first element
    c = g.standard_normal(4097 + 1).astype(np.float32); c[-1] = np.inf  # last element, unaligned view below
    d = g.standard_normal(1 << 22).astype(np.float32); d[(1 << 21) + 3] = -np.inf  # middle of a long slot
    e = np.array([np.finfo(np.float32).max, -np.finfo(np.float32).max, 1e-45, -0.0], np.float32)  # finite extremes
    f = g.standard_normal(4096).astype(np.float32)
    f[4095] = np.nan                                                # last element of a whole piece
    host_bufs = [a, b, c[1:], d, e, np.zeros(0, np.float32), None, f]
    tc = torch.from_numpy(c).to(dev())
    tbufs = [to_dev(a), to_dev(b), tc[1:], to_dev(d), to_dev(e), torch.zeros(0, device=dev()), None, to_dev(f)]
    init = [0, 0, 0, 0, 0, 0, 0, 0]
    got = _flags(m, tbufs, init)
    ref = sentinel.update_flags(init, host_bufs)
    assert np.array_equal(got, ref), (got, ref)
    assert list(ref) == [0, 1, 1, 1, 0, 0, 0, 1]


def test_piece_edges(m):
    """Special values at the edges of the kernel's 8192-element pieces: the
    last element of a whole piece, the first of the next whole piece, the
    first and last of a slot's partial last piece, and a clean slot of
    whole pieces only."""
    g = np.random.default_rng(5)
    P = 8192
    cases = []
    for n, pos, val in ((P, P - 1, np.nan), (3 * P, P, np.inf), (2 * P + 5, 2 * P, -np.inf),
                        (2 * P + 5, 2 * P + 4, np.nan), (4 * P, None, None)):
        x = g.standard_normal(n).astype(np.float32)
        if pos is not None:
            x[pos] = val
        cases.append(x)
    init = [0] * len(cases)
    got = _flags(m, [to_dev(x) for x in cases], init)
    ref = sentinel.update_flags(init, cases)
    assert np.array_equal(got, ref), (got, ref)
    assert list(ref) == [1, 1, 1, 1, 0]


def test_flags_are_sticky(m):
    clean = to_dev(np.ones(300, np.float32))
    got = _flags(m, [clean, clean, None], [1, 0, 1])
    assert list(got) == [1, 0, 1]


def test_random_bit_patterns(m):
    import torch
    r = np.random.default_rng(7).integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32)
    for lo in range(0, 20000, 997):
        chunk = r[lo:lo + 997].view(np.float32)
        t = torch.from_numpy(chunk.copy()).to(dev())
        got = _flags(m, [t], [0])
        assert got[0] == sentinel.update_flags([0], [chunk])[0]


def test_rejects_bad_arguments(m):
    t = to_dev(np.ones(4, np.float32))
    with pytest.raises(m.IqlhError):
        m.nonfinite_check([t] * 33, to_dev(np.zeros(33, np.int32)))
    with pytest.raises(m.IqlhError):
        m.nonfinite_check([t], None)


def test_adam_state_sentinel(m):
    """An Adam update whose decoupled weight decay overflows (lr * wd = 1e40
    in fp32: the decay factor is -inf) writes non-finite parameters; the state
    flag is raised and iql_status reports it.  A normal update does not."""
    w = synth.WORKLOADS["tiny_b256_s16_h32"]
    g = np.random.default_rng(0)
    X = to_dev(g.standard_normal((256, w.S)).astype(np.float32))
    q = to_dev(g.standard_normal(256).astype(np.float32))
    for lr, wd, expect in ((3e-4, 0.0, False), (1e20, 1e20, True)):
        cfg = m.make_config(w.S, w.H, 256, num_groups=1, compute_dtype=m.F32, states_ld=w.S, tau=w.taus, lr=lr,
                            weight_decay=wd)
        tr = m.IqlTrainer(cfg, synth.group_inits(w)[0])
        tr.train_step(X, q, 256)
        rc, flags = tr.status()
        assert bool(flags & m.FLAG_NONFINITE_STATE) == expect, (lr, wd, flags)
        assert (rc == m.ENONFINITE) == expect
        tr.close()


def test_budget_adam_state_sentinel(m):
    import torch
    n = 1000
    g = np.random.default_rng(2)
    src = [to_dev(g.standard_normal(n).astype(np.float32))]
    for lr, wd, expect in ((3e-4, 0.0, False), (1e20, 1e20, True)):
        theta = to_dev(g.standard_normal(n).astype(np.float32))
        mm, vv = torch.zeros(n, device=dev()), torch.zeros(n, device=dev())
        t = torch.zeros(1, dtype=torch.int32, device=dev())
        flags = torch.zeros(1, dtype=torch.int32, device=dev())
        grad = torch.zeros(n, device=dev())
        ws = torch.zeros(m.grad_budget_workspace_bytes(n, 1) // 4 + 1, device=dev())
        adam = m.make_adam(theta, mm, vv, t, lr=lr, weight_decay=wd, max_grad_norm=1.0, d_flags=flags)
        m.grad_budget_accumulate(grad, src, (1.0,), (1.0,), n, 1.0, None, adam, ws)
        sync()
        assert bool(host(flags)[0] & m.FLAG_NONFINITE_STATE) == expect
