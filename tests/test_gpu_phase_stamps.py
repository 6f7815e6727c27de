"""The measurement aid iql_aux_step_phase_stamps: the headline step (batch
16384, two bf16 trainers of hidden 128, HER and the budget's pass 1 inside
the forward/backward launch) run through the kernel instantiation that
records each workgroup's phase ends gives the same outputs and trainer
state as iql_aux_step, bit for bit, and its clock values are ordered within
every workgroup."""
import numpy as np
import pytest

import synth
from tests.gpu_util import dev, host, sync
from tests.test_gpu_step import Inputs, Rig

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import offline_rl_step_amd as m
    return m


def test_phase_stamps_step_equals_plain_step(m):
    import torch
    w = synth.WORKLOADS["b16384_s128_h128_bf16_g2_budget"]
    inp = Inputs(w, w.B, w.n_budget)
    a, b = Rig(m, inp), Rig(m, inp)
    ntile = (w.B + 127) // 128
    stamps = torch.zeros(w.groups * ntile * m.PHASE_STAMPS, dtype=torch.int64, device=dev())
    for _ in range(2):
        a.whole()
        her = m.her_step(b.hcfg, b.hbuf, inp.t_src, inp.n, b.seed, b.hout)
        bud = m.budget_step(b.grad, inp.t_sources, w.budget_fractions, (1.0, 1.0, 1.0, 1.0), inp.n_budget,
                            w.max_grad_norm, b.norms, b.adam, b.ws)
        b.tr.aux_step_phase_stamps(her, b.X, inp.t_q, inp.B, inp.t_Q, w.A, w.beta, b.pi, b.out_v, b.out_loss,
                                   b.out_gn, bud, stamps)
    sync()
    ta, tb = a.tensors(), b.tensors()
    for k in ta:
        assert torch.equal(ta[k], tb[k]), k
    st = host(stamps).reshape(w.groups, ntile, m.PHASE_STAMPS)
    assert (st > 0).all()
    assert (np.diff(st, axis=2) >= 0).all()
    # every workgroup of the launch ran within one short window
    assert st[..., -1].max() - st[..., 0].min() < 100000  # 1 ms at 100 MHz


def test_phase_stamps_reject_other_kernels(m):
    import torch
    w = synth.shrink(synth.WORKLOADS["tiny_b256_s16_h32"], B=256)
    inp = Inputs(w, w.B, 4096)
    r = Rig(m, inp, her=False, budget=False)
    stamps = torch.zeros(4096, dtype=torch.int64, device=dev())
    with pytest.raises(RuntimeError, match="hidden-128"):
        r.tr.aux_step_phase_stamps(None, r.X, inp.t_q, inp.B, inp.t_Q, w.A, w.beta, r.pi, r.out_v, r.out_loss,
                                   r.out_gn, None, stamps)
