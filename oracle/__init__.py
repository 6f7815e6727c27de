"""CPU reference (oracle) for the IQL + HER auxiliary-trainer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table
or constant generator with the HIP library in ``offline_rl_step_amd/``.

Everything here is written from the text of these pages (cited by page title
and section in each function):

* "GPU IQL + HER Porting Plan" -- the IQL value network, expectile loss,
  advantage-weighted policy, the HER relabel kernel and donor strategies.
* "DQN Backward-Path NaN Audit -- SP1 Phase A" -- the Adam / gradient-norm
  semantics (section on ``iqn_adam_kernel``).
* "Phase 2: Multi-Stream Graph Parallelism" -- grouped high/low IQL trainers.
* "Gradient Stability -- Proper Multi-Task Gradient Isolation + Full Spectral
  Norm" -- budgeted clipped-SAXPY accumulation.

Floating point is fp64 (NumPy) except where the pages fix the precision (the
HER reward decision, which the pages' relabel kernel takes in fp32).

Modules
-------
philox   Philox4x64-10 counter-based generator (Salmon et al., SC'11).
her      donor selection (final / future / random) and goal relabelling.
iql      value-MLP forward / backward, expectile loss, grad norm, Adam step.
aw       advantage-weighted policy.
budget   budgeted clipped-SAXPY gradient accumulation.
bf16     round-to-nearest-even float32 -> bfloat16 (storage rounding).

Parity status: every function is pinned by tests in ``tests/test_oracle_*.py``
(closed forms, library special cases, finite differences, brute force and
hand-worked fixtures); none is "parity unpinned".
"""

from . import philox, her, iql, aw, budget, bf16  # noqa: F401
