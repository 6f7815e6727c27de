#!/usr/bin/env python3
"""Throughput of the IQL + HER auxiliary-trainer step on one MI355X.

One step, on synthetic inputs resident in HBM (batch 16384, state_dim 128,
two value trainers of hidden width 128, 9 actions, bf16 GEMM operands), is
one iql_aux_step call:
  1. HER relabelling  -- 8192 rows, "future" donors, written into the tail of
                         the merged bf16 batch (replay buffer of 2^20 rows);
  2. the IQL step     -- both trainers: fused forward/backward (MFMA) with the
                         AW policy from this step's V in the same launch,
                         fixed-order gradient reduction, clipped Adam;
  3. the budget       -- four sources over 132612 parameters, budgets
                         0.70/0.15/0.10/0.05 of max_grad_norm 1.0, then Adam;
in three launches (forward/backward + policy + HER rows + budget norms |
reduction + SAXPY | both Adam updates): the HER rows form the batch tail from
a 128-row boundary, so the forward/backward kernel relabels them itself, and
the budget norms ride on its other workgroups.  Shapes where that does not
hold add a first launch (HER + budget norms).  --separate times her_relabel +
iql_train_step_aw + grad_budget_accumulate called one after the other
instead (same results bit for bit, seven launches).  Each step is one call
of the entry point, launched eagerly on one stream: with three launches per
step the host stays ahead of the GPU, and the launches run back to back
(measured 35.8 us per step, against 40.5 us when the step is captured once in
a HIP graph and replayed, because each graph replay adds about 4.7 us).
--graph times graph replay instead (the HER donor counter lives on the
device, so every replay draws new donors); the line carries the other mode's
time per step as well.

Prints ONE JSON line.  `value` = samples/s = batch / wall-clock time per step
over the timed replays.  `roofline` is for the dominant kernel (the fused
value-MLP forward/backward), timed with HIP events recorded by its own
dispatches.  `cpu_baseline` times the fp64 NumPy oracle on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "IQL+HER train samples/sec at B=16384; % bf16 MFMA peak / % HBM BW"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X dense fp32 matrix
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--graph", action="store_true", help="capture the step once in a HIP graph and replay it")
    p.add_argument("--no-graph", action="store_true", help="eager launches (the default)")
    p.add_argument("--separate", action="store_true",
                   help="the three entry points one after the other instead of iql_aux_step")
    p.add_argument("--workload", default=None,
                   help="time another workload of the input recipe (default: the batch-16384 two-trainer "
                        "step with the budget); the CPU baseline then runs only when --cpu-baseline is given")
    p.add_argument("--cpu-baseline", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-next-rows", action="store_true",
                   help="skip timing the widening entry points (forward values, target EMA, sentinel, sampling)")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--kernel-reps", type=int, default=200)
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run 10 plain device copies of MIB MiB (counter calibration) and exit")
    p.add_argument("--probe", choices=("team-fold", "xcc-map", "stream-sum"), default=None,
                   help="only run one measurement probe of libiqlh_probes.so and print one JSON line: "
                        "team-fold (the split-K partials summed inside the writing launch, against a "
                        "separate summing launch), xcc-map (the XCD of each block of a launch of the "
                        "forward/backward kernel's shape), stream-sum (a read-only four-array sum of squares "
                        "of 1 GiB cut into blocks three ways)")
    p.add_argument("--phases", action="store_true",
                   help="only run the headline step through iql_aux_step_phase_stamps and print one JSON line: "
                        "the forward/backward kernel's phase durations per workgroup (median over steps and "
                        "workgroups, HER tiles and plain tiles apart)")
    p.add_argument("--sweep", choices=("her", "aw", "budget", "sentinel", "copy"), default=None,
                   help="only time one HBM-bound entry point on working sets of at least 1 GiB (her_relabel over "
                        "a 2^22-row replay buffer, iql_aw_policy up to B*A = 2^26 for two trainers, "
                        "grad_budget_accumulate + Adam up to n = 2^26, iqlh_nonfinite_check over eight slots up to "
                        "4 GiB) and print one JSON line per size")
    p.add_argument("--sweep-calls", type=int, default=3, help="timed calls per sweep size (after one warm-up)")
    p.add_argument("--summarize-sweeps", metavar="DIR", default=None,
                   help="only write profiles/hbm_sweeps.md from the sweep logs and rocprofv3 CSV output under DIR "
                        "(sweep_KIND.json, sweep_KIND_FETCH_SIZE/, sweep_KIND_WRITE_SIZE/ for each sweep, copy_FETCH_SIZE/, "
                        "copy_WRITE_SIZE/); needs no GPU")
    p.add_argument("--summarize-profiles", metavar="DIR", default=None,
                   help="only write the profile summaries (markdown + traffic JSON) into profiles/ from the "
                        "rocprofv3 CSV output under DIR (trace/, FETCH_SIZE/, WRITE_SIZE/, copy_FETCH_SIZE/, "
                        "copy_WRITE_SIZE/); needs no GPU")
    return p.parse_args()


def copy_probe(mib):
    """A plain copy kernel of known size: HBM counters of one dispatch should
    read mib MiB and write mib MiB; the ratio calibrates FETCH_SIZE/WRITE_SIZE."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_mib": mib, "bytes_per_copy": n * 4}), flush=True)


def run_probe(name, reps=50):
    """One probe of libiqlh_probes.so (built by offline_rl_step_amd/build.py)."""
    import ctypes
    import torch
    torch.cuda.init()
    lib = ctypes.CDLL(os.path.join(ROOT, "offline_rl_step_amd", "libiqlh_probes.so"))
    if name == "team-fold":
        us = (ctypes.c_double * 9)()
        eq = (ctypes.c_int * 2)()
        to = ctypes.c_int(0)
        rc = lib.iqlh_probe_team_fold(ctypes.c_int(reps), us, eq, ctypes.byref(to))
        if rc != 0:
            raise RuntimeError(f"iqlh_probe_team_fold returned {rc}")
        out = {"probe": name, "reps": reps, "rows": 256, "row_floats": 33280, "team": 16}
        for i, v in enumerate(("base", "fold_all_release", "fold_one_release")):
            out[v] = {"rows_us": us[3 * i], "sum_us": us[3 * i + 1], "pair_us": us[3 * i + 2]}
        out["fold_all_release"]["bitwise_equal"] = bool(eq[0])
        out["fold_one_release"]["bitwise_equal"] = bool(eq[1])
        out["timed_out_waits"] = to.value
    elif name == "stream-sum":
        n = 1 << 26
        out = {"probe": name, "arrays": 4, "floats_each": n, "bytes": 16 * n, "reps": 10}
        for nb in (1024, 2048, 4096):
            us = (ctypes.c_double * 3)()
            rc = lib.iqlh_probe_stream_sum(ctypes.c_int64(n), ctypes.c_int(nb), ctypes.c_int(10), us)
            if rc != 0:
                raise RuntimeError(f"iqlh_probe_stream_sum returned {rc}")
            out[f"nb{nb}"] = {"strided_us": us[0], "chunked_us": us[1], "per_piece_us": us[2],
                              "strided_TBs": 16 * n / us[0] / 1e6, "chunked_TBs": 16 * n / us[1] / 1e6,
                              "per_piece_TBs": 16 * n / us[2] / 1e6}
    else:
        blocks, lds = 256, 154 * 1024
        xcc = (ctypes.c_int * blocks)()
        rc = lib.iqlh_probe_xcc_map(ctypes.c_int(blocks), ctypes.c_int(lds), xcc)
        if rc != 0:
            raise RuntimeError(f"iqlh_probe_xcc_map returned {rc}")
        got = list(xcc)
        out = {"probe": name, "blocks": blocks, "threads": 1024, "lds_bytes": lds,
               "block_i_on_xcc_i_mod_8": all(x == i % 8 for i, x in enumerate(got)),
               "blocks_per_xcc": [got.count(k) for k in range(8)], "xcc_of_first_16": got[:16]}
    print(json.dumps(out), flush=True)


PHASE_NAMES = ("S0 staging (HER relabelling, budget pass 1)", "F1", "F2 + V", "loss, dz2",
               "dW2 + W2^T + policy", "dh1, dz1", "dW1 (stores issued)")


def run_phases(steps, warmup):
    """Phase durations of the forward/backward kernel of the headline step,
    from the 100 MHz clock values each workgroup's thread 0 records at its
    phase ends (iql_aux_step_phase_stamps)."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import offline_rl_step_amd as m
    import synth
    w = synth.WORKLOADS[synth.BENCH_WORKLOAD]
    ctx = Context(m, w, torch, np, synth)
    ntile = (w.B + 127) // 128
    stamps = torch.zeros(w.groups * ntile * m.PHASE_STAMPS, dtype=torch.int64, device=ctx.d)
    for _ in range(warmup):
        ctx.step()
    runs = []
    for _ in range(steps):
        ctx.tr.aux_step_phase_stamps(ctx.her_step, ctx.X, ctx.q, w.B, ctx.Q, w.A, w.beta, ctx.pi, ctx.out_v,
                                     ctx.out_loss, ctx.out_gn, ctx.budget_step, stamps)
        torch.cuda.synchronize()
        runs.append(stamps.cpu().numpy().reshape(w.groups, ntile, m.PHASE_STAMPS).astype(np.int64))
    st = np.stack(runs)  # [steps][G][tile][8], 10 ns ticks
    her_tile = np.arange(ntile) >= (w.B - w.n_her) // 128
    dur = np.diff(st, axis=3) * 1e-2  # us
    rel_end = (st[..., -1] - st[..., 0].min(axis=(1, 2), keepdims=True)) * 1e-2
    out = {"probe": "phases", "workload": w.name, "steps": steps, "tiles": ntile, "groups": w.groups,
           "her_tiles": int(her_tile.sum()), "clock": "s_memrealtime, 100 MHz, thread 0 of each workgroup"}
    for name, sel in (("plain", ~her_tile), ("her", her_tile)):
        d = dur[:, :, sel, :].reshape(-1, m.PHASE_STAMPS - 1)
        out[name] = {"phase_us_median": {PHASE_NAMES[k]: float(np.median(d[:, k])) for k in range(len(PHASE_NAMES))},
                     "span_us_median": float(np.median(d.sum(axis=1))),
                     "end_after_first_start_us_median": float(np.median(rel_end[:, :, sel])),
                     "end_after_first_start_us_max": float(rel_end[:, :, sel].max())}
    out["kernel_event_us"] = ctx.time_launches(50)[1]
    print(json.dumps(out), flush=True)


def fused_flops_per_launch(w):
    """Algorithmic flops of one forward/backward launch over all groups:
    per sample and trainer 2SH + 2H^2 (forward GEMMs), 2H^2 + 2H^2 + 2SH
    (dh1, dW2, dW1) and 5H for the output layer, dw3 and the bias sums."""
    S, H = w.S, w.H
    return w.groups * w.B * (4 * S * H + 6 * H * H + 5 * H)


def partial_layout(w, layout=None):
    """Per-workgroup gradient partials of the forward/backward launch: `layout`
    = (rows per trainer, floats per row) as the library reports it; without
    it, the fused kernel's one row per 128-sample workgroup."""
    P = w.S * w.H + w.H + w.H * w.H + w.H + w.H + 1
    if layout is None:
        layout = ((w.B + 127) // 128, (P + 127) // 128 * 128)
    return P, layout[1], layout[0]


def budget_blocks(n):
    """Blocks of the budget's pass 1 (budget_num_blocks in budget.hip)."""
    return max(1, min(2048, ((n + 3) // 4 + 255) // 256))


def fused_parts(w):
    """Which first-launch passes the forward/backward launch hosts, by the
    rules of iql_fused_her_ok / iql_fused_norms_ok (16-wave kernel: bf16,
    hidden 128, state <= 128): HER rows that form the batch tail from a
    128-row boundary, with whole 8-float chunks and goals of at most 64
    entries; budget norms when their blocks fit four per host workgroup."""
    k16 = w.dtype == "bf16" and w.H == 128 and w.S <= 128
    n = w.n_her
    her = k16 and n > 0 and (w.B - n) % 128 == 0 and w.S % 8 == 0 and w.G <= 64
    hosts = w.groups * ((w.B - n) // 128 if her else (w.B + 127) // 128)
    norms = k16 and w.budget and budget_blocks(w.n_budget) <= 4 * hosts
    return her, norms


def launch_bytes(w, layout=None):
    """Bytes each launch of one step must read and write, given its inputs
    and outputs (what a perfect cache would leave of its traffic):
      relabel+norms: per HER row, source s and s' rows (f32), the donor's goal,
                     the source index, action, done and two episode ends;
                     written: the bf16 state row, the f32 s' row, action,
                     reward, done, donor, IS weight.  Norms: every budget source once.
                     Either part moves to fwd_bwd when that launch hosts it
                     (fused_parts); the HER rows are then not read back from
                     the batch.
      fwd_bwd:       the bf16 batch, q_taken, Q, the weight shadows and biases
                     of every trainer; written: V, the policy and the
                     per-workgroup gradient partials.
      reduce_saxpy:  the partials and loss partials, the gradient written; the
                     budget sources again, the accumulated gradient written.
      adam:          p, m, v, g read and written (g zeroed) per parameter of
                     both trainers and of the budgeted network, plus the bf16
                     weight shadows the trainers' update rewrites."""
    n, S, H, A, B, grp = w.n_her, w.S, w.H, w.A, w.B, w.groups
    k, nb = (4, w.n_budget) if w.budget else (0, 0)
    P, Pp, nwg = partial_layout(w, layout)
    e = 2 if w.dtype == "bf16" else 4
    shadows = e * (H * S + 2 * H * H)
    her = n * (8 * S + 4 * w.G + 4 + 4 + 4 + 8) + n * (e * S + 4 * S + 5 * 4)
    norms = k * nb * 4
    her_b, norms_b = fused_parts(w)
    batch_rows = B - n if her_b else B
    return {
        "relabel_norms": (0 if her_b else her) + (0 if norms_b else norms),
        "fwd_bwd": batch_rows * S * e + B * 4 + B * A * 4 + grp * (shadows + 4 * (3 * H + 1))
                   + grp * B * 4 + grp * B * A * 4 + grp * nwg * Pp * 4
                   + (her if her_b else 0) + (norms if norms_b else 0),
        "reduce_saxpy": grp * nwg * Pp * 4 + grp * nwg * 4 + grp * P * 4 + k * nb * 4 + nb * 4,
        "adam": grp * (P * 32 + shadows) + nb * 32,
    }


def mfma_from_profiles(name, src_hash):
    """MFMA busy fraction and counter flops from a committed counter summary,
    if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name}_mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != src_hash:
        return None
    return {k: d[k] for k in ("mfma_busy_frac", "mfma_flops_counter", "counter_rate_tflops", "lds_active_frac")
            if k in d}


def kernel_source_hash(extra=()):
    h = hashlib.sha256()
    for f in ("iql.hip", "common.hpp", "her_block.hpp", "budget_block.hpp", "iql_update.hpp", "launch.hpp", *extra):
        with open(os.path.join(ROOT, "offline_rl_step_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(name, src_hash):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_hash") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


class Context:
    def __init__(self, m, w, torch, np, synth):
        d = torch.device("cuda:0")
        self.m, self.w, self.d = m, w, d
        B, S, A, n = w.B, w.S, w.A, w.n_her
        self.host_buf = buf = synth.replay_buffer(w)
        self.host_src = src = synth.her_sources(w, buf)
        self.host_Xn = synth.batch_states(w)
        self.host_Q, _, self.host_q = synth.q_values(w, buf, src)
        self.inits = synth.group_inits(w)
        if w.budget:
            self.host_sources = synth.budget_sources(w)
            self.host_theta = synth.budget_params(w)

        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)  # noqa: E731
        self.rb_states, self.rb_next = t(buf["states"]), t(buf["next_states"])
        self.rb_actions, self.rb_dones = t(buf["actions"]), t(buf["dones"])
        self.rb_ends = t(buf["episode_ends"].astype(np.int32))
        self.src = t(src.astype(np.int32))
        bf16 = w.dtype == "bf16"
        xdt = torch.bfloat16 if bf16 else torch.float32
        self.X = torch.empty((B, S), dtype=xdt, device=d)
        self.X[: B - n] = t(self.host_Xn).to(xdt)
        self.Q, self.q = t(self.host_Q), t(self.host_q)
        self.her_next = torch.empty((n, S), dtype=torch.float32, device=d)
        self.her_act = torch.empty(n, dtype=torch.int32, device=d)
        self.her_rew = torch.empty(n, dtype=torch.float32, device=d)
        self.her_done = torch.empty(n, dtype=torch.float32, device=d)
        self.her_donor = torch.empty(n, dtype=torch.int32, device=d)
        self.isw = torch.ones(B, dtype=torch.float32, device=d)  # merged batch IS weights (HER tail written)

        cdt = m.BF16 if bf16 else m.F32
        cfg = m.make_config(S, w.H, B, num_groups=w.groups, compute_dtype=cdt, states_ld=S,
                            tau=w.taus, lr=w.lr, max_grad_norm=w.max_grad_norm)
        self.tr = m.IqlTrainer(cfg, np.concatenate(self.inits))
        self.out_v = torch.empty((w.groups, B), dtype=torch.float32, device=d)
        self.out_loss = torch.empty(w.groups, dtype=torch.float32, device=d)
        self.out_gn = torch.empty(w.groups, dtype=torch.float32, device=d)
        self.pi = torch.empty((w.groups, B, A), dtype=torch.float32, device=d)

        strategy = {"final": m.HER_FINAL, "future": m.HER_FUTURE, "random": m.HER_RANDOM}[w.strategy]
        self.hcfg = m.her_config(S, w.G, strategy)
        self.hbuf = m.her_buffer(self.rb_states, self.rb_next, self.rb_actions, self.rb_dones, self.rb_ends)
        tail = self.X.data_ptr() + (B - n) * S * self.X.element_size()
        self.hout = m.her_out(tail, cdt, S, self.her_rew, next_states=self.her_next,
                              actions=self.her_act, dones=self.her_done, donor_idx=self.her_donor,
                              d_flags=self.tr.flags,
                              is_weights=self.isw.data_ptr() + (B - n) * self.isw.element_size())

        self.her_step = m.her_step(self.hcfg, self.hbuf, self.src, w.n_her, 20261202, self.hout)
        self.budget_step = None
        if not w.budget:
            return
        P = w.n_budget
        self.sources = [t(s) for s in self.host_sources]
        self.theta = t(self.host_theta)
        self.theta_m = torch.zeros(P, dtype=torch.float32, device=d)
        self.theta_v = torch.zeros(P, dtype=torch.float32, device=d)
        self.theta_t = torch.zeros(1, dtype=torch.int32, device=d)
        self.grad = torch.zeros(P, dtype=torch.float32, device=d)
        self.norms = torch.zeros(len(self.sources) + 1, dtype=torch.float32, device=d)
        self.ws = torch.zeros(m.grad_budget_workspace_bytes(P, 4) // 4, dtype=torch.float32, device=d)
        self.adam = m.make_adam(self.theta, self.theta_m, self.theta_v, self.theta_t, lr=w.lr,
                                max_grad_norm=w.max_grad_norm, d_flags=self.tr.flags)

        self.budget_step = m.budget_step(self.grad, self.sources, w.budget_fractions, (1.0, 1.0, 1.0, 1.0),
                                         w.n_budget, w.max_grad_norm, self.norms, self.adam, self.ws)

    def step(self):
        """One whole step: iql_aux_step (four launches)."""
        w = self.w
        self.tr.aux_step(self.her_step, self.X, self.q, w.B, self.Q, w.A, w.beta, self.pi, self.out_v,
                         self.out_loss, self.out_gn, self.budget_step)

    def time_launches(self, reps):
        """Mean kernel time (us) of each launch of the whole step."""
        w = self.w
        return self.tr.time_aux_step(self.her_step, self.X, self.q, w.B, self.Q, w.A, w.beta, self.pi, self.out_v,
                                     self.out_loss, self.out_gn, self.budget_step, reps=reps)

    def step_separate(self):
        """The same step through the three separate entry points."""
        m, w = self.m, self.w
        m.her_relabel(self.hcfg, self.hbuf, self.src, w.n_her, 20261202, self.tr.step_counter, self.hout)
        self.tr.train_step_aw(self.X, self.q, w.B, self.Q, w.A, w.beta, self.pi, self.out_v, self.out_loss,
                              self.out_gn)
        if self.budget_step is not None:
            m.grad_budget_accumulate(self.grad, self.sources, w.budget_fractions, (1.0, 1.0, 1.0, 1.0),
                                     w.n_budget, w.max_grad_norm, self.norms, self.adam, self.ws)


LAUNCH_KERNELS = (("relabel_norms", ("step_her_norms_kernel", "her_relabel_kernel")),
                  ("fwd_bwd", ("iql_fused16w_kernel", "iql_fused_fs_kernel", "iql_fused_kernel", "big_fwd1_kernel",
                               "big_fwd2_kernel",
                               "big_wgrad_kernel", "layer_gemm_kernel", "iql_rows_kernel", "iql_wgrad_kernel",
                               "aw_policy_kernel", "aw_policy_vec_kernel")),
                  ("reduce_saxpy", ("step_reduce_saxpy_kernel",)),
                  ("adam", ("step_adam_kernel",)))


def profile_commands(workload):
    wl = "" if workload is None else f" --workload {workload}"
    sys.path.insert(0, ROOT)
    import synth
    mfma = mfma_counters(synth.WORKLOADS[workload or synth.BENCH_WORKLOAD].dtype)
    return (
        f"rocprofv3 --kernel-trace --stats -f csv -d OUT/trace -o step -- python3 $REPO/bench.py{wl} --steps 200 "
        "--no-cpu-baseline --no-next-rows",
        f"rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/FETCH_SIZE -o p -- python3 $REPO/bench.py{wl} --steps 5 "
        "--warmup 1 --no-graph --no-cpu-baseline --no-next-rows --kernel-reps 5",
        "rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/copy_FETCH_SIZE -o p -- python3 $REPO/bench.py --copy-probe 256",
        f"rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/WRITE_SIZE -o p -- python3 $REPO/bench.py{wl} --steps 5 "
        "--warmup 1 --no-graph --no-cpu-baseline --no-next-rows --kernel-reps 5",
        "rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/copy_WRITE_SIZE -o p -- python3 $REPO/bench.py --copy-probe 256",
        f"rocprofv3 --pmc {' '.join(mfma)} -f csv -d OUT/MFMA -o p -- python3 $REPO/bench.py{wl} "
        "--steps 5 --warmup 1 --no-graph --no-cpu-baseline --no-next-rows --kernel-reps 5",
        f"rocprofv3 --pmc {' '.join(LDS_COUNTERS)} -f csv -d OUT/LDS -o p -- python3 $REPO/bench.py{wl} "
        "--steps 5 --warmup 1 --no-graph --no-cpu-baseline --no-next-rows --kernel-reps 5",
        f"python3 $REPO/bench.py --summarize-profiles OUT{wl}",
    )


# matrix-core counters (one rocprofv3 pass): MFMA work of the workload's
# operand type in units of 512 flops, cycles the SIMDs' MFMA units were busy,
# MFMA instructions, GPU-active cycles
def mfma_counters(dtype):
    mops = "SQ_INSTS_VALU_MFMA_MOPS_BF16" if dtype == "bf16" else "SQ_INSTS_VALU_MFMA_MOPS_F32"
    return (mops, "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "GRBM_GUI_ACTIVE")
LDS_COUNTERS = ("SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "GRBM_GUI_ACTIVE")
MI355X_SIMDS = 256 * 4


def _counters_per_kernel(path):
    """{kernel: {counter: median over dispatches}} of a multi-counter run."""
    per = {}
    for r in _csv_rows(path):
        per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: {c: _median(v) for c, v in cs.items()} for k, cs in per.items()}


def _csv_rows(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _short(name):
    s = name[5:] if name.startswith("void ") else name
    s = s.replace("(anonymous namespace)::", "").split("(")[0]
    return s.replace("iqlh::", "")


def _median(xs):
    xs = sorted(xs)
    m = len(xs) // 2
    return xs[m] if len(xs) % 2 else 0.5 * (xs[m - 1] + xs[m])


def _counter_per_kernel(path):
    """Median counter value (KiB) per kernel over its dispatches."""
    per = {}
    for r in _csv_rows(path):
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: _median(v) for k, v in per.items()}


def summarize_profiles(d, workload=None):
    """Writes the committed summaries of one profiling session: kernel times
    from the kernel-trace stats, HBM bytes per dispatch from FETCH_SIZE and
    WRITE_SIZE scaled by what the same counters read for a plain copy of
    known size, and each launch's rate on the bytes it needs."""
    import glob
    import subprocess
    sys.path.insert(0, ROOT)
    import synth
    w = synth.WORKLOADS[workload or synth.BENCH_WORKLOAD]
    default = w.name == synth.BENCH_WORKLOAD
    stats = _csv_rows(glob.glob(os.path.join(d, "trace", "*_kernel_stats.csv"))[0])
    bench_line = None
    log = os.path.join(d, "trace.log")
    if os.path.exists(log):
        for line in open(log):
            if line.startswith("{"):
                bench_line = json.loads(line)
    layout = None
    if bench_line and "partials" in bench_line:
        layout = (bench_line["partials"]["rows"], bench_line["partials"]["floats"])
    cnt = {c: _counter_per_kernel(glob.glob(os.path.join(d, c, "*_counter_collection.csv"))[0])
           for c in ("FETCH_SIZE", "WRITE_SIZE", "copy_FETCH_SIZE", "copy_WRITE_SIZE")}
    factors, cf = {}, {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cf[c] = max(v for k, v in cnt["copy_" + c].items() if "copyBuffer" in k)
        factors[c] = (256 * 1024) / cf[c]
    abytes = launch_bytes(w, layout)
    try:
        commit = subprocess.run(["git", "-C", ROOT, "rev-parse", "--short", "HEAD"], capture_output=True,
                                text=True, check=True).stdout.strip()
    except Exception:  # pragma: no cover
        commit = "unknown"
    # the wide-hidden kernels' source counts for the other workloads' summaries
    src_hash = kernel_source_hash(() if default else ("iql_big.hip", "iql_layered.hip", "aw.hip"))
    launch_of = {}
    for launch, keys in LAUNCH_KERNELS:
        for r in stats:
            if any(k in r["Name"] for k in keys):
                launch_of[r["Name"]] = launch
    steps = max((int(r["Calls"]) for r in stats if "step_reduce_saxpy_kernel" in r["Name"]), default=1)

    L = []
    what = f"budget over {w.n_budget} parameters" if w.budget else "no budget part"
    L.append(f"# Kernel time and HBM traffic of one whole step, batch {w.B}, state {w.S}, hidden {w.H}, "
             f"{w.groups} trainer{'s' if w.groups > 1 else ''}, {what}")
    L.append("")
    her_b, norms_b = fused_parts(w)
    nl = 3 if (her_b or w.n_her == 0) and (norms_b or not w.budget) else 4
    L.append(f"Workload `{w.name}`.  One `iql_aux_step` per step ({nl} launches"
             + ("; the forward/backward launch also relabels the HER rows" if her_b else "")
             + ("; it also runs the budget norms" if norms_b else "")
             + f"), eager launches on one stream, one MI355X.  Source of commit {commit} (forward/backward source hash {src_hash}).")
    L.append("")
    L.append("Commands (from /tmp, each its own run, `REPO` = the repository root, `OUT` = an output folder):")
    L.append("")
    for c in profile_commands(None if default else w.name):
        L.append("    " + c)
    L.append("")
    if bench_line:
        L.append(f"bench line of the trace run: {bench_line['ms_per_step'] * 1e3:.1f} us per step, "
                 f"{bench_line['value']:.4g} samples/s (profiler attached).")
        L.append("")
    L.append("## Kernel time (`--kernel-trace --stats`)")
    L.append("")
    L.append("| kernel | launch | calls | average us | min us | % of GPU time |")
    L.append("|---|---|---:|---:|---:|---:|")
    for r in stats:
        L.append(f"| `{_short(r['Name'])}` | {launch_of.get(r['Name'], '-')} | {r['Calls']} | "
                 f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    L.append("")
    L.append("## HBM traffic per dispatch (median over the dispatches of the counter runs)")
    L.append("")
    L.append(f"Calibration: a plain 256 MiB device copy (`__amd_rocclr_copyBuffer`) reads FETCH_SIZE = "
             f"{cf['FETCH_SIZE']:.0f} KiB and WRITE_SIZE = {cf['WRITE_SIZE']:.0f} KiB for 262144 KiB moved each "
             f"way: factors {factors['FETCH_SIZE']:.3f} (fetch) and {factors['WRITE_SIZE']:.3f} (write).")
    L.append("")
    L.append("| kernel | launch | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB | write MB |")
    L.append("|---|---|---:|---:|---:|---:|")
    per_launch = {}
    fwd_kernels = []
    for nm, fk in cnt["FETCH_SIZE"].items():
        launch = next((ln for ln, keys in LAUNCH_KERNELS if any(k in nm for k in keys)), None)
        if launch is None:
            continue
        wk = cnt["WRITE_SIZE"].get(nm, float("nan"))
        rd, wr = fk * 1024 * factors["FETCH_SIZE"], wk * 1024 * factors["WRITE_SIZE"]
        L.append(f"| `{_short(nm)}` | {launch} | {fk:.0f} | {wk:.0f} | {rd / 1e6:.2f} | {wr / 1e6:.2f} |")
        per_launch.setdefault(launch, 0.0)
        per_launch[launch] += rd + wr
        if launch == "fwd_bwd":
            fwd_kernels.append((_short(nm), fk, wk))
    L.append("")
    L.append("## Per launch")
    L.append("")
    L.append("| launch | kernel us per step | measured MB | needed MB | GB/s on needed bytes | % of 8 TB/s |")
    L.append("|---|---:|---:|---:|---:|---:|")
    for launch, _ in LAUNCH_KERNELS:
        us = sum(float(r["AverageNs"]) / 1e3 * int(r["Calls"]) / steps for r in stats
                 if launch_of.get(r["Name"]) == launch)
        if us <= 0:
            continue
        gbs = abytes[launch] / (us * 1e-6) / 1e9
        L.append(f"| {launch} | {us:.2f} | {per_launch.get(launch, float('nan')) / 1e6:.2f} | "
                 f"{abytes[launch] / 1e6:.2f} | {gbs:.0f} | {100 * gbs / PEAK_HBM_GBS:.1f} |")
    L.append("")
    P, Pp, nwg = partial_layout(w, layout)
    mfma_json = None
    gm = glob.glob(os.path.join(d, "MFMA", "*_counter_collection.csv"))
    gl = glob.glob(os.path.join(d, "LDS", "*_counter_collection.csv"))
    if gm:
        mc = _counters_per_kernel(gm[0])
        lc = _counters_per_kernel(gl[0]) if gl else {}
        L.append("## Matrix cores and LDS (`--pmc`, median over dispatches)")
        L.append("")
        mops = mfma_counters(w.dtype)[0]
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        L.append(f"`MFMA flops` = {mops} x 512; `MFMA busy` = SQ_VALU_MFMA_BUSY_CYCLES "
                 f"(summed over the SIMDs) / ({MI355X_SIMDS} SIMDs x the kernel's average time above x 2.4 GHz); "
                 "`rate` = MFMA flops / that time; LDS `active` = SQ_LDS_IDX_ACTIVE (summed over the CUs) / "
                 "(256 CUs x the same cycles), `conflict` = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE.  "
                 "(GRBM_GUI_ACTIVE, summed over the XCDs, spans the profiler's serialised dispatch window rather "
                 "than the kernel, so the kernel-trace time is the denominator.)")
        L.append("")
        L.append(f"| kernel | MFMA flops | / algorithmic | MFMA busy | rate TFLOP/s | % of {w.dtype} peak | LDS instrs | "
                 "LDS active | LDS conflict |")
        L.append("|---|---:|---:|---:|---:|---:|---:|---:|---:|")
        alg = fused_flops_per_launch(w)
        for nm, cs in mc.items():
            fl = cs.get(mops, 0.0) * 512
            if fl <= 0:
                continue
            t_us = next((float(r["AverageNs"]) / 1e3 for r in stats if r["Name"] == nm), float("nan"))
            cycles = t_us * 1e-6 * 2.4e9
            busy = cs.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cycles * MI355X_SIMDS)
            rate = fl / (t_us * 1e-6) / 1e12
            ls = lc.get(nm, {})
            lact = ls.get("SQ_LDS_IDX_ACTIVE", float("nan")) / (cycles * 256)
            lcon = ls.get("SQ_LDS_BANK_CONFLICT", float("nan")) / ls.get("SQ_LDS_IDX_ACTIVE", float("nan"))
            fused = launch_of.get(nm) == "fwd_bwd" and len([1 for n2 in mc if launch_of.get(n2) == "fwd_bwd"]) == 1
            ratio = f"{fl / alg:.3f}" if fused else "-"
            L.append(f"| `{_short(nm)}` | {fl:.4g} | {ratio} | {100 * busy:.1f} % | {rate:.0f} | "
                     f"{100 * rate / peak:.1f} | {ls.get('SQ_INSTS_LDS', float('nan')):.4g} | "
                     f"{100 * lact:.1f} % | {100 * lcon:.2f} % |")
            if fused and default:
                mfma_json = {"kernel": _short(nm), "workload": w.name, "source_hash": src_hash, "commit": commit,
                             "mfma_flops_counter": fl, "algorithmic_flops": alg, "mfma_busy_frac": busy,
                             "counter_rate_tflops": rate, "avg_kernel_us": t_us,
                             "lds_active_frac": lact, "lds_conflict_frac": lcon}
        L.append("")
        single = len([1 for n2 in mc if launch_of.get(n2) == "fwd_bwd"]) == 1
        if mfma_json is not None:
            L.append("The forward/backward kernel's MFMA flops exceed the algorithmic count by its bias-gradient "
                     "products (an extra MFMA against an all-ones operand per weight-gradient sweep) and the zero "
                     "padding of tiles.")
        elif single and any("fused_fs" in n2 for n2 in mc) and 2 * -(-w.B // 32) * w.groups <= 256:
            L.append("The forward/backward kernel's MFMA flops exceed the algorithmic count by the zero padding "
                     "of its tiles (the state padded to the operand width) and by the forward pass, which both "
                     "workgroups of a 32-sample tile run while the tiles alone would leave compute units idle "
                     "(each then forms half of the tile's weight gradients).")
        elif single:
            L.append("The forward/backward kernel's MFMA flops differ from the algorithmic count by the zero "
                     "padding of its tiles (the state padded to the operand width).")
        else:
            L.append("Several kernels share the forward/backward launch here, so no single kernel's MFMA flops "
                     "are set against the algorithmic count; the rate column is each kernel's own.")
        L.append("")
    L.append(f"`needed MB` is each launch's inputs and outputs read or written once (`launch_bytes` in "
             f"bench.py).  For the forward/backward launch it includes its fp32 gradient partials "
             f"({w.groups} x {nwg} rows x {Pp} floats = {w.groups * nwg * Pp * 4 / 1e6:.1f} MB), which the "
             f"reduction reads back"
             + (", and the HER rows' replay reads and outputs" if her_b else "") + ".")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    md = os.path.join(ROOT, "profiles", f"step_{w.name}_kernels.md")
    with open(md, "w") as fh:
        fh.write("\n".join(L) + "\n")
    if default and len(fwd_kernels) == 1:
        nm, fk, wk = fwd_kernels[0]
        traffic = {"kernel": nm, "workload": w.name, "source_hash": src_hash,
                   "hbm_bytes_per_launch": fk * 1024 * factors["FETCH_SIZE"] + wk * 1024 * factors["WRITE_SIZE"],
                   "fetch_kib_raw": fk, "write_kib_raw": wk, "fetch_factor": factors["FETCH_SIZE"],
                   "write_factor": factors["WRITE_SIZE"], "commit": commit}
        with open(os.path.join(ROOT, "profiles", "iql_fused_b16384_s128_h128_g2_traffic.json"), "w") as fh:
            json.dump(traffic, fh, indent=1)
            fh.write("\n")
    if mfma_json:
        with open(os.path.join(ROOT, "profiles", "iql_fused_b16384_s128_h128_g2_mfma.json"), "w") as fh:
            json.dump(mfma_json, fh, indent=1)
            fh.write("\n")
    print(md)


def time_next_rows(ctx, torch, np, reps=100):
    """Mean GPU time per call (inside a captured graph) of the widening entry
    points on the bench workload, each with its roofline: V(s') + bootstrap target (MFMA flops of the two
    forward products), the Polyak target update and the non-finite sentinel
    (bytes each must move), prioritized sampling of the HER sources over the
    whole replay buffer (bytes: the priorities once and the draws' indices and
    weights; the prefix sums are never stored, and each draw's block table,
    sub-block sums and 1 KB of rows come from the caches)."""
    m, w, d = ctx.m, ctx.w, ctx.d
    B, S, H, G = w.B, w.S, w.H, w.groups

    def timed(fn, calls=50):
        # `calls` back-to-back calls captured in one graph, replayed: GPU time
        # per call, not the rate at which Python can issue them
        fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(calls):
                fn()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        stream = torch.cuda.current_stream()
        e0.record(stream)
        for _ in range(max(1, reps // 10)):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (max(1, reps // 10) * calls)

    out = {}
    g = np.random.default_rng(5)
    nxt = torch.from_numpy(g.standard_normal((B, S)).astype(np.float32)).to(d).to(torch.bfloat16)
    rew = torch.zeros(B, dtype=torch.float32, device=d)
    don = torch.zeros(B, dtype=torch.float32, device=d)
    vn = torch.zeros((G, B), dtype=torch.float32, device=d)
    tg = torch.zeros_like(vn)
    us = timed(lambda: ctx.tr.forward_values(nxt, B, vn, rewards=rew, dones=don, gamma=0.99, out_target=tg))
    fl = 2.0 * B * G * (S * H + H * H + H)
    out["forward_values_target"] = {"us": us, "flops": fl, "achieved": fl / (us * 1e-6) / 1e12, "unit": "TFLOP/s",
                                    "peak": PEAK_BF16_TFLOPS, "frac": fl / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS}
    P = w.n_params
    us = timed(lambda: ctx.tr.target_ema_update(0.005))
    by = 12.0 * G * P
    out["target_ema"] = {"us": us, "bytes": by, "achieved": by / (us * 1e-6) / 1e9, "unit": "GB/s",
                         "peak": PEAK_HBM_GBS, "frac": by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    bufs = [ctx.Q, ctx.q, ctx.out_v, ctx.pi, ctx.her_next, ctx.her_rew]
    if w.budget:
        bufs += [ctx.theta, ctx.theta_m, ctx.theta_v]
    flags = torch.zeros(len(bufs), dtype=torch.int32, device=d)
    us = timed(lambda: m.nonfinite_check(bufs, flags))
    by = 4.0 * sum(b.numel() for b in bufs)
    out["nonfinite_check"] = {"us": us, "bytes": by, "slots": len(bufs), "achieved": by / (us * 1e-6) / 1e9,
                              "unit": "GB/s", "peak": PEAK_HBM_GBS, "frac": by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    C = w.C
    pr = torch.from_numpy(g.random(C).astype(np.float32)).to(d)
    ws = torch.zeros((m.per_workspace_bytes(C) + 7) // 8, dtype=torch.float64, device=d)
    idx = torch.zeros(w.n_her, dtype=torch.int32, device=d)
    wt = torch.zeros(w.n_her, dtype=torch.float32, device=d)
    us = timed(lambda: m.per_sample_indices(pr, w.n_her, 1, 0.4, idx, wt, ws))
    by = 4.0 * C + 8.0 * w.n_her
    out["per_sample_indices"] = {"us": us, "bytes": by, "replay_rows": C, "draws": w.n_her,
                                 "achieved": by / (us * 1e-6) / 1e9, "unit": "GB/s", "peak": PEAK_HBM_GBS,
                                 "frac": by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
    return out


# ------------------------------------------------------------ HBM sweeps
SWEEP_POINTS = {
    "her": [1 << 16, 1 << 18, 1 << 20],      # relabelled rows
    "aw": [1 << 20, 1 << 22, 1 << 24],       # rows B at A = 16, two trainers (B * A up to 2^26)
    "budget": [1 << 22, 1 << 24, 1 << 26],   # elements n, four sources
    "sentinel": [1 << 23, 1 << 25, 1 << 27], # elements per slot, eight slots
    "copy": [1 << 26, 1 << 28],              # a plain device copy of n floats (torch), for reference
}
SWEEP_KERNELS = {"her": ("her_relabel_kernel",), "aw": ("aw_policy",),
                 "budget": ("budget_norms_kernel", "budget_saxpy_kernel", "adam_flat_kernel"),
                 "sentinel": ("nonfinite_sentinel_kernel",), "copy": ("copy",)}
# bytes per element each pass of a multi-kernel sweep must move: the budget's
# pass 1 reads the four sources, pass 2 reads them again and writes grad,
# Adam reads and writes p, m, v and grad
SWEEP_PASS_BYTES = {"budget": (("budget_norms_kernel", "pass 1: per-source sums of squares", 16),
                               ("budget_saxpy_kernel", "pass 2: clip + SAXPY", 20),
                               ("adam_flat_kernel", "pass 3: clipped Adam", 32))}


def sweep_bytes(kind, x):
    """Bytes one call must move (each input read once, each output written
    once; what no cache can save at these sizes):
      her:    per row the source's s and s' (f32), the donor's goal, the
              source index, action, done and two episode ends; written the
              bf16 state row, the f32 s' row, action, reward, done, donor and
              importance weight (state 128, goal 8);
      aw:     Q [B, 16] once, V [2, B], the policy [2, B, 16] written;
      budget: pass 1 reads the four sources; pass 2 reads them again (the
              clip needs every norm first) and writes grad; Adam reads grad,
              p, m, v and writes p, m, v and the zeroed grad: 68 B/element;
      sentinel: eight slots of x floats, read once."""
    if kind == "her":
        S, G = 128, 8
        return x * ((8 * S + 4 * G + 4 + 4 + 4 + 8) + (2 * S + 4 * S + 5 * 4))
    if kind == "aw":
        A, G = 16, 2
        return x * (4 * A + G * (4 + 4 * A))
    if kind == "copy":
        return x * 8
    if kind == "sentinel":
        return x * 8 * 4
    return x * 68


def run_sweep(kind, calls):
    """Times each size of one HBM-bound entry point with HIP events around
    `calls` back-to-back calls (after one warm-up call); one JSON line each."""
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import offline_rl_step_amd as m
    d = torch.device("cuda:0")
    gen = torch.Generator(device=d)
    gen.manual_seed(20261202)
    stream = torch.cuda.current_stream()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(calls):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / calls

    rows = []
    if kind == "her":
        C, S, G, L = 1 << 22, 128, 8, 64
        st = torch.randn((C, S), generator=gen, device=d)
        nx = torch.randn((C, S), generator=gen, device=d)
        act = torch.randint(0, 9, (C,), generator=gen, device=d, dtype=torch.int32)
        done = torch.zeros(C, device=d)
        ends = torch.arange(1, C // L + 1, device=d, dtype=torch.int32) * L
        done[ends.long() - 1] = 1.0
        buf = m.her_buffer(st, nx, act, done, ends)
        cfg = m.her_config(S, G, m.HER_FUTURE)
        step = torch.zeros(1, dtype=torch.int64, device=d)
        for n in SWEEP_POINTS[kind]:
            src = torch.randint(0, C, (n,), generator=gen, device=d, dtype=torch.int32)
            X = torch.empty((n, S), dtype=torch.bfloat16, device=d)
            o_next = torch.empty((n, S), device=d)
            o_i = [torch.empty(n, dtype=torch.int32, device=d) for _ in range(2)]
            o_f = [torch.empty(n, device=d) for _ in range(3)]
            out = m.her_out(X, m.BF16, S, o_f[0], next_states=o_next, actions=o_i[0], dones=o_f[1],
                            donor_idx=o_i[1], is_weights=o_f[2])
            us = timed(lambda: m.her_relabel(cfg, buf, src, n, 7, step, out))
            rows.append((n, us, f"{n} rows over a {C}-row replay buffer ({2 * C * S * 4 / 2**30:.0f} GiB)"))
    elif kind == "aw":
        A, G = 16, 2
        for B in SWEEP_POINTS[kind]:
            q = torch.randn((B, A), generator=gen, device=d)
            v = torch.randn((G, B), generator=gen, device=d)
            pi = torch.empty((G, B, A), device=d)
            us = timed(lambda: m.iql_aw_policy(q, v, G, B, A, 3.0, pi))
            rows.append((B, us, f"B = {B}, A = {A}, {G} trainers (B A = 2^{int(np.log2(B * A))})"))
    elif kind == "sentinel":
        flags = torch.zeros(8, dtype=torch.int32, device=d)
        for n in SWEEP_POINTS[kind]:
            bufs = [torch.randn(n, generator=gen, device=d) for _ in range(8)]
            us = timed(lambda: m.nonfinite_check(bufs, flags))
            rows.append((n, us, f"eight slots of {n} floats ({8 * n * 4 / 2**30:.2f} GiB), all finite"))
            del bufs
            torch.cuda.empty_cache()
    elif kind == "copy":
        for n in SWEEP_POINTS[kind]:
            a_, b_ = torch.randn(n, generator=gen, device=d), torch.empty(n, device=d)
            us = timed(lambda: b_.copy_(a_))
            rows.append((n, us, f"device copy of {n * 4 / 2**20:.0f} MiB (reference)"))
            del a_, b_
    else:
        for n in SWEEP_POINTS[kind]:
            srcs = [torch.randn(n, generator=gen, device=d) * sc for sc in (1.0, 5.0, 0.5, 0.2)]
            grad = torch.zeros(n, device=d)
            p = torch.randn(n, generator=gen, device=d) * 0.05
            mm, vv = torch.zeros(n, device=d), torch.zeros(n, device=d)
            t = torch.zeros(1, dtype=torch.int32, device=d)
            norms = torch.zeros(5, device=d)
            ws = torch.zeros(m.grad_budget_workspace_bytes(n, 4) // 4, device=d)
            adam = m.make_adam(p, mm, vv, t)
            us = timed(lambda: m.grad_budget_accumulate(grad, srcs, (0.7, 0.15, 0.1, 0.05), (1.0,) * 4, n, 1.0,
                                                        norms, adam, ws))
            rows.append((n, us, f"n = {n} (2^{int(np.log2(n))}), four sources + Adam"))
            del srcs, grad, p, mm, vv, ws
            torch.cuda.empty_cache()
    for x, us, what in rows:
        by = sweep_bytes(kind, x)
        print(json.dumps({"sweep": kind, "size": x, "what": what, "us_per_call": us, "bytes_per_call": by,
                          "GB/s": by / (us * 1e-6) / 1e9, "frac_of_8TBs": by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                          "calls": calls}), flush=True)


def sweep_commands():
    return [f"rocprofv3 --kernel-trace --stats -f csv -d OUT/sweep_{k}_trace -o t -- python3 $REPO/bench.py "
            f"--sweep {k} > OUT/sweep_{k}.json" for k in SWEEP_POINTS] + \
           [f"rocprofv3 --pmc {c} -f csv -d OUT/sweep_{k}_{c} -o p -- python3 $REPO/bench.py --sweep {k}"
            for k in SWEEP_POINTS for c in ("FETCH_SIZE", "WRITE_SIZE")] + \
           [f"rocprofv3 --pmc {c} -f csv -d OUT/copy_{c} -o p -- python3 $REPO/bench.py --copy-probe 256"
            for c in ("FETCH_SIZE", "WRITE_SIZE")] + \
           ["python3 $REPO/bench.py --summarize-sweeps OUT"]


def _counter_dispatches(path):
    """Counter value (KiB) of every dispatch, in dispatch order, per kernel."""
    per = {}
    rows = sorted(_csv_rows(path), key=lambda r: int(r.get("Dispatch_Id", 0)))
    for r in rows:
        per.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return per


def summarize_sweeps(d):
    """profiles/hbm_sweeps.md: per sweep size, the event-timed rate on the
    bytes the call must move, and the HBM bytes the counters saw (FETCH_SIZE /
    WRITE_SIZE summed over the call's kernels, median over the timed calls,
    scaled by the plain-copy calibration)."""
    import glob
    cf = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        per = _counter_dispatches(glob.glob(os.path.join(d, "copy_" + c, "*_counter_collection.csv"))[0])
        cf[c] = (256 * 1024) / max(v for k, vs in per.items() if "copyBuffer" in k for v in vs)
    L = ["# HBM-bound entry points on working sets of at least 1 GiB", "",
         "Each size is timed with HIP events around back-to-back calls after one warm-up call (`bench.py --sweep`), "
         "in its own process per sweep; MI355X HBM3E peak 8 TB/s.  `needed` = the bytes the call must move "
         "(`sweep_bytes` in bench.py).  `measured` = FETCH_SIZE + WRITE_SIZE of the call's kernels (median over "
         f"the calls of the counter runs), scaled by a plain 256 MiB copy's counters (factors "
         f"{cf['FETCH_SIZE']:.3f} fetch, {cf['WRITE_SIZE']:.3f} write).", "",
         "Commands (from /tmp, each its own run, `REPO` = the repository root, `OUT` = an output folder):", ""]
    L += ["    " + c for c in sweep_commands()]
    L += ["", "| entry point | size | us per call | needed GB | measured read GB | measured write GB | "
              "TB/s on needed bytes | % of 8 TB/s |", "|---|---|---:|---:|---:|---:|---:|---:|"]
    for kind in SWEEP_POINTS:
        jpath = os.path.join(d, f"sweep_{kind}.json")
        if not os.path.exists(jpath):
            continue
        pts = [json.loads(x) for x in open(jpath) if x.startswith("{")]
        meas = {}
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            g = glob.glob(os.path.join(d, f"sweep_{kind}_{c}", "*_counter_collection.csv"))
            if not g:
                continue
            per = _counter_dispatches(g[0])
            calls = pts[0]["calls"] + 1 if pts else 1
            tot = []
            for i in range(len(pts)):
                per_call = []
                for j in range(1, calls):  # skip the warm-up call
                    v = 0.0
                    for kn in SWEEP_KERNELS[kind]:
                        vs = [x for k, x in per.items() if kn in k]
                        vs = vs[0] if vs else []
                        if len(vs) >= calls * len(pts):
                            v += vs[i * calls + j]
                    per_call.append(v)
                tot.append(_median(per_call) * 1024 * cf[c])
            meas[c] = tot
        names = {"her": "her_relabel", "aw": "iql_aw_policy", "budget": "grad_budget_accumulate + Adam",
                 "sentinel": "iqlh_nonfinite_check", "copy": "plain copy (torch)"}
        for i, p in enumerate(pts):
            rd = meas.get("FETCH_SIZE", [float("nan")] * len(pts))[i]
            wr = meas.get("WRITE_SIZE", [float("nan")] * len(pts))[i]
            L.append(f"| {names[kind]} | {p['what']} | {p['us_per_call']:.1f} | {p['bytes_per_call'] / 1e9:.3f} | "
                     f"{rd / 1e9:.3f} | {wr / 1e9:.3f} | {p['GB/s'] / 1e3:.2f} | {100 * p['frac_of_8TBs']:.1f} |")
    # the passes of a multi-kernel entry point on their own: kernel-trace
    # durations per dispatch (median over the timed calls of each size)
    for kind, passes in SWEEP_PASS_BYTES.items():
        jpath = os.path.join(d, f"sweep_{kind}.json")
        g = glob.glob(os.path.join(d, f"sweep_{kind}_trace", "*_kernel_trace.csv"))
        if not os.path.exists(jpath) or not g:
            continue
        pts = [json.loads(x) for x in open(jpath) if x.startswith("{")]
        calls = pts[0]["calls"] + 1 if pts else 1
        rows = sorted(_csv_rows(g[0]), key=lambda r: int(r["Dispatch_Id"]))
        L += ["", f"Passes of {names[kind]} on their own (kernel trace of the timing run; bytes per element: "
              + ", ".join(f"{b} for {k}" for k, _, b in passes) + "):", "",
              "| pass | size | us per call | needed GB | TB/s on needed bytes | % of 8 TB/s |",
              "|---|---|---:|---:|---:|---:|"]
        for kn, what, bpe in passes:
            durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows if kn in r["Kernel_Name"]]
            if len(durs) < calls * len(pts):
                continue
            for i, p in enumerate(pts):
                us = _median(durs[i * calls + 1:(i + 1) * calls])
                by = bpe * p["size"]
                L.append(f"| {what} | {p['what']} | {us:.1f} | {by / 1e9:.3f} | {by / (us * 1e-6) / 1e12:.2f} | "
                         f"{100 * by / (us * 1e-6) / 1e9 / PEAK_HBM_GBS:.1f} |")
    md = os.path.join(ROOT, "profiles", "hbm_sweeps.md")
    os.makedirs(os.path.dirname(md), exist_ok=True)
    with open(md, "w") as fh:
        fh.write("\n".join(L) + "\n")
    print(md)


def cpu_baseline(ctx, seconds, np):
    """The oracle as it stands, one full step at a time, on the host cores."""
    from oracle import aw, budget, her, iql
    w = ctx.w
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        cores = max(blas) if blas else 1
    except Exception:  # pragma: no cover
        cores = 1
    Xn = ctx.host_Xn.astype(np.float64)
    states = [iql.AdamState.fresh(p) for p in ctx.inits]
    theta = iql.AdamState.fresh(ctx.host_theta) if w.budget else None
    strategy = {"final": her.FINAL, "future": her.FUTURE, "random": her.RANDOM}[w.strategy]
    hp = iql.AdamHP(lr=w.lr, max_grad_norm=w.max_grad_norm)
    t0 = time.perf_counter()
    steps = 0
    while True:
        r = her.her_step(ctx.host_buf, ctx.host_src, w.G, strategy, 20261202, steps, out_bf16=w.dtype == "bf16")
        X = np.concatenate([Xn, r["states"].astype(np.float64)])
        vs = [iql.train_step(states[g], X, ctx.host_q, w.S, w.H, w.H, w.taus[g], hp).v for g in range(w.groups)]
        for g in range(w.groups):
            aw.aw_policy(ctx.host_Q, vs[g], w.beta)
        if w.budget:
            grad, _, _, _ = budget.accumulate(ctx.host_sources, w.budget_fractions, (1, 1, 1, 1),
                                              w.max_grad_norm)
            iql.adam_step(theta, grad, hp)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), model)
    except OSError:  # pragma: no cover
        pass
    return {"value": w.B * steps / el, "unit": "samples/s", "cores": int(cores), "cpu_model": model,
            "kind": "oracle",
            "sample": f"{steps} full steps of the same workload (fp64 NumPy oracle; BLAS threads = cores), "
                      f"{el:.1f} s", "s_per_step": el / steps, "host_cpus": os.cpu_count()}


def main():
    a = parse()
    if a.summarize_sweeps:
        summarize_sweeps(a.summarize_sweeps)
        return
    if a.sweep:
        run_sweep(a.sweep, a.sweep_calls)
        return
    if a.summarize_profiles:
        summarize_profiles(a.summarize_profiles, a.workload)
        return
    if a.copy_probe:
        copy_probe(a.copy_probe)
        return
    if a.probe:
        run_probe(a.probe)
        return
    if a.phases:
        run_phases(min(a.steps, 200), a.warmup)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU: the step has no cross-GPU exchange, so --gpus {a.gpus} "
              "is not supported.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import offline_rl_step_amd as m
    import synth

    default = a.workload is None or a.workload == synth.BENCH_WORKLOAD
    w = synth.WORKLOADS[a.workload or synth.BENCH_WORKLOAD]
    ctx = Context(m, w, torch, np, synth)
    torch.cuda.synchronize()

    step = ctx.step_separate if a.separate else ctx.step
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if a.graph and not a.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()

    run = graph.replay if graph is not None else step
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(a.steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1)
    rc, flags = ctx.tr.status()
    ms_per_step = wall * 1e3 / a.steps

    # the other launch mode, for comparison: graph replay (one step per
    # replay) when the timed run was eager, and the reverse
    if graph is None:
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2):
            step()
        other = g2.replay
    else:
        g2, other = None, step
    for _ in range(3):
        other()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(a.steps):
        other()
    torch.cuda.synchronize()
    other_us = (time.perf_counter() - t1) * 1e6 / a.steps
    del g2

    # every launch of the step timed by its own dispatch events, on the
    # stream the step runs on; the dominant one is the forward/backward
    launch_us = ctx.time_launches(a.kernel_reps)
    names = [k for k, _ in LAUNCH_KERNELS]
    layout = ctx.tr.partial_layout(w.B)
    lb = launch_bytes(w, layout)
    avg_us = launch_us[1]
    flops = fused_flops_per_launch(w)
    achieved = flops / (avg_us * 1e-6) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    src_hash = kernel_source_hash()
    if default:
        kernel = "iql_fused16w_kernel<128,128,xvec>"
    elif w.H in (256, 512) and w.dtype == "bf16" and w.S % 32 == 0:
        kernel = "wide forward/backward (big_fwd2, big_wgrad and the policy; events around the launch)"
    elif w.H > 128:
        kernel = "layered forward/backward (events around the group)"
    else:
        kernel = "fused forward/backward"
    # the roof that bounds this launch: its algorithmic flops over the bytes
    # it must move (inputs and outputs once, without the split-K partials)
    # against the ridge point peak flops / peak bandwidth
    P_, Pp_, nwg_ = partial_layout(w, layout)
    alg_bytes = lb["fwd_bwd"] - w.groups * nwg_ * Pp_ * 4
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    intensity = flops / alg_bytes
    mfma_frac = achieved / peak
    bytes_rate = alg_bytes / (avg_us * 1e-6) / 1e9
    counters = mfma_from_profiles("iql_fused_b16384_s128_h128_g2", src_hash) if default else None
    if intensity < ridge:
        roofline = {"bound": "hbm", "kernel": kernel, "achieved": bytes_rate, "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": bytes_rate / PEAK_HBM_GBS}
    else:
        roofline = {"bound": "mfma", "kernel": kernel, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                    "frac": mfma_frac}
    roofline.update({
        "traffic": traffic_from_profiles("iql_fused_b16384_s128_h128_g2", src_hash) if default else None,
        "avg_kernel_us": avg_us, "flops_per_launch": flops, "algorithmic_bytes_per_launch": alg_bytes,
        "intensity_flop_per_byte": intensity, "ridge_flop_per_byte": ridge,
        "mfma_tflops": achieved, "mfma_frac": mfma_frac, "hbm_GBs_on_algorithmic_bytes": bytes_rate,
        "hbm_frac": bytes_rate / PEAK_HBM_GBS, "mfma_counters": counters, "source_hash": src_hash})

    out = {"metric": METRIC, "value": w.B / (ms_per_step * 1e-3), "unit": "samples/s", "n_gpus": 1,
           "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
           "config": {"workload": w.name, "global_batch": w.B, "state_dim": w.S, "hidden": w.H,
                      "actions": w.A, "groups": w.groups, "her_rows": w.n_her, "her_strategy": w.strategy,
                      "replay_rows": w.C, "budget_params": w.n_budget if w.budget else 0,
                      "budget_sources": 4 if w.budget else 0,
                      "graph_replay": graph is not None,
                      "entry_point": "separate calls" if a.separate else "iql_aux_step",
                      "parallelism": "single-gpu"},
           "event_ms_per_step": ev_ms / a.steps, "device_flags": flags, "status": rc,
           ("graph_replay_us_per_step" if graph is None else "eager_us_per_step"): other_us,
           "partials": {"rows": layout[0], "floats": layout[1]},
           "launch_us": dict(zip(names, launch_us)),
           "launch_hbm": {k: {"needed_bytes": lb[k], "GB/s": lb[k] / (us * 1e-6) / 1e9,
                              "frac_of_8TBs": lb[k] / (us * 1e-6) / 1e9 / PEAK_HBM_GBS}
                          for k, us in zip(names, launch_us) if us > 0.0},
           "roofline": roofline}
    if not a.no_next_rows:
        out["next_rows"] = time_next_rows(ctx, torch, np)
    if (default or a.cpu_baseline) and not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(ctx, a.cpu_seconds, np)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
