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
in four launches (HER + budget norms | forward/backward + policy | reduction
+ SAXPY | both Adam updates).  --separate times her_relabel +
iql_train_step_aw + grad_budget_accumulate called one after the other
instead (same results bit for bit, seven launches).  The step is captured
once in a HIP graph and replayed (the HER donor counter lives on the device,
so every replay draws new donors).

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
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1000)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-graph", action="store_true", help="eager launches instead of graph replay")
    p.add_argument("--separate", action="store_true",
                   help="the three entry points one after the other instead of iql_aux_step")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--kernel-reps", type=int, default=200)
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run 10 plain device copies of MIB MiB (counter calibration) and exit")
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


def fused_flops_per_launch(w):
    """Algorithmic flops of one forward/backward launch over all groups:
    per sample and trainer 2SH + 2H^2 (forward GEMMs), 2H^2 + 2H^2 + 2SH
    (dh1, dW2, dW1) and 5H for the output layer, dw3 and the bias sums."""
    S, H = w.S, w.H
    return w.groups * w.B * (4 * S * H + 6 * H * H + 5 * H)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in ("iql.hip", "common.hpp", "her_block.hpp", "iql_update.hpp", "launch.hpp"):
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
        self.host_sources = synth.budget_sources(w)
        self.host_theta = synth.budget_params(w)

        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)  # noqa: E731
        self.rb_states, self.rb_next = t(buf["states"]), t(buf["next_states"])
        self.rb_actions, self.rb_dones = t(buf["actions"]), t(buf["dones"])
        self.rb_ends = t(buf["episode_ends"].astype(np.int32))
        self.src = t(src.astype(np.int32))
        self.X = torch.empty((B, S), dtype=torch.bfloat16, device=d)
        self.X[: B - n] = t(self.host_Xn).to(torch.bfloat16)
        self.Q, self.q = t(self.host_Q), t(self.host_q)
        self.her_next = torch.empty((n, S), dtype=torch.float32, device=d)
        self.her_act = torch.empty(n, dtype=torch.int32, device=d)
        self.her_rew = torch.empty(n, dtype=torch.float32, device=d)
        self.her_done = torch.empty(n, dtype=torch.float32, device=d)
        self.her_donor = torch.empty(n, dtype=torch.int32, device=d)

        cfg = m.make_config(S, w.H, B, num_groups=w.groups, compute_dtype=m.BF16, states_ld=S,
                            tau=w.taus, lr=w.lr, max_grad_norm=w.max_grad_norm)
        self.tr = m.IqlTrainer(cfg, np.concatenate(self.inits))
        self.out_v = torch.empty((w.groups, B), dtype=torch.float32, device=d)
        self.out_loss = torch.empty(w.groups, dtype=torch.float32, device=d)
        self.out_gn = torch.empty(w.groups, dtype=torch.float32, device=d)
        self.pi = torch.empty((w.groups, B, A), dtype=torch.float32, device=d)

        self.hcfg = m.her_config(S, w.G, m.HER_FUTURE)
        self.hbuf = m.her_buffer(self.rb_states, self.rb_next, self.rb_actions, self.rb_dones, self.rb_ends)
        tail = self.X.data_ptr() + (B - n) * S * self.X.element_size()
        self.hout = m.her_out(tail, m.BF16, S, self.her_rew, next_states=self.her_next,
                              actions=self.her_act, dones=self.her_done, donor_idx=self.her_donor,
                              d_flags=self.tr.flags)

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

        self.her_step = m.her_step(self.hcfg, self.hbuf, self.src, w.n_her, 20261202, self.hout)
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
        m.grad_budget_accumulate(self.grad, self.sources, w.budget_fractions, (1.0, 1.0, 1.0, 1.0),
                                 w.n_budget, w.max_grad_norm, self.norms, self.adam, self.ws)


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
    theta = iql.AdamState.fresh(ctx.host_theta)
    hp = iql.AdamHP(lr=w.lr, max_grad_norm=w.max_grad_norm)
    t0 = time.perf_counter()
    steps = 0
    while True:
        r = her.her_step(ctx.host_buf, ctx.host_src, w.G, her.FUTURE, 20261202, steps, out_bf16=True)
        X = np.concatenate([Xn, r["states"].astype(np.float64)])
        vs = [iql.train_step(states[g], X, ctx.host_q, w.S, w.H, w.H, w.taus[g], hp).v for g in range(w.groups)]
        for g in range(w.groups):
            aw.aw_policy(ctx.host_Q, vs[g], w.beta)
        grad, _, _, _ = budget.accumulate(ctx.host_sources, w.budget_fractions, (1, 1, 1, 1), w.max_grad_norm)
        iql.adam_step(theta, grad, hp)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": w.B * steps / el, "unit": "samples/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{steps} full steps of the same workload (fp64 NumPy oracle; BLAS threads = cores), "
                      f"{el:.1f} s", "s_per_step": el / steps, "host_cpus": os.cpu_count()}


def main():
    a = parse()
    if a.copy_probe:
        copy_probe(a.copy_probe)
        return
    if a.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {a.gpus} is not supported by this build "
              "(the step has no cross-GPU exchange; see the sharding notes).", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    sys.path.insert(0, ROOT)
    import offline_rl_step_amd as m
    import synth

    w = synth.WORKLOADS[synth.BENCH_WORKLOAD]
    ctx = Context(m, w, torch, np, synth)
    torch.cuda.synchronize()

    step = ctx.step_separate if a.separate else ctx.step
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if not a.no_graph:
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

    # every launch of the step timed by its own dispatch events, on the
    # stream the step runs on; the dominant one is the forward/backward
    launch_us = ctx.time_launches(a.kernel_reps)
    avg_us = launch_us[1]
    flops = fused_flops_per_launch(w)
    achieved = flops / (avg_us * 1e-6) / 1e12
    src_hash = kernel_source_hash()
    roofline = {"bound": "mfma", "kernel": "iql_fused16_kernel<128,128,xvec>", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": traffic_from_profiles("iql_fused_b16384_s128_h128_g2", src_hash),
                "avg_kernel_us": avg_us, "flops_per_launch": flops, "source_hash": src_hash}

    out = {"metric": METRIC, "value": w.B / (ms_per_step * 1e-3), "unit": "samples/s", "n_gpus": 1,
           "steps": a.steps, "warmup": a.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": w.name, "global_batch": w.B, "state_dim": w.S, "hidden": w.H,
                      "actions": w.A, "groups": w.groups, "her_rows": w.n_her, "her_strategy": w.strategy,
                      "replay_rows": w.C, "budget_params": w.n_budget, "budget_sources": 4,
                      "graph_replay": graph is not None,
                      "entry_point": "separate calls" if a.separate else "iql_aux_step",
                      "parallelism": "single-gpu"},
           "event_ms_per_step": ev_ms / a.steps, "device_flags": flags, "status": rc,
           "launch_us": {"relabel_norms": launch_us[0], "fwd_bwd": launch_us[1], "reduce_saxpy": launch_us[2],
                         "adam": launch_us[3]},
           "roofline": roofline}
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(ctx, a.cpu_seconds, np)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
