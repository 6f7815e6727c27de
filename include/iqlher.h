/*
 * iqlher.h -- C ABI of the MI355X (gfx950) IQL + HER auxiliary-trainer step.
 *
 * One training step of an Implicit Q-Learning value trainer fed by Hindsight
 * Experience Replay, as described on these pages:
 *   [P1] "GPU IQL + HER Porting Plan"
 *   [P2] "DQN Backward-Path NaN Audit -- SP1 Phase A"
 *   [P3] "Phase 2: Multi-Stream Graph Parallelism"
 *   [P5] "Gradient Stability -- Proper Multi-Task Gradient Isolation +
 *        Full Spectral Norm"
 *
 * Conventions shared by every entry point
 *   - Pointers named d_* or documented "device" are HIP device pointers (any
 *     allocation visible to the current device); "host" pointers are read
 *     during the call only.  No entry point keeps a caller pointer.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every call that takes a stream only enqueues work on it: no host
 *     synchronisation, no allocation, no memset node -- all of them may be
 *     captured into a HIP graph and replayed.
 *   - Return value: IQLH_OK or a negative iqlh_status.  Argument errors are
 *     detected on the host before any HIP call; iqlh_last_error() then holds a
 *     message (thread-local).  Errors the device detects (non-finite gradient,
 *     an index outside the buffer) are recorded in a sticky device flag word
 *     and reported by iql_status().
 *   - Floating-point tensors are IEEE binary32 unless the config selects
 *     IQLH_BF16 for the GEMM operand `states` (bfloat16, stored as uint16).
 *   - Row-major layouts throughout; weights are [out, in].
 */
#ifndef IQLHER_H
#define IQLHER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    IQLH_OK = 0,
    IQLH_EINVAL = -1,     /* null pointer, bad size or hyper-parameter       */
    IQLH_ESHAPE = -2,     /* shape the library has no kernel for             */
    IQLH_ENOMEM = -3,     /* device allocation failed (iql_create only)      */
    IQLH_EHIP = -4,       /* a HIP runtime call failed                       */
    IQLH_ENONFINITE = -5  /* iql_status: the device saw a non-finite value   */
} iqlh_status;

typedef enum { IQLH_F32 = 0, IQLH_BF16 = 1 } iqlh_dtype;

/* Sticky device flag bits (iql_status, her_out.d_flags, iqlh_adam.d_flags). */
#define IQLH_FLAG_NONFINITE_GRAD 0x1  /* Adam saw a non-finite clipped grad  */
#define IQLH_FLAG_BAD_INDEX      0x2  /* HER source/donor outside the buffer */
#define IQLH_FLAG_NONFINITE_LOSS 0x4  /* non-finite expectile loss term      */
#define IQLH_FLAG_NONFINITE_STATE 0x8 /* Adam wrote a non-finite p, m or v   */

/* ------------------------------------------------------------------------
 * IQL value trainer ([P1] "Current State / IQL (CPU)", "CUDA Kernel:
 * iql_value_kernel.cu", "Rust Integration: gpu_iql_trainer.rs"; grouped
 * high/low trainers: [P3] "2C. Grouped GEMM for IQL").
 *
 * V(s) = w3 . relu(W2 relu(W1 s + b1) + b2) + b3, W1 [H1, state_dim],
 * W2 [H2, H1], w3 [H2], b3 scalar, with H1 = hidden and H2 = hidden2 (the
 * pages' IqlGpuConfig has separate v_h1 / v_h2, [P1] "Rust Integration:
 * gpu_iql_trainer.rs").  Flat parameter order per group: w1, b1, w2, b2, w3,
 * b3 (iql_config_num_params elements).
 * ---------------------------------------------------------------------- */
typedef struct iqlh_config {
    int32_t state_dim;      /* S >= 1                                          */
    int32_t hidden;         /* H1: width of the first hidden layer (and of the
                               second when hidden2 is 0)                       */
    int32_t max_batch;      /* largest B passed to iql_train_step              */
    int32_t num_groups;     /* 1 or 2 trainers sharing states and q_taken      */
    int32_t compute_dtype;  /* iqlh_dtype of `states` and of the GEMM operands */
    int32_t hidden2;        /* H2: width of the second hidden layer, 0 = H1.
                               H2 != H1 runs on the layered GEMM kernels (the
                               fused and wide kernels are built for H2 = H1) */
    int64_t states_ld;      /* row stride of `states`, elements, >= state_dim  */
    float tau[2];           /* expectile tau per group, in [0, 1]              */
    float lr, beta1, beta2, eps, weight_decay, max_grad_norm;
    float weight_clamp_max_abs;  /* post-update |p| bound, 0 = off ([P2] Mech 9) */
} iqlh_config;

typedef struct iql_trainer* iql_handle;

/* Parameters per group with H1 = H2 = hidden: S*H + H + H*H + H + H + 1.
 * Host only. */
int iql_num_params(int32_t state_dim, int32_t hidden, int64_t* out_count);
/* Parameters per group of a config: S*H1 + H1 + H2*H1 + H2 + H2 + 1.  Host
 * only; checks only the three widths. */
int iql_config_num_params(const iqlh_config* cfg, int64_t* out_count);

/* Creates a trainer on the current device.  `init_params_host` holds
 * num_groups * iql_config_num_params floats (group-major) and is copied; Adam
 * moments start at zero and the step counter t at 0.  The handle owns the
 * fp32 master weights, Adam moments, gradients, the GEMM-operand shadows of
 * the weights and the per-workgroup partial buffers sized for max_batch.
 * Returns IQLH_ESHAPE when no kernel is built for (dtype, state_dim, hidden). */
int iql_create(const iqlh_config* cfg, const float* init_params_host, iql_handle* out);
int iql_destroy(iql_handle h);

/* One IQL step for every group, enqueued on `stream`:
 *   V(s) forward, expectile loss on diff = q_taken - V with weight tau where
 *   diff >= 0 and 1 - tau elsewhere, loss = mean over the B rows ([P1] "Current
 *   State / IQL (CPU)"); backward through the MLP (q_taken is a stop-gradient
 *   target, [P1] "IQL GPU Porting"); global L2 norm of the flat gradient; clip
 *   by max_grad_norm / norm when norm > max_grad_norm; Adam with bias
 *   correction, t incremented before use, non-finite elements skipped and the
 *   gradient zeroed after use ([P2] section on iqn_adam_kernel).
 *   states   device [B, states_ld] of compute_dtype (only the first state_dim
 *            columns are read).
 *   q_taken  device [B] f32, Q(s, a_taken).
 *   out_v    device [num_groups, B] f32, V(s) before the update, or NULL.
 *   out_loss device [num_groups] f32, or NULL.
 *   out_grad_norm device [num_groups] f32, pre-clip norm, or NULL.
 * 1 <= B <= max_batch.  Also increments the device step counter. */
int iql_train_step(iql_handle h, const void* states, const float* q_taken, int32_t batch,
                   float* out_v, float* out_loss, float* out_grad_norm, void* stream);

/* iql_train_step plus the advantage-weighted policy of every group from this
 * step's V(s) (the policy of iql_aw_policy below):
 *   q_all  device [B, num_actions] f32 Q(s, .);  out_pi device [G, B, A] f32;
 *   out_v  required here.
 * With bf16 operands, hidden 128 and num_actions <= 16 the policy is
 * computed inside the forward/backward launch (V never leaves registers);
 * otherwise the iql_aw_policy kernel runs after it.  The IQL trainer feeds
 * its advantage weights to later trainers ([P3] "2A. Aux Child", IQL runs
 * first because CQL reads the IQL advantage weights). */
int iql_train_step_aw(iql_handle h, const void* states, const float* q_taken, int32_t batch,
                      const float* q_all, int32_t num_actions, float beta, float* out_pi,
                      float* out_v, float* out_loss, float* out_grad_norm, void* stream);

/* The two halves of iql_train_step, for callers that time or schedule them
 * separately ([P1] "CUDA Kernel: iql_value_kernel.cu" fuses forward, loss and
 * backward into one launch; the norm and Adam follow as separate phases):
 *   iql_compute_gradients: V(s) into out_v (or NULL) and the expectile-loss
 *     gradient of every group into the handle's per-workgroup partial
 *     buffers (overwritten, not accumulated).  Parameters are not changed.
 *   iql_apply_gradients: sums those partials in a fixed order, writes the
 *     mean loss and the pre-clip norm, clips, applies Adam and increments t
 *     and the step counter.  `batch` must equal the preceding
 *     iql_compute_gradients call's batch. */
int iql_compute_gradients(iql_handle h, const void* states, const float* q_taken, int32_t batch,
                          float* out_v, void* stream);
int iql_apply_gradients(iql_handle h, int32_t batch, float* out_loss, float* out_grad_norm,
                        void* stream);

/* Measurement aid: launches the iql_compute_gradients kernel `reps` times,
 * each bracketed by HIP events that the dispatch itself records, waits for
 * each, and writes the mean kernel duration in microseconds.  Synchronous and
 * not capturable; the partial buffers are overwritten, parameters unchanged. */
int iql_time_compute_gradients(iql_handle h, const void* states, const float* q_taken,
                               int32_t batch, int32_t reps, float* out_avg_us, void* stream);

/* Measurement aid: the layout of the per-workgroup gradient partials that
 * iql_compute_gradients writes for `batch` rows -- *out_rows partial rows per
 * group, each *out_row_floats floats (the parameter count rounded up to 128).
 * Host only, no HIP call. */
int iql_partial_layout(iql_handle h, int32_t batch, int32_t* out_rows, int64_t* out_row_floats);

/* Copies one group's state to / from device buffers of iql_num_params floats
 * (params, m, v) and one int32 (t).  set_state also refreshes the shadows. */
int iql_get_state(iql_handle h, int32_t group, float* d_params, float* d_m, float* d_v,
                  int32_t* d_t, void* stream);
int iql_set_state(iql_handle h, int32_t group, const float* d_params, const float* d_m,
                  const float* d_v, const int32_t* d_t, void* stream);

/* Forward-only V on next states and the IQL bootstrap target ([P1]
 * "Rust Integration: gpu_iql_trainer.rs", forward_values; "Phase 2
 * Integration": the DQN target becomes r + gamma V(s') in place of the
 * target network's maximum).  Uses the online parameters of every group; no
 * loss, no gradient, no state change.
 *   next_states  device [B, states_ld] of states_dtype (IQLH_F32 or
 *                IQLH_BF16; e.g. her_out.next_states, f32).  A dtype other
 *                than the trainer's compute dtype is converted once (bf16
 *                round to nearest even) into a handle-owned buffer first.
 *   out_v        device [num_groups, B] f32: V(s').
 *   rewards      device [B] f32, or NULL (then out_target must be NULL).
 *   dones        device [B] f32 (1 = terminal), or NULL (no terminal rows).
 *   out_target   device [num_groups, B] f32: r + gamma (1 - done) V(s').
 * 1 <= B <= max_batch, gamma finite.  V(s') equals, bit for bit, the V(s)
 * that iql_train_step reports for the same rows and parameters. */
int iql_forward_values(iql_handle h, const void* next_states, int32_t states_dtype, int64_t states_ld,
                       int32_t batch, float* out_v, const float* rewards, const float* dones, float gamma,
                       float* out_target, void* stream);

/* Polyak (EMA) target copy of the value network ([P1] "Rust Integration:
 * gpu_iql_trainer.rs", target_ema_update; run after the IQL step in "Where
 * in the Training Loop IQL Gets Called").  The handle keeps a target copy of
 * every group's flat parameters, equal to the initial parameters at
 * iql_create, updated elementwise as
 *   target <- target + tau (params - target)      (fp32, one rounding per step)
 * iql_target_ema_update: one update of every group with the current params,
 *   enqueued on `stream`.  0 <= tau <= 1.
 * iql_set_target_ema: host-side setting; with tau > 0 every later step
 *   (iql_train_step, iql_train_step_aw, iql_apply_gradients, iql_aux_step)
 *   applies the same update to each parameter right after Adam writes it, in
 *   the Adam launch (no extra pass).  0 (the default) turns it off.  The
 *   result equals the step followed by iql_target_ema_update(tau), bit for bit.
 * iql_get_target / iql_set_target: copy one group's target (iql_num_params
 *   floats) to / from a device buffer. */
int iql_target_ema_update(iql_handle h, float tau, void* stream);
int iql_set_target_ema(iql_handle h, float tau);
int iql_get_target(iql_handle h, int32_t group, float* d_params, void* stream);
int iql_set_target(iql_handle h, int32_t group, const float* d_params, void* stream);

/* Device int64 step counter owned by the handle (0 before the first step);
 * pass it to her_relabel as d_step so a replayed graph draws new donors. */
const int64_t* iql_step_counter(iql_handle h);
/* Device int32 sticky flag word owned by the handle (IQLH_FLAG_*). */
int32_t* iql_flags(iql_handle h);
/* Synchronises the device, copies the flag word to *flags_host (may be NULL)
 * and returns IQLH_ENONFINITE if a non-finite flag is set, IQLH_ESHAPE if a
 * bad-index flag is set, else IQLH_OK.  Never call it inside a timed loop. */
int iql_status(iql_handle h, int32_t* flags_host);

/* ------------------------------------------------------------------------
 * Advantage-weighted policy ([P1] "Current State / IQL (CPU)", item
 * "Advantage-weighted action selection"):
 *   pi[g, b, a] = softmax_a(beta * clamp(q[b, a] - v[g, b], -10, 10)),
 * with the row maximum subtracted before exponentiation.
 *   q  device [B, A] f32;  v device [G, B] f32;  out_pi device [G, B, A] f32.
 * 1 <= A <= 64.  NaN gaps clamp to the bound (fminf/fmaxf semantics). */
int iql_aw_policy(const float* q, const float* v, int32_t num_groups, int32_t batch,
                  int32_t num_actions, float beta, float* out_pi, void* stream);

/* ------------------------------------------------------------------------
 * HER relabelling ([P1] "CUDA Kernel: her_relabel_kernel.cu", "Donor Index
 * Generation", "How HER Interacts with GPU PER").
 *
 * For each row i < n with src = source_idx[i] and donor chosen by strategy:
 *   FINAL  donor = end - 1, end = exclusive end of src's episode;
 *   FUTURE donor uniform in [src + 1, end), or src when that range is empty;
 *   RANDOM donor uniform in [0, buffer_size).
 * Uniform draws: word 0 of Philox4x64-10 (Salmon et al., SC'11) with key
 * (seed, 0x484552646F6E6F72) and counter (i, *d_step, 0, 0), mapped to
 * lo + floor(word * span / 2^64).
 *   out.states[i]      = states[src] with entries [0, goal_dim) replaced by
 *                        next_states[donor][0, goal_dim)  (f32 or bf16 RNE)
 *   out.next_states[i] = next_states[src], same goal replacement (f32)
 *   out.actions[i] = actions[src], out.dones[i] = dones[src]
 *   out.rewards[i] = reward_hit if sqrt(sum_d (next_states[src][d] -
 *                    next_states[donor][d])^2) < goal_threshold else
 *                    reward_miss, summed in goal order in binary32 without
 *                    fused multiply-add, correctly rounded sqrt.
   out.is_weights[i] = 1.0
 * Writing out.states = X + (B - n) * ld appends the relabelled rows to a
 * merged batch X without a copy (normal rows first). */
typedef enum { HER_FINAL = 0, HER_FUTURE = 1, HER_RANDOM = 2 } her_strategy;

typedef struct her_config {
    int32_t state_dim;       /* S                                         */
    int32_t goal_dim;        /* G, 0 <= G <= S                             */
    int32_t strategy;        /* her_strategy                               */
    int32_t reserved0;
    float goal_threshold;    /* 0.01 on the pages                          */
    float reward_hit;        /* +1.0                                       */
    float reward_miss;       /* -0.01                                      */
    float reserved1;
} her_config;

typedef struct her_buffer {
    const float* states;        /* device [capacity, state_dim] f32        */
    const float* next_states;   /* device [capacity, state_dim] f32        */
    const int32_t* actions;     /* device [capacity]                       */
    const float* rewards;       /* device [capacity]; not read (the reward is
                                   recomputed), may be NULL               */
    const float* dones;         /* device [capacity]                       */
    const int32_t* episode_ends;/* device [num_episodes], exclusive ends,
                                   ascending; episode e = [ends[e-1], ends[e]) */
    int64_t capacity;           /* rows allocated                          */
    int64_t buffer_size;        /* rows filled, <= capacity, <= ends[last] */
    int32_t num_episodes;       /* >= 1                                    */
    int32_t reserved0;
} her_buffer;

typedef struct her_out {
    int32_t* donor_idx;         /* device [n] or NULL                      */
    void* states;               /* device [n, states_ld], states_dtype     */
    int32_t states_dtype;       /* iqlh_dtype                              */
    int32_t reserved0;
    int64_t states_ld;          /* >= state_dim                            */
    float* next_states;         /* device [n, state_dim] f32 or NULL       */
    int32_t* actions;           /* device [n] or NULL                      */
    float* rewards;             /* device [n]                              */
    float* dones;               /* device [n] or NULL                      */
    int32_t* d_flags;           /* device sticky flag word or NULL         */
    float* is_weights;          /* device [n] f32 or NULL: the rows' importance-
                                   sampling weights in the merged batch, 1.0
                                   for every relabelled row ([P1] "How HER
                                   Interacts with GPU PER": HER rows are not
                                   drawn by priority); 0 for a zeroed row.
                                   Pointing it at W + (B - n) for the batch's
                                   weight vector W completes the merged weights
                                   in place, as out.states does for the rows. */
} her_out;

/* n >= 0 rows (n == 0 is a no-op).  d_step: device int64 counter (NULL = 0).
 * A source index outside [0, buffer_size) or a donor outside it (malformed
 * episode_ends) sets IQLH_FLAG_BAD_INDEX; that row's outputs are zeroed and
 * its donor_idx is -1. */
int her_relabel(const her_config* cfg, const her_buffer* buf, const int32_t* source_idx,
                int32_t n, uint64_t seed, const int64_t* d_step, const her_out* out,
                void* stream);

/* ------------------------------------------------------------------------
 * Budgeted clipped-SAXPY accumulation ([P5] "Design -- Why the current
 * per-component clipping is wrong" / "Proper design", "Task 1", "Task 2"):
 *   n_k = ||s_k||,  c_k = f_k*mgn / n_k if n_k > f_k*mgn and n_k > 0 else 1,
 *   grad = sum_k alpha_k * c_k * s_k  (k = 0 is the primary source),
 * then optionally Adam on the parameters with the safety clip at mgn.
 *   grad_buf     device [n] f32 output; may alias sources[0] (in place).
 *   sources      host array of k device pointers [n] f32.
 *   fractions, alphas  host [k] f32.
 *   out_norms    device [k + 1] f32: n_0 .. n_{k-1}, then ||grad||; or NULL.
 *   adam         NULL, or Adam state for the parameters grad belongs to; when
 *                given, grad_buf is consumed and left zeroed.
 *   workspace    device, >= grad_budget_workspace_bytes(n, k) bytes, no
 *                initial contents required.
 * 1 <= k <= 8, n >= 1. */
typedef struct iqlh_adam {
    float* params;              /* device [n] */
    float* m;                   /* device [n] */
    float* v;                   /* device [n] */
    int32_t* t;                 /* device step counter, incremented before use */
    int32_t* d_flags;           /* device sticky flag word or NULL */
    float lr, beta1, beta2, eps, weight_decay, max_grad_norm, weight_clamp_max_abs;
    float reserved0;
} iqlh_adam;

int grad_budget_workspace_bytes(int64_t n, int32_t num_sources, size_t* bytes);
int grad_budget_accumulate(float* grad_buf, const float* const* sources, const float* fractions,
                           const float* alphas, int32_t num_sources, int64_t n,
                           float max_grad_norm, float* out_norms, const iqlh_adam* adam,
                           void* workspace, size_t workspace_bytes, void* stream);

/* grad_budget_accumulate for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results, bit for bit, without the
 * workspace -- the passes use a library-owned static device array of 73,736
 * bytes ((8 + 1) * 2048 + 2 floats, enough for every n and k <= 8) instead.
 * Nothing is allocated or freed, by the call or by the library.  The array's
 * address is looked up once per device, on the first call with that device
 * current.  Every call on one device shares that device's array and no
 * contents carry over between calls, so calls that overlap in time on one
 * device (other streams, other threads) race: serialise them.  A workspace
 * the scratch cannot hold is rejected with IQLH_EINVAL (none can, for valid
 * n and k); the other errors are those of grad_budget_accumulate. */
int grad_budget_accumulate_noalloc(float* grad_buf, const float* const* sources, const float* fractions,
                                   const float* alphas, int32_t num_sources, int64_t n,
                                   float max_grad_norm, float* out_norms, const iqlh_adam* adam,
                                   void* stream);

/* ------------------------------------------------------------------------
 * The whole auxiliary step in one call: HER rows into the merged batch, the
 * IQL step on it with the advantage-weighted policy, and the budgeted
 * accumulation + Adam of the main network's gradient ([P1] "Phase 3:
 * Combined IQL + HER" and "How HER Interacts with GPU PER"; [P5] "Task 1").
 * The results equal, bit for bit, those of
 *   her_relabel(her->cfg, her->buf, her->source_idx, her->n, her->seed,
 *               iql_step_counter(h), her->out, stream);
 *   iql_train_step_aw(h, states, q_taken, batch, q_all, ...)
 *       (iql_train_step when q_all is NULL);
 *   grad_budget_accumulate(budget->grad_buf, ..., stream);
 * but the work is enqueued as four launches: passes that do not depend on
 * each other share a launch.
 *   her     NULL: no relabelling.  The Philox step word is the handle's step
 *           counter before this step increments it.  her->out->states may
 *           point into `states` (the merged batch); no other buffer of one
 *           part may overlap a buffer of another part.
 *   q_all   NULL: no policy (num_actions, beta, out_pi ignored).
 *   budget  NULL: no accumulation.
 * Each part is validated as its own entry point validates it; when any check
 * fails nothing is enqueued. */
typedef struct iqlh_her_step {
    const her_config* cfg;
    const her_buffer* buf;
    const int32_t* source_idx;  /* device [n] */
    const her_out* out;
    uint64_t seed;
    int32_t n;
    int32_t reserved0;
} iqlh_her_step;

typedef struct iqlh_budget_step {
    float* grad_buf;            /* as grad_budget_accumulate */
    const float* const* sources;
    const float* fractions;
    const float* alphas;
    float* out_norms;
    const iqlh_adam* adam;
    void* workspace;
    size_t workspace_bytes;
    int64_t n;
    int32_t num_sources;
    float max_grad_norm;
} iqlh_budget_step;

int iql_aux_step(iql_handle h, const iqlh_her_step* her, const void* states, const float* q_taken,
                 int32_t batch, const float* q_all, int32_t num_actions, float beta, float* out_pi,
                 float* out_v, float* out_loss, float* out_grad_norm, const iqlh_budget_step* budget,
                 void* stream);

/* Measurement: enqueues `reps` whole steps with the arguments of
 * iql_aux_step (they update the state like any other step), each launch
 * timed by its own dispatch events (kernel time only, no launch gaps), and
 * writes the mean duration in microseconds of each of the four launches:
 * out_avg_us[0] relabelling and budget norms (0 when that launch is not
 * needed: HER rows that form the bf16 batch tail from a 128-row boundary and
 * the budget norms then ride in the forward/backward launch), [1]
 * forward/backward, [2] reduction and SAXPY, [3] both Adam updates.
 * Synchronises the stream. */
int iql_time_aux_step(iql_handle h, const iqlh_her_step* her, const void* states,
                      const float* q_taken, int32_t batch, const float* q_all,
                      int32_t num_actions, float beta, float* out_pi, float* out_v,
                      float* out_loss, float* out_grad_norm, const iqlh_budget_step* budget,
                      int32_t reps, float* out_avg_us, void* stream);

/* Measurement aid: iql_aux_step (same arguments, same results, bit for
 * bit) with the forward/backward launch run by an instantiation of its
 * kernel that also records, per workgroup, the 100 MHz clock at the ends of
 * its phases: d_stamps device [groups][ceil(batch / 128)][8] uint64 (tile
 * order, the layout of the gradient partials): kernel start, then the ends
 * of the staging of weights and rows (with the HER relabelling and the
 * budget's pass 1 when the launch hosts them), F1, F2 + V, loss / dz2,
 * dW2 (+ W2^T and the policy), dh1 / dz1, and the issue of the last dW1
 * partial stores.  stamps_len = elements available.  Only for the kernel
 * of bf16 trainers at hidden 128 (IQLH_ESHAPE otherwise). */
int iql_aux_step_phase_stamps(iql_handle h, const iqlh_her_step* her, const void* states,
                              const float* q_taken, int32_t batch, const float* q_all,
                              int32_t num_actions, float beta, float* out_pi, float* out_v,
                              float* out_loss, float* out_grad_norm,
                              const iqlh_budget_step* budget, uint64_t* d_stamps,
                              int32_t stamps_len, void* stream);

/* ------------------------------------------------------------------------
 * Prioritized-replay source sampling ([P1] "Current State": the GPU PER
 * buffer samples by a prefix sum of the priorities and a search in it and
 * returns indices and IS weights; "How HER Interacts with GPU PER":
 * sample_indices for the HER sources).
 *   Row i is drawn with probability p_i / sum(p), n times independently, by
 *   inverse transform: u = U * total with U = (word >> 11) * 2^-53, word =
 *   word 0 of Philox4x64-10 with key (seed, 0x5045526472617773) and counter
 *   (k, *d_step, 0, 0) for draw k, u capped just below the total; the row is
 *   the first i whose inclusive binary64 prefix sum exceeds u.
 *   IS weight of draw k: (p_min / p_idx[k])^beta, p_min the smallest drawn
 *   priority (prioritized replay's (N P(i))^-beta over the batch maximum).
 *   d_priorities  device [size] f32, >= 0 (already raised to any exponent).
 *   d_out_idx     device [n] int32; d_out_weights device [n] f32 (both also
 *                 hold each draw's counter word between the launches: they
 *                 must not overlap each other or the priorities).
 *   d_step        device int64 counter or NULL (= 0).
 *   d_flags       device sticky flag word or NULL: IQLH_FLAG_BAD_INDEX when a
 *                 priority is negative or non-finite or the total is not > 0
 *                 (then the draws are -1 with weight 0).
 *   workspace     device, >= per_workspace_bytes(size), 8-byte aligned; starts
 *                 afterwards with the binary64 sum of every 2048-row block
 *                ([ceil(size / 2048)]).
 * 1 <= size < 2^31, n >= 0 (0 computes the block sums only), beta >= 0. */
int per_workspace_bytes(int64_t size, size_t* bytes);
int per_sample_indices(const float* d_priorities, int64_t size, int32_t n, uint64_t seed, const int64_t* d_step,
                       float beta, int32_t* d_out_idx, float* d_out_weights, int32_t* d_flags, void* workspace,
                       size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Fused non-finite sentinel ([P2] "Phase E -- SP2 fused NaN check kernel":
 * one launch over a table of buffers, a sticky flag per slot that is written
 * 1 and never cleared, null entries skipped).
 *   d_bufs        host array of num_slots device pointers to fp32 buffers
 *                 (NULL entries are skipped; any alignment).
 *   lens          host array of element counts (>= 0).
 *   d_slot_flags  device int32 [num_slots]: slot s is set to 1 when buffer s
 *                 holds a NaN or an infinity; a clean slot keeps its value.
 * 1 <= num_slots <= 32.  Reads only.  (Every Adam launch of this library
 * also checks the p, m, v it writes and raises IQLH_FLAG_NONFINITE_STATE.) */
int iqlh_nonfinite_check(const float* const* d_bufs, const int64_t* lens, int32_t num_slots,
                         int32_t* d_slot_flags, void* stream);

/* Thread-local text of the last error returned on this thread ("" if none). */
const char* iqlh_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* IQLHER_H */
