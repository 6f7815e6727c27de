// C ABI of the IQL + HER step (include/iqlher.h): argument validation, the
// trainer handle and its device buffers, and kernel dispatch.  Every check
// that can fail on the host runs before the first HIP call.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "iqlher.h"
#include "launch.hpp"

using namespace iqlh;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(IQLH_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool finite_pos(float x) { return std::isfinite(x) && x > 0.f; }

}  // namespace

struct iql_trainer {
    iqlh_config cfg;
    IqlDims dims;
    IqlBuffers buf;
    int device;
    float ema_tau;  // Polyak weight folded into every step's Adam launch, 0 = off
    void* fv_states;  // [max_batch][S_pad] compute dtype: next states converted for iql_forward_values
    std::vector<void*> allocs;
};

extern "C" {

const char* iqlh_last_error(void) { return g_err; }

int iql_num_params(int32_t state_dim, int32_t hidden, int64_t* out_count) {
    if (!out_count) return fail(IQLH_EINVAL, "iql_num_params: out_count is NULL");
    if (state_dim < 1 || hidden < 1) return fail(IQLH_EINVAL, "iql_num_params: dims must be >= 1");
    const int64_t S = state_dim, H = hidden;
    *out_count = S * H + H + H * H + H + H + 1;
    return IQLH_OK;
}

static int32_t hidden2_of(const iqlh_config* c) { return c->hidden2 ? c->hidden2 : c->hidden; }

int iql_config_num_params(const iqlh_config* cfg, int64_t* out_count) {
    if (!cfg || !out_count) return fail(IQLH_EINVAL, "iql_config_num_params: NULL argument");
    if (cfg->state_dim < 1 || cfg->hidden < 1 || cfg->hidden2 < 0)
        return fail(IQLH_EINVAL, "iql_config_num_params: state_dim and hidden must be >= 1, hidden2 >= 0");
    const int64_t S = cfg->state_dim, H1 = cfg->hidden, H2 = hidden2_of(cfg);
    *out_count = S * H1 + H1 + H2 * H1 + H2 + H2 + 1;
    return IQLH_OK;
}

static int check_config(const iqlh_config* c) {
    if (!c) return fail(IQLH_EINVAL, "config is NULL");
    if (c->state_dim < 1 || c->hidden < 1) return fail(IQLH_EINVAL, "state_dim and hidden must be >= 1");
    if (c->hidden2 < 0) return fail(IQLH_EINVAL, "hidden2 must be >= 0 (0: the same as hidden)");
    if (c->max_batch < 1) return fail(IQLH_EINVAL, "max_batch must be >= 1");
    if (c->num_groups < 1 || c->num_groups > 2) return fail(IQLH_EINVAL, "num_groups must be 1 or 2");
    if (c->compute_dtype != IQLH_F32 && c->compute_dtype != IQLH_BF16)
        return fail(IQLH_EINVAL, "compute_dtype must be IQLH_F32 or IQLH_BF16");
    if (c->states_ld < c->state_dim) return fail(IQLH_EINVAL, "states_ld < state_dim");
    for (int g = 0; g < c->num_groups; ++g)
        if (!(c->tau[g] >= 0.f && c->tau[g] <= 1.f)) return fail(IQLH_EINVAL, "tau[%d] outside [0, 1]", g);
    if (!(c->lr >= 0.f) || !std::isfinite(c->lr)) return fail(IQLH_EINVAL, "lr must be finite and >= 0");
    if (!(c->beta1 >= 0.f && c->beta1 < 1.f) || !(c->beta2 >= 0.f && c->beta2 < 1.f))
        return fail(IQLH_EINVAL, "beta1 and beta2 must be in [0, 1)");
    if (!finite_pos(c->eps)) return fail(IQLH_EINVAL, "eps must be finite and > 0");
    if (!(c->weight_decay >= 0.f) || !std::isfinite(c->weight_decay))
        return fail(IQLH_EINVAL, "weight_decay must be finite and >= 0");
    if (!(c->max_grad_norm > 0.f)) return fail(IQLH_EINVAL, "max_grad_norm must be > 0");
    if (!(c->weight_clamp_max_abs >= 0.f)) return fail(IQLH_EINVAL, "weight_clamp_max_abs must be >= 0");
    const int32_t h2 = hidden2_of(c);
    if (!iql_supported(c->compute_dtype, c->state_dim, c->hidden) &&
        !iql_layered_supported(c->compute_dtype, c->state_dim, c->hidden))
        return fail(IQLH_ESHAPE, "no kernel for dtype=%d state_dim=%d hidden=%d", c->compute_dtype,
                    c->state_dim, c->hidden);
    if (h2 != c->hidden && !iql_layered_supported(c->compute_dtype, c->state_dim, h2))
        return fail(IQLH_ESHAPE, "no kernel for hidden2=%d", h2);
    return IQLH_OK;
}

static void free_all(iql_trainer* t) {
    for (void* p : t->allocs) (void)hipFree(p);
    t->allocs.clear();
}

static int dev_alloc(iql_trainer* t, void** p, size_t bytes) {
    hipError_t e = hipMalloc(p, bytes < 256 ? 256 : bytes);
    if (e != hipSuccess) return fail(IQLH_ENOMEM, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
    t->allocs.push_back(*p);
    e = hipMemset(*p, 0, bytes < 256 ? 256 : bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMemset");
    return IQLH_OK;
}

int iql_create(const iqlh_config* cfg, const float* init_params_host, iql_handle* out) {
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!init_params_host) return fail(IQLH_EINVAL, "init_params_host is NULL");
    if (!out) return fail(IQLH_EINVAL, "out is NULL");
    *out = nullptr;
    iql_trainer* t = new (std::nothrow) iql_trainer();
    if (!t) return fail(IQLH_ENOMEM, "host allocation failed");
    t->cfg = *cfg;
    hipError_t e = hipGetDevice(&t->device);
    if (e != hipSuccess) { delete t; return hip_fail(e, "hipGetDevice"); }
    const int G = cfg->num_groups, S = cfg->state_dim, H = cfg->hidden, H2 = hidden2_of(cfg);
    int64_t P = 0;
    iql_config_num_params(cfg, &P);
    IqlDims& d = t->dims;
    d.S = S; d.H = H; d.H2 = H2; d.G = G; d.dtype = cfg->compute_dtype;
    // two different hidden widths: the layered GEMMs (the fused and wide
    // kernels are built for one width)
    d.layered = (H2 == H && iql_supported(d.dtype, S, H)) ? 0 : 1;
    d.big = d.layered && H2 == H && iql_big_supported(d.dtype, S, H) && cfg->states_ld % 8 == 0;
    d.S_pad = d.layered ? (S + 7) / 8 * 8 : iql_s_pad(d.dtype, S, H);
    d.P = P;
    d.Pp = (P + 127) / 128 * 128;
    const int64_t MB = cfg->max_batch;
    int max_wg, max_loss;
    if (d.big) {
        max_wg = iql_big_max_chunks(S, H);
        max_loss = iql_big_blocks((int)MB);
    } else if (d.layered) {
        max_wg = (int)((MB + iql_layered_chunk() - 1) / iql_layered_chunk());
        max_loss = (int)((MB + 63) / 64);
    } else {
        const int BT = iql_tile_samples(d.dtype, S, H);
        max_wg = max_loss = (int)((MB + BT - 1) / BT);
    }
    const int rb = iql_reduce_blocks(P);
    const size_t esz = d.dtype == IQLH_BF16 ? 2 : 4;
    IqlBuffers& b = t->buf;
    b.max_wg = max_wg;
    b.max_rb = rb;
    b.act_h1 = b.act_dz2 = b.act_p2 = b.act_dz1 = nullptr;
    b.act_z2 = b.act_dv = nullptr;
    b.big_spart = nullptr;
    // activations: h1, dz1 [G][MB][H]; z2, dz2, p2 [G][MB][H2] (layered-only:
    // z2, p2 and dv)
    const size_t nact = d.layered ? (size_t)G * MB * H : 0;
    const size_t nact2 = d.layered ? (size_t)G * MB * H2 : 0;
    const size_t nlay2 = d.layered && !d.big ? nact2 : 0;
    const size_t nlay = d.layered && !d.big ? nact : 0;
    struct { void** p; size_t bytes; } plan[] = {
        {(void**)&b.params, sizeof(float) * G * P},
        {&t->fv_states, esz * (size_t)MB * d.S_pad},
        {(void**)&b.m, sizeof(float) * G * P},
        {(void**)&b.v, sizeof(float) * G * P},
        {(void**)&b.grad, sizeof(float) * G * P},
        {(void**)&b.target, sizeof(float) * G * P},
        {(void**)&b.t, sizeof(int32_t) * G},
        {(void**)&b.bc, sizeof(float) * G * 2},
        {(void**)&b.step, sizeof(int64_t)},
        {(void**)&b.flags, sizeof(int32_t)},
        {(void**)&b.w1s, esz * G * H * d.S_pad},
        {(void**)&b.w2s, esz * G * H2 * H},
        {(void**)&b.w2ts, esz * G * H2 * H},
        {(void**)&b.part, sizeof(float) * G * (size_t)max_wg * d.Pp},
        {(void**)&b.loss_part, sizeof(float) * G * (size_t)max_loss},
        {(void**)&b.sq_part, sizeof(float) * G * (size_t)rb},
        {(void**)&b.act_h1, esz * nact},
        {(void**)&b.act_z2, sizeof(float) * nlay2},
        {(void**)&b.act_dz2, esz * nact2},
        {(void**)&b.act_p2, esz * nlay2},
        {(void**)&b.act_dz1, esz * nact},
        {(void**)&b.act_dv, sizeof(float) * (nlay ? (size_t)G * MB : 0)},
        {(void**)&b.big_spart, sizeof(float) * (d.big ? (size_t)G * iql_big_blocks((int)MB) * iql_big_spart_width(H) : 0)},
    };
    for (auto& a : plan) {
        if (a.bytes == 0) continue;
        rc = dev_alloc(t, a.p, a.bytes);
        if (rc) { free_all(t); delete t; return rc; }
    }
    e = hipMemcpy(b.params, init_params_host, sizeof(float) * G * P, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemcpy(b.target, init_params_host, sizeof(float) * G * P, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = launch_iql_refresh_shadows(d, b, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) { free_all(t); delete t; return hip_fail(e, "iql_create upload"); }
    *out = t;
    return IQLH_OK;
}

int iql_destroy(iql_handle h) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    (void)hipDeviceSynchronize();
    free_all(h);
    delete h;
    return IQLH_OK;
}

static int check_step_args(iql_handle h, const void* states, const float* q_taken, int32_t batch) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    if (!states || !q_taken) return fail(IQLH_EINVAL, "states and q_taken must be non-NULL");
    if (batch < 1 || batch > h->cfg.max_batch)
        return fail(IQLH_EINVAL, "batch %d outside [1, max_batch=%d]", batch, h->cfg.max_batch);
    if (h->dims.big && ((uintptr_t)states & 15u))
        return fail(IQLH_EINVAL, "states must be 16-byte aligned for bf16 operands at hidden %d", h->dims.H);
    return IQLH_OK;
}

static int check_policy_args(const float* q_all, int32_t num_actions, float beta, const float* out_pi,
                             const float* out_v) {
    if (!q_all || !out_pi || !out_v) return fail(IQLH_EINVAL, "policy: q_all, out_pi and out_v are required");
    if (num_actions < 1 || num_actions > 64) return fail(IQLH_EINVAL, "num_actions must be in [1, 64]");
    if (!std::isfinite(beta)) return fail(IQLH_EINVAL, "beta must be finite");
    return IQLH_OK;
}

static AdamHyper adam_hyper(const iql_trainer* h) {
    const iqlh_config& c = h->cfg;
    return AdamHyper{c.lr, c.beta1, c.beta2, c.eps, c.weight_decay, c.max_grad_norm, c.weight_clamp_max_abs, h->ema_tau};
}

int iql_compute_gradients(iql_handle h, const void* states, const float* q_taken, int32_t batch,
                          float* out_v, void* stream) {
    int rc = check_step_args(h, states, q_taken, batch);
    if (rc) return rc;
    hipError_t e = launch_iql_fwd_bwd(h->dims, h->buf, h->cfg.tau, states, h->cfg.states_ld, q_taken, batch,
                                      out_v, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "iql_compute_gradients launch");
    return IQLH_OK;
}

int iql_time_compute_gradients(iql_handle h, const void* states, const float* q_taken, int32_t batch,
                               int32_t reps, float* out_avg_us, void* stream) {
    int rc = check_step_args(h, states, q_taken, batch);
    if (rc) return rc;
    if (reps < 1 || !out_avg_us) return fail(IQLH_EINVAL, "reps must be >= 1 and out_avg_us non-NULL");
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    double total_ms = 0.0;
    for (int r = 0; r < reps && e == hipSuccess; ++r) {
        e = launch_iql_fwd_bwd(h->dims, h->buf, h->cfg.tau, states, h->cfg.states_ld, q_taken, batch,
                               nullptr, (hipStream_t)stream, e0, e1);
        if (e == hipSuccess) e = hipEventSynchronize(e1);
        float ms = 0.f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
        total_ms += ms;
    }
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    if (e != hipSuccess) return hip_fail(e, "iql_time_compute_gradients");
    *out_avg_us = (float)(total_ms * 1000.0 / reps);
    return IQLH_OK;
}

int iql_partial_layout(iql_handle h, int32_t batch, int32_t* out_rows, int64_t* out_row_floats) {
    if (!h || !out_rows || !out_row_floats) return fail(IQLH_EINVAL, "NULL argument");
    if (batch < 1 || batch > h->cfg.max_batch)
        return fail(IQLH_EINVAL, "batch %d outside [1, max_batch=%d]", batch, h->cfg.max_batch);
    int nwg = 0, nloss = 0;
    if (!iql_partial_counts(h->dims, batch, &nwg, &nloss)) return fail(IQLH_ESHAPE, "no kernel for this shape");
    *out_rows = nwg;
    *out_row_floats = h->dims.Pp;
    return IQLH_OK;
}

int iql_apply_gradients(iql_handle h, int32_t batch, float* out_loss, float* out_grad_norm, void* stream) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    if (batch < 1 || batch > h->cfg.max_batch)
        return fail(IQLH_EINVAL, "batch %d outside [1, max_batch=%d]", batch, h->cfg.max_batch);
    hipError_t e = launch_iql_update(h->dims, h->buf, adam_hyper(h), batch, out_loss, out_grad_norm,
                                     (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "iql_apply_gradients launch");
    return IQLH_OK;
}

int iql_train_step_aw(iql_handle h, const void* states, const float* q_taken, int32_t batch,
                      const float* q_all, int32_t num_actions, float beta, float* out_pi, float* out_v,
                      float* out_loss, float* out_grad_norm, void* stream) {
    int rc = check_step_args(h, states, q_taken, batch);
    if (rc) return rc;
    rc = check_policy_args(q_all, num_actions, beta, out_pi, out_v);
    if (rc) return rc;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (iql_policy_in_launch(h->dims, batch, num_actions, q_all, out_pi)) {
        e = launch_iql_fwd_bwd(h->dims, h->buf, h->cfg.tau, states, h->cfg.states_ld, q_taken, batch, out_v, s,
                               nullptr, nullptr, q_all, num_actions, beta, out_pi);
    } else {
        e = launch_iql_fwd_bwd(h->dims, h->buf, h->cfg.tau, states, h->cfg.states_ld, q_taken, batch, out_v, s);
        if (e == hipSuccess) e = launch_aw_policy(q_all, out_v, h->dims.G, batch, num_actions, beta, out_pi, s);
    }
    if (e == hipSuccess)
        e = launch_iql_update(h->dims, h->buf, adam_hyper(h), batch, out_loss, out_grad_norm, s);
    if (e != hipSuccess) return hip_fail(e, "iql_train_step_aw launch");
    return IQLH_OK;
}

int iql_train_step(iql_handle h, const void* states, const float* q_taken, int32_t batch,
                   float* out_v, float* out_loss, float* out_grad_norm, void* stream) {
    int rc = iql_compute_gradients(h, states, q_taken, batch, out_v, stream);
    if (rc) return rc;
    return iql_apply_gradients(h, batch, out_loss, out_grad_norm, stream);
}

int iql_get_state(iql_handle h, int32_t group, float* d_params, float* d_m, float* d_v, int32_t* d_t,
                  void* stream) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    if (group < 0 || group >= h->dims.G) return fail(IQLH_EINVAL, "group %d out of range", group);
    const int64_t P = h->dims.P;
    hipStream_t s = (hipStream_t)stream;
    const size_t bytes = sizeof(float) * P;
    hipError_t e = hipSuccess;
    if (d_params) e = hipMemcpyAsync(d_params, h->buf.params + group * P, bytes, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && d_m) e = hipMemcpyAsync(d_m, h->buf.m + group * P, bytes, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && d_v) e = hipMemcpyAsync(d_v, h->buf.v + group * P, bytes, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess && d_t)
        e = hipMemcpyAsync(d_t, h->buf.t + group, sizeof(int32_t), hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "iql_get_state");
    return IQLH_OK;
}

int iql_set_state(iql_handle h, int32_t group, const float* d_params, const float* d_m, const float* d_v,
                  const int32_t* d_t, void* stream) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    if (group < 0 || group >= h->dims.G) return fail(IQLH_EINVAL, "group %d out of range", group);
    if (!d_params || !d_m || !d_v || !d_t) return fail(IQLH_EINVAL, "set_state needs params, m, v and t");
    const int64_t P = h->dims.P;
    hipStream_t s = (hipStream_t)stream;
    const size_t bytes = sizeof(float) * P;
    hipError_t e = hipMemcpyAsync(h->buf.params + group * P, d_params, bytes, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h->buf.m + group * P, d_m, bytes, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = hipMemcpyAsync(h->buf.v + group * P, d_v, bytes, hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(h->buf.t + group, d_t, sizeof(int32_t), hipMemcpyDeviceToDevice, s);
    if (e == hipSuccess) e = launch_iql_refresh_shadows(h->dims, h->buf, s);
    if (e != hipSuccess) return hip_fail(e, "iql_set_state");
    return IQLH_OK;
}

int iql_forward_values(iql_handle h, const void* next_states, int32_t states_dtype, int64_t states_ld, int32_t batch,
                       float* out_v, const float* rewards, const float* dones, float gamma, float* out_target,
                       void* stream) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    if (!next_states || !out_v) return fail(IQLH_EINVAL, "next_states and out_v must be non-NULL");
    if (batch < 1 || batch > h->cfg.max_batch)
        return fail(IQLH_EINVAL, "batch %d outside [1, max_batch=%d]", batch, h->cfg.max_batch);
    if (states_dtype != IQLH_F32 && states_dtype != IQLH_BF16)
        return fail(IQLH_EINVAL, "states_dtype must be IQLH_F32 or IQLH_BF16");
    if (states_ld < h->dims.S) return fail(IQLH_EINVAL, "states_ld < state_dim");
    if ((rewards == nullptr) != (out_target == nullptr))
        return fail(IQLH_EINVAL, "rewards and out_target go together");
    if (dones && !rewards) return fail(IQLH_EINVAL, "dones without rewards");
    if (!std::isfinite(gamma)) return fail(IQLH_EINVAL, "gamma must be finite");
    const IqlDims& d = h->dims;
    hipStream_t s = (hipStream_t)stream;
    const void* x = next_states;
    int64_t ld = states_ld;
    const bool aligned = ((uintptr_t)next_states & 15u) == 0 && states_ld % 8 == 0;
    if (states_dtype != d.dtype || (d.big && !aligned)) {
        // one conversion pass into the handle's buffer (row stride S_pad)
        hipError_t e = launch_convert_rows(next_states, states_dtype, states_ld, h->fv_states, d.dtype, d.S_pad, batch,
                                           d.S, s);
        if (e != hipSuccess) return hip_fail(e, "iql_forward_values convert");
        x = h->fv_states;
        ld = d.S_pad;
    }
    ValueOut vo{out_v, rewards, dones, gamma, out_target};
    hipError_t e = launch_iql_forward_values(d, h->buf, x, ld, batch, vo, s);
    if (e != hipSuccess) return hip_fail(e, "iql_forward_values launch");
    return IQLH_OK;
}

int iql_target_ema_update(iql_handle h, float tau, void* stream) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    if (!(tau >= 0.f && tau <= 1.f)) return fail(IQLH_EINVAL, "tau must be in [0, 1]");
    hipError_t e = launch_iql_target_ema(h->dims, h->buf, tau, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "iql_target_ema_update");
    return IQLH_OK;
}

int iql_set_target_ema(iql_handle h, float tau) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    if (!(tau >= 0.f && tau <= 1.f)) return fail(IQLH_EINVAL, "tau must be in [0, 1]");
    h->ema_tau = tau;
    return IQLH_OK;
}

int iql_get_target(iql_handle h, int32_t group, float* d_params, void* stream) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    if (group < 0 || group >= h->dims.G) return fail(IQLH_EINVAL, "group %d out of range", group);
    if (!d_params) return fail(IQLH_EINVAL, "d_params is NULL");
    const int64_t P = h->dims.P;
    hipError_t e = hipMemcpyAsync(d_params, h->buf.target + group * P, sizeof(float) * P, hipMemcpyDeviceToDevice,
                                  (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "iql_get_target");
    return IQLH_OK;
}

int iql_set_target(iql_handle h, int32_t group, const float* d_params, void* stream) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    if (group < 0 || group >= h->dims.G) return fail(IQLH_EINVAL, "group %d out of range", group);
    if (!d_params) return fail(IQLH_EINVAL, "d_params is NULL");
    const int64_t P = h->dims.P;
    hipError_t e = hipMemcpyAsync(h->buf.target + group * P, d_params, sizeof(float) * P, hipMemcpyDeviceToDevice,
                                  (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "iql_set_target");
    return IQLH_OK;
}

const int64_t* iql_step_counter(iql_handle h) { return h ? h->buf.step : nullptr; }
int32_t* iql_flags(iql_handle h) { return h ? h->buf.flags : nullptr; }

int iql_status(iql_handle h, int32_t* flags_host) {
    if (!h) return fail(IQLH_EINVAL, "handle is NULL");
    int32_t f = 0;
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMemcpy(&f, h->buf.flags, sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "iql_status");
    if (flags_host) *flags_host = f;
    if (f & (IQLH_FLAG_NONFINITE_GRAD | IQLH_FLAG_NONFINITE_LOSS | IQLH_FLAG_NONFINITE_STATE))
        return fail(IQLH_ENONFINITE, "device flagged a non-finite value (flags=0x%x)", f);
    if (f & IQLH_FLAG_BAD_INDEX) return fail(IQLH_ESHAPE, "device flagged an index outside the buffer");
    return IQLH_OK;
}

int per_workspace_bytes(int64_t size, size_t* bytes) {
    if (!bytes) return fail(IQLH_EINVAL, "bytes is NULL");
    if (size < 1 || size > INT32_MAX) return fail(IQLH_EINVAL, "size must be in [1, 2^31 - 1]");
    *bytes = per_workspace_bytes_for(size);
    return IQLH_OK;
}

int per_sample_indices(const float* d_priorities, int64_t size, int32_t n, uint64_t seed, const int64_t* d_step,
                       float beta, int32_t* d_out_idx, float* d_out_weights, int32_t* d_flags, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (size < 1 || size > INT32_MAX) return fail(IQLH_EINVAL, "size must be in [1, 2^31 - 1]");
    if (n < 0) return fail(IQLH_EINVAL, "n must be >= 0");
    if (!(beta >= 0.f) || !std::isfinite(beta)) return fail(IQLH_EINVAL, "beta must be finite and >= 0");
    if (!d_priorities || !workspace || (n > 0 && (!d_out_idx || !d_out_weights)))
        return fail(IQLH_EINVAL, "per_sample_indices: NULL pointer");
    if (workspace_bytes < per_workspace_bytes_for(size))
        return fail(IQLH_EINVAL, "workspace too small: %zu < %zu bytes", workspace_bytes, per_workspace_bytes_for(size));
    if (((uintptr_t)workspace & 7u) != 0) return fail(IQLH_EINVAL, "workspace must be 8-byte aligned");
    if (n > 0) {
        // the outputs hold the draws' counter words between the launches
        auto overlap = [](const void* a, size_t na, const void* b, size_t nb) {
            const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
            return x < y + nb && y < x + na;
        };
        const size_t no = 4 * (size_t)n, np = 4 * (size_t)size;
        if (overlap(d_out_idx, no, d_out_weights, no) || overlap(d_out_idx, no, d_priorities, np) ||
            overlap(d_out_weights, no, d_priorities, np))
            return fail(IQLH_EINVAL, "per_sample_indices: the outputs overlap each other or the priorities");
    }
    hipError_t e = launch_per_sample(d_priorities, size, n, seed, d_step, beta, d_out_idx, d_out_weights, d_flags,
                                     workspace, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "per_sample_indices launch");
    return IQLH_OK;
}

int iqlh_nonfinite_check(const float* const* d_bufs, const int64_t* lens, int32_t num_slots,
                         int32_t* d_slot_flags, void* stream) {
    if (!d_bufs || !lens || !d_slot_flags) return fail(IQLH_EINVAL, "iqlh_nonfinite_check: NULL argument");
    if (num_slots < 1 || num_slots > kSentinelSlots)
        return fail(IQLH_EINVAL, "num_slots must be in [1, %d]", kSentinelSlots);
    SentinelArgs a{};
    a.flags = d_slot_flags;
    a.nslots = num_slots;
    int64_t blocks = 0;
    for (int s = 0; s < num_slots; ++s) {
        if (lens[s] < 0) return fail(IQLH_EINVAL, "lens[%d] < 0", s);
        const int64_t n = d_bufs[s] ? lens[s] : 0;  // null entries are skipped
        a.ptr[s] = d_bufs[s];
        a.n[s] = n;
        a.block0[s] = (int)blocks;
        if ((((uintptr_t)d_bufs[s]) & 15u) == 0) a.vec |= 1u << s;
        blocks += (n + kSentinelPiece - 1) / kSentinelPiece;
        if (blocks > (int64_t)1 << 30) return fail(IQLH_EINVAL, "iqlh_nonfinite_check: buffers too large");
    }
    a.block0[num_slots] = (int)blocks;
    hipError_t e = launch_nonfinite_sentinel(a, (int)blocks, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "iqlh_nonfinite_check");
    return IQLH_OK;
}

int iql_aw_policy(const float* q, const float* v, int32_t num_groups, int32_t batch, int32_t num_actions,
                  float beta, float* out_pi, void* stream) {
    if (!q || !v || !out_pi) return fail(IQLH_EINVAL, "iql_aw_policy: NULL pointer");
    if (num_groups < 1 || batch < 1) return fail(IQLH_EINVAL, "iql_aw_policy: num_groups and batch must be >= 1");
    if (num_actions < 1 || num_actions > 64) return fail(IQLH_EINVAL, "iql_aw_policy: num_actions must be in [1, 64]");
    if (!std::isfinite(beta)) return fail(IQLH_EINVAL, "iql_aw_policy: beta must be finite");
    hipError_t e = launch_aw_policy(q, v, num_groups, batch, num_actions, beta, out_pi, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "iql_aw_policy launch");
    return IQLH_OK;
}

static int make_her_args(const her_config* cfg, const her_buffer* buf, const int32_t* source_idx, int32_t n,
                         uint64_t seed, const int64_t* d_step, const her_out* out, HerArgs* ap) {
    if (!cfg || !buf || !out) return fail(IQLH_EINVAL, "her_relabel: NULL argument struct");
    if (n < 0) return fail(IQLH_EINVAL, "her_relabel: n < 0");
    if (cfg->state_dim < 1) return fail(IQLH_EINVAL, "her_relabel: state_dim < 1");
    if (cfg->goal_dim < 0 || cfg->goal_dim > cfg->state_dim)
        return fail(IQLH_EINVAL, "her_relabel: goal_dim outside [0, state_dim]");
    if (cfg->strategy < HER_FINAL || cfg->strategy > HER_RANDOM)
        return fail(IQLH_EINVAL, "her_relabel: unknown strategy %d", cfg->strategy);
    if (!std::isfinite(cfg->goal_threshold)) return fail(IQLH_EINVAL, "her_relabel: threshold not finite");
    if (buf->capacity < 1 || buf->buffer_size < 1 || buf->buffer_size > buf->capacity)
        return fail(IQLH_EINVAL, "her_relabel: need 1 <= buffer_size <= capacity");
    if (buf->buffer_size > 0x7FFFFFFFLL) return fail(IQLH_EINVAL, "her_relabel: buffer_size exceeds int32 indices");
    if (cfg->strategy != HER_RANDOM && (buf->num_episodes < 1 || !buf->episode_ends))
        return fail(IQLH_EINVAL, "her_relabel: final/future need episode_ends");
    if (out->states_dtype != IQLH_F32 && out->states_dtype != IQLH_BF16)
        return fail(IQLH_EINVAL, "her_relabel: bad out.states_dtype");
    if (out->states_ld < cfg->state_dim) return fail(IQLH_EINVAL, "her_relabel: out.states_ld < state_dim");
    HerArgs& a = *ap;
    std::memset(&a, 0, sizeof(a));
    a.n = n;
    if (n == 0) return IQLH_OK;
    if (!buf->states || !buf->next_states || !source_idx || !out->states || !out->rewards)
        return fail(IQLH_EINVAL, "her_relabel: NULL device pointer");
    if ((out->actions && !buf->actions) || (out->dones && !buf->dones))
        return fail(IQLH_EINVAL, "her_relabel: out.actions/out.dones need buf.actions/buf.dones");
    a.states = buf->states; a.next_states = buf->next_states; a.actions = buf->actions; a.dones = buf->dones;
    a.episode_ends = buf->episode_ends; a.source_idx = source_idx; a.d_step = d_step;
    a.donor_out = out->donor_idx; a.out_states = out->states; a.out_next_states = out->next_states;
    a.out_actions = out->actions; a.out_rewards = out->rewards; a.out_dones = out->dones; a.flags = out->d_flags;
    a.out_isw = out->is_weights;
    a.buffer_size = buf->buffer_size; a.out_ld = out->states_ld; a.seed = seed;
    a.num_episodes = buf->num_episodes;
    a.S = cfg->state_dim; a.G = cfg->goal_dim; a.strategy = cfg->strategy;
    a.out_bf16 = out->states_dtype == IQLH_BF16;
    a.threshold = cfg->goal_threshold; a.reward_hit = cfg->reward_hit; a.reward_miss = cfg->reward_miss;
    return IQLH_OK;
}

int her_relabel(const her_config* cfg, const her_buffer* buf, const int32_t* source_idx, int32_t n,
                uint64_t seed, const int64_t* d_step, const her_out* out, void* stream) {
    HerArgs a;
    int rc = make_her_args(cfg, buf, source_idx, n, seed, d_step, out, &a);
    if (rc || n == 0) return rc;
    hipError_t e = launch_her_relabel(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "her_relabel launch");
    return IQLH_OK;
}

int grad_budget_workspace_bytes(int64_t n, int32_t num_sources, size_t* bytes) {
    if (!bytes) return fail(IQLH_EINVAL, "bytes is NULL");
    if (n < 1) return fail(IQLH_EINVAL, "n must be >= 1");
    if (num_sources < 1 || num_sources > kMaxSources)
        return fail(IQLH_EINVAL, "num_sources must be in [1, %d]", kMaxSources);
    const int nb = budget_num_blocks(n);
    // [k][nb] source partials, [nb] combined partials, 2 Adam bias corrections
    *bytes = sizeof(float) * ((size_t)(num_sources + 1) * nb + 2);
    return IQLH_OK;
}

static int make_budget_args(float* grad_buf, const float* const* sources, const float* fractions,
                            const float* alphas, int32_t num_sources, int64_t n, float max_grad_norm,
                            float* out_norms, const iqlh_adam* adam, void* workspace, size_t workspace_bytes,
                            BudgetArgs* bp) {
    size_t need = 0;
    int rc = grad_budget_workspace_bytes(n, num_sources, &need);
    if (rc) return rc;
    if (!grad_buf || !sources || !fractions || !alphas || !workspace)
        return fail(IQLH_EINVAL, "grad_budget_accumulate: NULL argument");
    if (workspace_bytes < need) return fail(IQLH_EINVAL, "workspace too small: %zu < %zu", workspace_bytes, need);
    if (!(max_grad_norm > 0.f) || !std::isfinite(max_grad_norm))
        return fail(IQLH_EINVAL, "max_grad_norm must be finite and > 0");
    BudgetArgs& b = *bp;
    std::memset(&b, 0, sizeof(b));
    SourceSet& s = b.s;
    s.k = num_sources;
    for (int j = 0; j < num_sources; ++j) {
        if (!sources[j]) return fail(IQLH_EINVAL, "sources[%d] is NULL", j);
        if (!(fractions[j] >= 0.f) || !std::isfinite(fractions[j]))
            return fail(IQLH_EINVAL, "fractions[%d] must be finite and >= 0", j);
        if (!std::isfinite(alphas[j])) return fail(IQLH_EINVAL, "alphas[%d] must be finite", j);
        s.ptr[j] = sources[j];
        s.frac[j] = fractions[j];
        s.alpha[j] = alphas[j];
    }
    if (adam) {
        if (!adam->params || !adam->m || !adam->v || !adam->t)
            return fail(IQLH_EINVAL, "adam: params, m, v and t must be non-NULL");
        if (!(adam->beta1 >= 0.f && adam->beta1 < 1.f) || !(adam->beta2 >= 0.f && adam->beta2 < 1.f))
            return fail(IQLH_EINVAL, "adam: beta1 and beta2 must be in [0, 1)");
        if (!finite_pos(adam->eps) || !std::isfinite(adam->lr) || !(adam->lr >= 0.f))
            return fail(IQLH_EINVAL, "adam: bad eps or lr");
        if (!(adam->max_grad_norm > 0.f)) return fail(IQLH_EINVAL, "adam: max_grad_norm must be > 0");
        b.hp = AdamHyper{adam->lr, adam->beta1, adam->beta2, adam->eps, adam->weight_decay, adam->max_grad_norm,
                         adam->weight_clamp_max_abs};
        b.params = adam->params;
        b.m = adam->m;
        b.v = adam->v;
        b.t = adam->t;
        b.flags = adam->d_flags;
    }
    b.n = n;
    b.mgn = max_grad_norm;
    b.grad = grad_buf;
    b.out_norms = out_norms;
    b.work = (float*)workspace;
    return IQLH_OK;
}

int grad_budget_accumulate(float* grad_buf, const float* const* sources, const float* fractions,
                           const float* alphas, int32_t num_sources, int64_t n, float max_grad_norm,
                           float* out_norms, const iqlh_adam* adam, void* workspace, size_t workspace_bytes,
                           void* stream) {
    BudgetArgs b;
    int rc = make_budget_args(grad_buf, sources, fractions, alphas, num_sources, n, max_grad_norm, out_norms,
                              adam, workspace, workspace_bytes, &b);
    if (rc) return rc;
    hipError_t e = launch_budget(b.grad, b.s, b.n, b.mgn, b.out_norms, b.params, b.m, b.v, b.t, b.flags,
                                 b.params ? &b.hp : nullptr, b.work, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "grad_budget_accumulate launch");
    return IQLH_OK;
}

int grad_budget_accumulate_noalloc(float* grad_buf, const float* const* sources, const float* fractions,
                                   const float* alphas, int32_t num_sources, int64_t n, float max_grad_norm,
                                   float* out_norms, const iqlh_adam* adam, void* stream) {
    size_t need = 0;
    int rc = grad_budget_workspace_bytes(n, num_sources, &need);
    if (rc) return rc;
    if (need > budget_scratch_bytes())
        return fail(IQLH_EINVAL, "grad_budget_accumulate_noalloc: workspace of %zu bytes exceeds the %zu-byte scratch",
                    need, budget_scratch_bytes());
    // every argument is checked before the first HIP call (the scratch
    // address is filled in afterwards)
    BudgetArgs b;
    static char placeholder;
    rc = make_budget_args(grad_buf, sources, fractions, alphas, num_sources, n, max_grad_norm, out_norms, adam,
                          &placeholder, budget_scratch_bytes(), &b);
    if (rc) return rc;
    hipError_t e = budget_scratch_ptr(&b.work);
    if (e != hipSuccess) return hip_fail(e, "grad_budget_accumulate_noalloc: scratch address");
    e = launch_budget(b.grad, b.s, b.n, b.mgn, b.out_norms, b.params, b.m, b.v, b.t, b.flags,
                      b.params ? &b.hp : nullptr, b.work, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "grad_budget_accumulate_noalloc launch");
    return IQLH_OK;
}

struct AuxPlan {
    HerArgs ha;
    BudgetArgs ba;
    bool her, budget;
};

static int plan_aux_step(iql_handle h, const iqlh_her_step* her, const void* states, const float* q_taken,
                         int32_t batch, const float* q_all, int32_t num_actions, float beta, const float* out_pi,
                         const float* out_v, const iqlh_budget_step* budget, AuxPlan* p) {
    int rc = check_step_args(h, states, q_taken, batch);
    if (rc) return rc;
    if (q_all) {
        rc = check_policy_args(q_all, num_actions, beta, out_pi, out_v);
        if (rc) return rc;
    }
    p->her = her != nullptr;
    p->budget = budget != nullptr;
    if (her) {
        rc = make_her_args(her->cfg, her->buf, her->source_idx, her->n, her->seed, h->buf.step, her->out, &p->ha);
        if (rc) return rc;
    }
    if (budget) {
        rc = make_budget_args(budget->grad_buf, budget->sources, budget->fractions, budget->alphas,
                              budget->num_sources, budget->n, budget->max_grad_norm, budget->out_norms,
                              budget->adam, budget->workspace, budget->workspace_bytes, &p->ba);
        if (rc) return rc;
    }
    return IQLH_OK;
}

int iql_aux_step(iql_handle h, const iqlh_her_step* her, const void* states, const float* q_taken,
                 int32_t batch, const float* q_all, int32_t num_actions, float beta, float* out_pi,
                 float* out_v, float* out_loss, float* out_grad_norm, const iqlh_budget_step* budget,
                 void* stream) {
    AuxPlan p;
    int rc = plan_aux_step(h, her, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v, budget, &p);
    if (rc) return rc;
    hipError_t e = launch_aux_step(h->dims, h->buf, adam_hyper(h), h->cfg.tau, p.her ? &p.ha : nullptr,
                                   states, h->cfg.states_ld, q_taken, batch, q_all, num_actions, beta, out_pi,
                                   out_v, out_loss, out_grad_norm, p.budget ? &p.ba : nullptr, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "iql_aux_step launch");
    return IQLH_OK;
}

int iql_time_aux_step(iql_handle h, const iqlh_her_step* her, const void* states, const float* q_taken,
                      int32_t batch, const float* q_all, int32_t num_actions, float beta, float* out_pi,
                      float* out_v, float* out_loss, float* out_grad_norm, const iqlh_budget_step* budget,
                      int32_t reps, float* out_avg_us, void* stream) {
    AuxPlan p;
    int rc = plan_aux_step(h, her, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v, budget, &p);
    if (rc) return rc;
    if (reps < 1 || !out_avg_us) return fail(IQLH_EINVAL, "reps must be >= 1 and out_avg_us non-NULL");
    hipEvent_t ev[8] = {};
    hipError_t e = hipSuccess;
    for (int i = 0; i < 8 && e == hipSuccess; ++i) e = hipEventCreate(&ev[i]);
    double total[4] = {0.0, 0.0, 0.0, 0.0};
    for (int r = 0; r < reps && e == hipSuccess; ++r) {
        bool ran_a = false;
        e = launch_aux_step(h->dims, h->buf, adam_hyper(h), h->cfg.tau, p.her ? &p.ha : nullptr, states,
                            h->cfg.states_ld, q_taken, batch, q_all, num_actions, beta, out_pi, out_v, out_loss,
                            out_grad_norm, p.budget ? &p.ba : nullptr, (hipStream_t)stream, ev, &ran_a);
        if (e == hipSuccess) e = hipEventSynchronize(ev[7]);
        for (int k = ran_a ? 0 : 1; k < 4 && e == hipSuccess; ++k) {
            float ms = 0.f;
            e = hipEventElapsedTime(&ms, ev[2 * k], ev[2 * k + 1]);
            total[k] += ms;
        }
    }
    for (int i = 0; i < 8; ++i)
        if (ev[i]) (void)hipEventDestroy(ev[i]);
    if (e != hipSuccess) return hip_fail(e, "iql_time_aux_step");
    for (int k = 0; k < 4; ++k) out_avg_us[k] = (float)(total[k] * 1000.0 / reps);
    return IQLH_OK;
}

int iql_aux_step_phase_stamps(iql_handle h, const iqlh_her_step* her, const void* states, const float* q_taken,
                              int32_t batch, const float* q_all, int32_t num_actions, float beta, float* out_pi,
                              float* out_v, float* out_loss, float* out_grad_norm, const iqlh_budget_step* budget,
                              uint64_t* d_stamps, int32_t stamps_len, void* stream) {
    AuxPlan p;
    int rc = plan_aux_step(h, her, states, q_taken, batch, q_all, num_actions, beta, out_pi, out_v, budget, &p);
    if (rc) return rc;
    if (!d_stamps) return fail(IQLH_EINVAL, "iql_aux_step_phase_stamps: d_stamps is NULL");
    if (!iql_runs_fused16w(h->dims))
        return fail(IQLH_ESHAPE, "iql_aux_step_phase_stamps: phase ends are recorded by the bf16 hidden-128 kernel only");
    const int64_t need = (int64_t)h->dims.G * ((batch + 127) / 128) * kPhaseStamps;
    if (stamps_len < need)
        return fail(IQLH_EINVAL, "iql_aux_step_phase_stamps: stamps_len %d < %lld", stamps_len, (long long)need);
    hipError_t e = launch_aux_step(h->dims, h->buf, adam_hyper(h), h->cfg.tau, p.her ? &p.ha : nullptr, states,
                                   h->cfg.states_ld, q_taken, batch, q_all, num_actions, beta, out_pi, out_v,
                                   out_loss, out_grad_norm, p.budget ? &p.ba : nullptr, (hipStream_t)stream, nullptr,
                                   nullptr, d_stamps);
    if (e != hipSuccess) return hip_fail(e, "iql_aux_step_phase_stamps launch");
    return IQLH_OK;
}

}  // extern "C"
