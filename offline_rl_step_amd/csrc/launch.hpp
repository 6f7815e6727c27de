// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iqlh {

// ------------------------------------------------------------------- HER
struct HerArgs {
    const float* states;
    const float* next_states;
    const int32_t* actions;
    const float* dones;
    const int32_t* episode_ends;
    const int32_t* source_idx;
    const int64_t* d_step;
    int32_t* donor_out;
    void* out_states;
    float* out_next_states;
    int32_t* out_actions;
    float* out_rewards;
    float* out_dones;
    float* out_isw;  // importance-sampling weights of the HER rows (1; 0 for a zeroed row) or null
    int32_t* flags;
    int64_t buffer_size;
    int64_t out_ld;
    uint64_t seed;
    int32_t num_episodes;
    int32_t n;
    int32_t S, G, strategy, out_bf16;
    float threshold, reward_hit, reward_miss;
};
hipError_t launch_her_relabel(const HerArgs& a, hipStream_t stream);

// ------------------------------------------------------------- AW policy
hipError_t launch_aw_policy(const float* q, const float* v, int G, int B, int A, float beta,
                            float* pi, hipStream_t stream);

// ---------------------------------------------------- gradient budget
constexpr int kMaxSources = 8;
struct SourceSet {
    const float* ptr[kMaxSources];
    float frac[kMaxSources];
    float alpha[kMaxSources];
    int32_t k;
};
// Pass 1 of the budgeted accumulation (per-source sums of squares, blocks
// 0 .. nb - 1 of 256 threads) run inside another launch.
struct NormsArgs {
    SourceSet s;
    int64_t n;
    float* partials;  // [k][nb]
    int vec, nb;
};
// Outputs of a forward-only pass: V and, with rewards, the bootstrap target
// r + gamma (1 - done) V.
struct ValueOut {
    float* v;           // [G][B]
    const float* rew;   // [B] or null: no target
    const float* done;  // [B] or null: no terminal rows
    float gamma;
    float* target;      // [G][B] (with rew)
};
__device__ __forceinline__ void write_value(const ValueOut& o, int g, int B, int b, float v) {
    const int64_t i = (int64_t)g * B + b;
    o.v[i] = v;
    if (o.target) o.target[i] = fmaf(o.gamma * (1.f - (o.done ? o.done[b] : 0.f)), v, o.rew[b]);
}

struct AdamHyper {
    float lr, beta1, beta2, eps, weight_decay, max_grad_norm, clamp;
    float ema;  // IQL trainers: Polyak weight of the target copy updated with the step, 0 = off
};
int budget_num_blocks(int64_t n);
// workspace floats: k * nb (source partials) + nb (combined partials)
hipError_t launch_budget(float* grad, const SourceSet& s, int64_t n, float mgn,
                         float* out_norms, float* params, float* m, float* v, int32_t* t,
                         int32_t* flags, const AdamHyper* hp, float* work, hipStream_t stream);

// The allocation-free entry point's workspace: a static device array of
// budget_scratch_bytes() bytes (enough for any n and k), addressed per device.
size_t budget_scratch_bytes();
hipError_t budget_scratch_ptr(float** out);

// Flat clipped Adam over n elements whose gradient L2 norm is the fixed-order
// sum of `nb` partial sums of squares.  Zeroes grad.  bc holds the bias
// corrections 1 - beta1^t, 1 - beta2^t of the already incremented step count
// t.  out_norm (nullable) receives the pre-clip norm.
hipError_t launch_adam_flat(float* params, float* grad, float* m, float* v, const float* bc,
                            const float* sq_partials, int nb, int64_t n, const AdamHyper& hp,
                            float* out_norm, int32_t* flags, hipStream_t stream);

// ------------------------------------------------------------------ IQL
struct IqlDims {
    int S, H, G, dtype;  // H: first hidden width; dtype: 0 f32, 1 bf16
    int H2;              // second hidden width (== H except on the layered path)
    int layered;         // 0: fused tile kernel; 1: layered GEMMs through HBM
    int big;             // with layered: the wide-hidden bf16 kernels (iql_big.hip)
    int S_pad;           // columns of the W1 shadow (multiple of 32)
    int64_t P;           // parameters per group
    int64_t Pp;          // row stride of the gradient partials (P rounded up to 128)
};
// Per-group device buffers, group stride = P (or the shadow sizes).
struct IqlBuffers {
    float* params;    // [G][P] fp32 master
    float* m;         // [G][P]
    float* v;         // [G][P]
    float* grad;      // [G][P]
    float* target;    // [G][P] Polyak (EMA) target copy of params
    int32_t* t;       // [G]
    float* bc;        // [G][2] Adam bias corrections 1 - beta1^t, 1 - beta2^t for the current t
    int64_t* step;    // [1]
    int32_t* flags;   // [1]
    void* w1s;        // [G][H][S_pad]   operand-typed shadow of W1 (zero padded)
    void* w2s;        // [G][H][H]       shadow of W2
    void* w2ts;       // [G][H][H]       shadow of W2 transposed
    float* part;      // [G][max_wg][Pp] per-workgroup gradient partials
    float* loss_part; // [G][max_wg]
    float* sq_part;   // [G][max_rb]     per-block sums of squares of grad
    int max_wg;
    int max_rb;
    // layered path only: activations [G][max_batch][H] and dv [G][max_batch]
    void* act_h1;
    float* act_z2;
    void* act_dz2;
    void* act_p2;
    void* act_dz1;
    float* act_dv;
    // wide-hidden path: per-128-sample-block sums of db2, dw3, db3, db1
    // [G][nblk][iql_big_spart_width(H)]
    float* big_spart;
};
bool iql_supported(int dtype, int S, int H);
int iql_tile_samples(int dtype, int S, int H);
int iql_reduce_blocks(int64_t P);
// Fused forward/backward: V(s) and the per-workgroup gradient partials.
// With out_pi non-null and iql_policy_in_launch(d, B, A, q_all, out_pi), the
// advantage-weighted policy of every group is computed in the same launch
// from this V (by the fused tile kernels, or by the spare workgroups of the
// wide-hidden weight-gradient kernel).
// With `her` (iql_fused_her_ok), the HER rows that form the batch tail from
// row her_row0 on are relabelled inside the launch instead of read from
// `states` (group 0 also writes every HER output); with `nrm`
// (iql_fused_norms_ok), the launch also runs the budget's pass 1.
hipError_t launch_iql_fwd_bwd(const IqlDims& d, const IqlBuffers& b, const float* tau,
                              const void* states, int64_t ld, const float* q, int B,
                              float* out_v, hipStream_t stream, hipEvent_t ev0 = nullptr,
                              hipEvent_t ev1 = nullptr, const float* q_all = nullptr, int A = 0,
                              float beta = 0.f, float* out_pi = nullptr, const HerArgs* her = nullptr,
                              const NormsArgs* nrm = nullptr, uint64_t* stamps = nullptr);
// Phase ends recorded per workgroup by the 16-wave kernel for measurement
// (launch_iql_fwd_bwd's `stamps`, [G][nwg][kPhaseStamps]): kernel start, the
// ends of the staging (S0), F1, F2 + V, loss / dz2, dW2 (+ W2^T, policy) and
// dh1 / dz1 phases, and the issue of the last dW1 partial stores.
constexpr int kPhaseStamps = 8;
// The forward/backward launch runs the 16-wave kernel (bf16, hidden 128,
// state <= 128), the one that can record phase ends.
bool iql_runs_fused16w(const IqlDims& d);
bool iql_fused_policy(const IqlDims& d, int A);
bool iql_policy_in_launch(const IqlDims& d, int B, int A, const void* q_all, const void* out_pi);
bool iql_fused_her_ok(const IqlDims& d, const HerArgs& her, const void* states, int64_t ld, int B);
bool iql_fused_norms_ok(const IqlDims& d, int B, int her_rows, int nb);
// Fixed-order reduction of the partials of a batch of B rows, clip, Adam.
hipError_t launch_iql_update(const IqlDims& d, const IqlBuffers& b, const AdamHyper& hp, int B,
                             float* out_loss, float* out_gnorm, hipStream_t stream);
int iql_s_pad(int dtype, int S, int H);
bool iql_layered_supported(int dtype, int S, int H);
int iql_layered_chunk();
hipError_t launch_iql_layered_fwd_bwd(const IqlDims& d, const IqlBuffers& b, const float* tau,
                                      const void* states, int64_t ld, const float* q, int B,
                                      float* out_v, hipStream_t stream);
bool iql_big_supported(int dtype, int S, int H);
int iql_big_blocks(int B);
int iql_big_max_chunks(int S, int H);
int iql_big_chunk(int S, int H, int G, int B);
int iql_big_spart_width(int H);
// The policy (out_pi non-null) runs in the weight-gradient launch's spare
// workgroups when iql_big_policy_ok; otherwise hipErrorInvalidValue.
bool iql_big_policy_ok(const IqlDims& d, int B, int A, const void* q_all, const void* out_pi);
hipError_t launch_iql_big_fwd_bwd(const IqlDims& d, const IqlBuffers& b, const float* tau, const void* states,
                                  int64_t ld, const float* q, int B, float* out_v, hipStream_t stream,
                                  const float* q_all = nullptr, int A = 0, float beta = 0.f,
                                  float* out_pi = nullptr);
hipError_t launch_iql_target_ema(const IqlDims& d, const IqlBuffers& b, float tau, hipStream_t stream);
hipError_t launch_iql_layered_forward(const IqlDims& d, const IqlBuffers& b, const void* states, int64_t ld,
                                      int B, const ValueOut& vo, hipStream_t stream);
hipError_t launch_iql_big_forward(const IqlDims& d, const IqlBuffers& b, const void* states, int64_t ld, int B,
                                  const ValueOut& vo, hipStream_t stream);
// V(s) of every group for B rows of `states` (compute dtype, row stride ld),
// and the bootstrap target when vo.rew is set; no loss, no gradients.
hipError_t launch_iql_forward_values(const IqlDims& d, const IqlBuffers& b, const void* states, int64_t ld, int B,
                                     const ValueOut& vo, hipStream_t stream);
// dst[r][c] = src[r][c] converted between f32 and the compute dtype (bf16 RNE)
hipError_t launch_convert_rows(const void* src, int src_dtype, int64_t src_ld, void* dst, int dst_dtype,
                               int64_t dst_ld, int rows, int cols, hipStream_t stream);
hipError_t launch_iql_refresh_shadows(const IqlDims& d, const IqlBuffers& b, hipStream_t stream);
// workgroup and loss partials that a batch of B rows leaves for the reduction
bool iql_partial_counts(const IqlDims& d, int B, int* nwg, int* nloss);
int iql_adam_blocks(int64_t P);

// ------------------------------------------------- prioritized sampling
size_t per_workspace_bytes_for(int64_t size);
hipError_t launch_per_sample(const float* p, int64_t size, int n, uint64_t seed, const int64_t* d_step, float beta,
                             int32_t* idx, float* w, int32_t* flags, void* workspace, hipStream_t stream);

// ------------------------------------------------- non-finite sentinel
constexpr int kSentinelSlots = 32;
constexpr int kSentinelPiece = 8192;  // elements per block
struct SentinelArgs {
    const float* ptr[kSentinelSlots];
    int64_t n[kSentinelSlots];
    int block0[kSentinelSlots + 1];  // first block of each slot
    int32_t* flags;                  // [nslots]
    uint32_t vec;                    // bit s: slot s is 16-byte aligned
    int nslots;
};
hipError_t launch_nonfinite_sentinel(const SentinelArgs& a, int blocks, hipStream_t stream);

// ------------------------------------------------------- whole step
// One pass of the hot path in four launches:
//   A  HER relabelling + budget source norms   (independent of each other)
//   B  fused V forward/backward (+ AW policy)   (reads the relabelled rows)
//   C  IQL partial reduction + budget SAXPY
//   D  IQL clipped Adam + budget clipped Adam (or the combined norm only)
// `her` and `budget` may be null (that part is skipped).
struct BudgetArgs {
    SourceSet s;
    int64_t n;
    float mgn;
    float* grad;
    float* out_norms;
    float* work;
    // flat Adam over grad (params null: accumulation only)
    float* params;
    float* m;
    float* v;
    int32_t* t;
    int32_t* flags;
    AdamHyper hp;
};
hipError_t launch_aux_step(const IqlDims& d, const IqlBuffers& b, const AdamHyper& hp, const float* tau,
                           const HerArgs* her, const void* states, int64_t ld, const float* q, int B,
                           const float* q_all, int A, float beta, float* out_pi, float* out_v,
                           float* out_loss, float* out_gnorm, const BudgetArgs* budget, hipStream_t stream,
                           hipEvent_t* ev = nullptr, bool* ran_a = nullptr, uint64_t* stamps = nullptr);
// ev (optional): 8 events, start/stop of launches A, B, C, D (A's are not
// recorded when A is not needed: its HER rows and budget norms both ride in
// B).  ran_a (optional) receives whether A was launched.

}  // namespace iqlh
