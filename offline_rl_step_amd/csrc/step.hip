// The whole auxiliary step in four launches.  The pages run HER, the IQL
// update and the budgeted accumulation as separate kernels ("GPU IQL + HER
// Porting Plan", sections "Phase 3: Combined IQL + HER" and "How HER
// Interacts with GPU PER"; "Gradient Stability -- Proper Multi-Task Gradient
// Isolation + Full Spectral Norm", section "Task 1"); HER and the IQL value
// net share no state beyond the relabelled rows, and the budgeted
// accumulation touches neither.  Each small pass is too short to cover a
// launch, so here
// independent passes share a launch, each taking a contiguous range of its
// blocks (a block-uniform branch, no divergence inside a wave):
//   A  HER rows                 | budget: per-source sums of squares
//   B  fused V forward/backward and advantage-weighted policy (with the 16-wave
//      kernel also the HER rows that form the batch tail from a 128-row
//      boundary and the budget norms, so that A is not launched)
//   C  IQL: fixed-order sum of the workgroup partials | budget: clip + SAXPY |
//      the step counts and Adam bias corrections of both updates
//   D  IQL: clip + Adam + shadows | budget: clip + Adam (or the norm only)
// Results are bit-for-bit those of the separate launches: every block runs
// the same block function with the same block index and count.
#include <hip/hip_ext.h>

#include "budget_block.hpp"
#include "her_block.hpp"
#include "iql_update.hpp"
#include "launch.hpp"

namespace iqlh {

__global__ __launch_bounds__(256) void step_her_norms_kernel(HerArgs her, int her_blocks, NormsArgs np) {
    const int bx = blockIdx.x;
    if (bx < her_blocks) her_block(her, bx);
    else norms_block(np.s, np.n, np.vec, np.partials, bx - her_blocks, np.nb);
}

struct ReducePart {
    const float* part;
    const float* loss_part;
    float* grad;
    float* sq_part;
    int32_t* tcount;
    int64_t* step;
    float* bc;
    float* out_loss;
    int32_t* flags;
    int64_t P, Pp;
    float invB, beta1, beta2;
    int nwg, nloss, rb, G;
};
struct SaxpyPart {
    SourceSet s;
    int64_t n;
    const float* partials;
    float* grad;
    float* gpart;
    float* out_norms;
    int32_t* adam_t;  // null: no Adam update, no counter block
    float* bc;
    float mgn, beta1, beta2;
    int vec, nb;
};

// Blocks: the budget's SAXPY blocks first (their chain of dependent loads is
// longer than the reduction's streaming, and blocks are dispatched in order),
// the reduction's, one counter block per trainer, then the budget's counter
// block when it updates with Adam.
__global__ __launch_bounds__(256) void step_reduce_saxpy_kernel(ReducePart r, SaxpyPart x) {
    const int bx = blockIdx.x, nr = r.rb * r.G;
    if (bx < x.nb) {
        saxpy_block(x.s, x.n, x.vec, x.mgn, x.partials, x.grad, x.gpart, x.out_norms, bx, x.nb);
    } else if (bx < x.nb + nr) {
        const int br = bx - x.nb;
        iql_reduce_block(r.part, r.loss_part, r.nwg, r.nloss, r.P, r.Pp, r.invB, r.grad, r.sq_part, r.rb,
                         r.out_loss, r.flags, br % r.rb, br / r.rb);
    } else if (bx < x.nb + nr + r.G) {
        iql_count_block(r.tcount, r.step, r.bc, r.beta1, r.beta2, bx - x.nb - nr);
    } else {
        adam_count_block(x.adam_t, x.bc, x.beta1, x.beta2);
    }
}

struct FlatPart {
    float* params;  // null: the combined norm only (one block)
    float* grad;
    float* m;
    float* v;
    const float* bc;
    const float* gpart;
    float* out_norm;
    int32_t* flags;
    AdamHyper hp;
    int64_t n;
    int vec, nb;
};

template <typename T>
__global__ __launch_bounds__(256) void step_adam_kernel(IqlDims d, IqlBuffers b, AdamHyper hp,
                                                        float* __restrict__ out_gnorm, int rb, int ab,
                                                        FlatPart f) {
    const int bx = blockIdx.x, na = ab * d.G;
    if (bx < na) {
        iql_adam_block<T>(d, b, hp, out_gnorm, rb, bx % ab, bx / ab, ab);
    } else if (f.params) {
        adam_flat_block(f.params, f.grad, f.m, f.v, f.bc, f.gpart, f.nb, f.n, f.vec, f.hp, f.out_norm, f.flags,
                        bx - na, f.nb);
    } else {
        norm_finalize_block(f.gpart, f.nb, f.out_norm);
    }
}

static bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// A launch of 256-thread blocks, with dispatch events (kernel time only) when
// the caller times the step.
#define STEP_LAUNCH(kern, blocks, evp, ...)                                                               \
    do {                                                                                                  \
        if (evp)                                                                                          \
            hipExtLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, stream, (evp)[0], (evp)[1], 0, __VA_ARGS__); \
        else                                                                                              \
            hipLaunchKernelGGL(kern, dim3(blocks), dim3(256), 0, stream, __VA_ARGS__);                    \
    } while (0)

hipError_t launch_aux_step(const IqlDims& d, const IqlBuffers& b, const AdamHyper& hp, const float* tau,
                           const HerArgs* her, const void* states, int64_t ld, const float* q, int B,
                           const float* q_all, int A, float beta, float* out_pi, float* out_v,
                           float* out_loss, float* out_gnorm, const BudgetArgs* bud, hipStream_t stream,
                           hipEvent_t* ev, bool* ran_a, uint64_t* stamps) {
    int nwg, nloss;
    if (!iql_partial_counts(d, B, &nwg, &nloss)) return hipErrorInvalidValue;
    const int nb = bud ? budget_num_blocks(bud->n) : 0;
    int vec = 0;
    float* partials = nullptr;
    float* gpart = nullptr;
    float* bud_bc = nullptr;
    if (bud) {
        partials = bud->work;
        gpart = bud->work + (int64_t)bud->s.k * nb;
        bud_bc = gpart + nb;
        vec = al16(bud->grad);
        for (int j = 0; j < bud->s.k; ++j) vec = vec && al16(bud->s.ptr[j]);
    }
    const bool flat_adam = bud && bud->params;

    // HER rows that are the tail of the batch, and the budget's pass 1, move
    // into the forward/backward launch when its kernel can host them
    const bool her_in_b = her && her->n > 0 && iql_fused_her_ok(d, *her, states, ld, B);
    const bool norms_in_b = bud && iql_fused_norms_ok(d, B, her_in_b ? her->n : 0, nb);
    NormsArgs np{};
    if (bud) np = NormsArgs{bud->s, bud->n, partials, vec, nb};

    // A: HER + budget norms (what launch B does not host)
    const int her_blocks = (her && her->n > 0 && !her_in_b) ? (her->n + kHerRows - 1) / kHerRows : 0;
    const int nb_a = norms_in_b ? 0 : nb;
    if (her_blocks + nb_a > 0) {
        HerArgs ha{};
        if (her_blocks) ha = *her;
        NormsArgs npa{};
        if (nb_a) npa = np;
        STEP_LAUNCH(step_her_norms_kernel, her_blocks + nb_a, ev, ha, her_blocks, npa);
    }
    if (ran_a) *ran_a = her_blocks + nb_a > 0;

    // B: fused forward/backward (+ policy, HER rows, budget norms)
    hipError_t e;
    const bool fused_pi = q_all && out_pi && iql_policy_in_launch(d, B, A, q_all, out_pi);
    hipEvent_t e0 = ev ? ev[2] : nullptr, e1 = ev ? ev[3] : nullptr;
    const HerArgs* hb = her_in_b ? her : nullptr;
    const NormsArgs* nbp = norms_in_b ? &np : nullptr;
    if (fused_pi) {
        e = launch_iql_fwd_bwd(d, b, tau, states, ld, q, B, out_v, stream, e0, e1, q_all, A, beta, out_pi, hb, nbp,
                               stamps);
    } else {
        e = launch_iql_fwd_bwd(d, b, tau, states, ld, q, B, out_v, stream, e0, e1, nullptr, 0, 0.f, nullptr, hb,
                               nbp, stamps);
        if (e == hipSuccess && q_all) e = launch_aw_policy(q_all, out_v, d.G, B, A, beta, out_pi, stream);
    }
    if (e != hipSuccess) return e;

    // C: reduce + SAXPY
    const int rb = iql_reduce_blocks(d.P);
    ReducePart rp{b.part, b.loss_part, b.grad, b.sq_part, b.t, b.step, b.bc, out_loss, b.flags, d.P, d.Pp,
                  1.f / (float)B, hp.beta1, hp.beta2, nwg, nloss, rb, d.G};
    SaxpyPart sp{};
    if (bud)
        sp = SaxpyPart{bud->s, bud->n, partials, bud->grad, gpart, bud->out_norms,
                       flat_adam ? bud->t : (int32_t*)nullptr, bud_bc, bud->mgn,
                       flat_adam ? bud->hp.beta1 : 0.f, flat_adam ? bud->hp.beta2 : 0.f, vec, nb};
    STEP_LAUNCH(step_reduce_saxpy_kernel, nb + rb * d.G + d.G + (flat_adam ? 1 : 0), ev ? ev + 4 : nullptr, rp, sp);

    // D: both Adam updates
    const int ab = iql_adam_blocks(d.P);
    FlatPart fp{};
    int extra = 0;
    if (flat_adam) {
        const int fvec = al16(bud->grad) && al16(bud->params) && al16(bud->m) && al16(bud->v);
        fp = FlatPart{bud->params, bud->grad, bud->m, bud->v, bud_bc, gpart,
                      bud->out_norms ? bud->out_norms + bud->s.k : nullptr, bud->flags, bud->hp, bud->n, fvec, nb};
        extra = nb;
    } else if (bud && bud->out_norms) {
        fp.gpart = gpart;
        fp.nb = nb;
        fp.out_norm = bud->out_norms + bud->s.k;
        extra = 1;
    }
    if (d.dtype == 1)
        STEP_LAUNCH((step_adam_kernel<uint16_t>), ab * d.G + extra, ev ? ev + 6 : nullptr, d, b, hp, out_gnorm, rb,
                    ab, fp);
    else
        STEP_LAUNCH((step_adam_kernel<float>), ab * d.G + extra, ev ? ev + 6 : nullptr, d, b, hp, out_gnorm, rb, ab,
                    fp);
    return hipGetLastError();
}

}  // namespace iqlh
