// Budgeted clipped-SAXPY gradient accumulation and flat clipped Adam, gfx950.
//
// Follows "Gradient Stability -- Proper Multi-Task Gradient Isolation + Full
// Spectral Norm", section "Design -- Why the current per-component clipping is
// wrong" / "Proper design" (source k owns the fraction f_k of max_grad_norm;
// each source is clipped to its own budget in isolation and added with its
// scale; Adam keeps its safety clip at max_grad_norm) and "Task 1" (clipped
// SAXPY grad += alpha * clip(scratch, budget) with the scratch buffer's own
// norm).  The Adam step follows "DQN Backward-Path NaN Audit -- SP1 Phase A",
// section on iqn_adam_kernel.
//
// HBM-bound, three launches, all reductions in a fixed order (no float
// atomics, bitwise reproducible):
//   1. norms : one pass reads all k sources, per-block partial sums of squares;
//   2. saxpy : every block folds the partials into the k clip scales (same
//              order in every block), writes grad = sum_k alpha_k c_k s_k and a
//              per-block partial of ||grad||^2;
//   3. adam  : every block folds the grad partials into the combined norm and
//              applies the clipped Adam update, zeroing grad.
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

constexpr int kBT = 256;          // threads per block; each thread owns float4 quads
constexpr int kMaxBlocks = 2048;

int budget_num_blocks(int64_t n) {
    const int64_t quads = (n + 3) / 4;
    int64_t nb = (quads + kBT - 1) / kBT;
    if (nb < 1) nb = 1;
    if (nb > kMaxBlocks) nb = kMaxBlocks;
    return (int)nb;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Quad qd covers elements 4qd .. 4qd+3 (those < n); 16-byte loads when every
// pointer involved is 16-byte aligned.
IQLH_DEV f32x4 ld4(const float* __restrict__ p, int64_t i, int64_t n, bool vec) {
    if (vec && i + 3 < n) return *(const f32x4*)(p + i);
    f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (i + e < n) r[e] = p[i + e];
    return r;
}
IQLH_DEV void st4(float* __restrict__ p, int64_t i, int64_t n, bool vec, f32x4 x) {
    if (vec && i + 3 < n) {
        *(f32x4*)(p + i) = x;
        return;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (i + e < n) p[i + e] = x[e];
}

__global__ __launch_bounds__(kBT) void budget_norms_kernel(SourceSet s, int64_t n, int vec,
                                                             float* __restrict__ partials) {
    __shared__ float red[kBT / kWave];
    float acc[kMaxSources];
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j) acc[j] = 0.f;
    const int64_t quads = (n + 3) / 4, stride = (int64_t)gridDim.x * kBT;
    for (int64_t qd = (int64_t)blockIdx.x * kBT + threadIdx.x; qd < quads; qd += stride) {
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j) {
            if (j < s.k) {
                const f32x4 x = ld4(s.ptr[j], 4 * qd, n, vec);
                acc[j] = fmaf(x.x, x.x, fmaf(x.y, x.y, fmaf(x.z, x.z, fmaf(x.w, x.w, acc[j]))));
            }
        }
    }
    for (int j = 0; j < s.k; ++j) {
        const float t = block_sum<kBT>(acc[j], red);
        if (threadIdx.x == 0) partials[(int64_t)j * gridDim.x + blockIdx.x] = t;
    }
}

// Fixed-order fold of nb partials by one block; every block gets the same value.
IQLH_DEV float fold_partials(const float* __restrict__ p, int nb, float* red) {
    float a = 0.f;
    for (int i = threadIdx.x; i < nb; i += kBT) a += p[i];
    return block_sum<kBT>(a, red);
}

// Per-source budget clip, the page's rule taken literally (a NaN norm leaves
// the source unscaled, an infinite one scales it by 0).
IQLH_DEV float budget_scale(float norm, float budget) {
    return (norm > budget && norm > 0.f) ? budget / norm : 1.f;
}

// Adam's clip: a non-finite norm poisons every clipped element so the finite
// guard skips the whole update.
IQLH_DEV float adam_clip(float norm, float max_norm) {
    if (!isfinite(norm)) return __int_as_float(0x7FC00000);
    return (norm > max_norm && norm > 0.f) ? max_norm / norm : 1.f;
}

__global__ __launch_bounds__(kBT) void budget_saxpy_kernel(SourceSet s, int64_t n, int vec, float mgn,
                                                            const float* __restrict__ partials,
                                                            float* __restrict__ grad,
                                                            float* __restrict__ gpart,
                                                            float* __restrict__ out_norms,
                                                            int32_t* __restrict__ adam_t) {
    __shared__ float red[kBT / kWave];
    __shared__ float coef[kMaxSources];
    const int nb = gridDim.x;
    // this thread's first quad of every source does not depend on the clip
    // scales: load it before folding the norm partials
    const int64_t quads = (n + 3) / 4, stride = (int64_t)nb * kBT;
    const int64_t q0 = (int64_t)blockIdx.x * kBT + threadIdx.x;
    f32x4 pre[kMaxSources];
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j)
        pre[j] = (j < s.k && q0 < quads) ? ld4(s.ptr[j], 4 * q0, n, vec) : f32x4{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < s.k; ++j) {
        const float sq = fold_partials(partials + (int64_t)j * nb, nb, red);
        if (threadIdx.x == 0) {
            const float nrm = sqrtf(sq);
            coef[j] = s.alpha[j] * budget_scale(nrm, s.frac[j] * mgn);
            if (blockIdx.x == 0 && out_norms) out_norms[j] = nrm;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0 && adam_t) *adam_t += 1;
    __syncthreads();
    float c[kMaxSources];
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j) c[j] = j < s.k ? coef[j] : 0.f;
    float acc = 0.f;
    for (int64_t qd = q0; qd < quads; qd += stride) {
        f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j)
            if (j < s.k) g += c[j] * (qd == q0 ? pre[j] : ld4(s.ptr[j], 4 * qd, n, vec));
        st4(grad, 4 * qd, n, vec, g);
        acc = fmaf(g.x, g.x, fmaf(g.y, g.y, fmaf(g.z, g.z, fmaf(g.w, g.w, acc))));
    }
    const float t = block_sum<kBT>(acc, red);
    if (threadIdx.x == 0) gpart[blockIdx.x] = t;
}

__global__ __launch_bounds__(kBT) void norm_finalize_kernel(const float* __restrict__ p, int nb,
                                                             float* __restrict__ out) {
    __shared__ float red[kBT / kWave];
    const float sq = fold_partials(p, nb, red);
    if (threadIdx.x == 0) *out = sqrtf(sq);
}

__global__ __launch_bounds__(kBT) void adam_flat_kernel(float* __restrict__ params,
                                                         float* __restrict__ grad,
                                                         float* __restrict__ m,
                                                         float* __restrict__ v,
                                                         const int32_t* __restrict__ tptr,
                                                         const float* __restrict__ sq_part, int nb,
                                                         int64_t n, int vec, AdamHyper hp,
                                                         float* __restrict__ out_norm,
                                                         int32_t* __restrict__ flags) {
    __shared__ float red[kBT / kWave];
    const int64_t quads = (n + 3) / 4, stride = (int64_t)gridDim.x * kBT;
    const int64_t q0 = (int64_t)blockIdx.x * kBT + threadIdx.x;
    // first quad's state loaded before the norm fold (independent of it)
    f32x4 pg = {0.f, 0.f, 0.f, 0.f}, pm = pg, pv = pg, pp = pg;
    if (q0 < quads) {
        pg = ld4(grad, 4 * q0, n, vec);
        pm = ld4(m, 4 * q0, n, vec);
        pv = ld4(v, 4 * q0, n, vec);
        pp = ld4(params, 4 * q0, n, vec);
    }
    const float sq = fold_partials(sq_part, nb, red);
    const float nrm = sqrtf(sq);
    if (blockIdx.x == 0 && threadIdx.x == 0 && out_norm) *out_norm = nrm;
    const float c = adam_clip(nrm, hp.max_grad_norm);
    const float tt = (float)(*tptr);
    const float bc1 = 1.f - powf(hp.beta1, tt);
    const float bc2 = 1.f - powf(hp.beta2, tt);
    const float decay = 1.f - hp.lr * hp.weight_decay;
    bool bad = false;
    for (int64_t qd = q0; qd < quads; qd += stride) {
        const int64_t i = 4 * qd;
        const bool first = qd == q0;
        const f32x4 g4 = (first ? pg : ld4(grad, i, n, vec)) * c;
        f32x4 m4 = first ? pm : ld4(m, i, n, vec), v4 = first ? pv : ld4(v, i, n, vec);
        f32x4 p4 = first ? pp : ld4(params, i, n, vec);
        st4(grad, i, n, vec, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float g = g4[e];
            if (!isfinite(g)) { bad |= (i + e < n); continue; }
            const float mi = hp.beta1 * m4[e] + (1.f - hp.beta1) * g;
            const float vi = hp.beta2 * v4[e] + (1.f - hp.beta2) * g * g;
            const float mh = mi / bc1, vh = vi / bc2;
            float p = p4[e];
            if (hp.weight_decay != 0.f) p *= decay;
            p -= hp.lr * mh / (sqrtf(vh) + hp.eps);
            if (hp.clamp > 0.f) p = fminf(fmaxf(p, -hp.clamp), hp.clamp);
            p4[e] = p;
            m4[e] = mi;
            v4[e] = vi;
        }
        st4(params, i, n, vec, p4);
        st4(m, i, n, vec, m4);
        st4(v, i, n, vec, v4);
    }
    if (bad) set_flag(flags, 0x1);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

hipError_t launch_adam_flat(float* params, float* grad, float* m, float* v, const int32_t* t,
                            const float* sq_partials, int nb, int64_t n, const AdamHyper& hp,
                            float* out_norm, int32_t* flags, hipStream_t stream) {
    const int blocks = budget_num_blocks(n);
    const int vec = aligned16(params) && aligned16(grad) && aligned16(m) && aligned16(v);
    hipLaunchKernelGGL(adam_flat_kernel, dim3(blocks), dim3(kBT), 0, stream, params, grad, m, v, t,
                       sq_partials, nb, n, vec, hp, out_norm, flags);
    return hipGetLastError();
}

hipError_t launch_budget(float* grad, const SourceSet& s, int64_t n, float mgn, float* out_norms,
                         float* params, float* m, float* v, int32_t* t, int32_t* flags,
                         const AdamHyper* hp, float* work, hipStream_t stream) {
    const int nb = budget_num_blocks(n);
    float* partials = work;
    float* gpart = work + (int64_t)s.k * nb;
    int vec = aligned16(grad);
    for (int j = 0; j < s.k; ++j) vec = vec && aligned16(s.ptr[j]);
    hipLaunchKernelGGL(budget_norms_kernel, dim3(nb), dim3(kBT), 0, stream, s, n, vec, partials);
    hipLaunchKernelGGL(budget_saxpy_kernel, dim3(nb), dim3(kBT), 0, stream, s, n, vec, mgn, partials,
                       grad, gpart, out_norms, hp ? t : (int32_t*)nullptr);
    if (hp) {
        float* comb = out_norms ? out_norms + s.k : nullptr;
        return launch_adam_flat(params, grad, m, v, t, gpart, nb, n, *hp, comb, flags, stream);
    }
    if (out_norms)
        hipLaunchKernelGGL(norm_finalize_kernel, dim3(1), dim3(kBT), 0, stream, gpart, nb,
                           out_norms + s.k);
    return hipGetLastError();
}

}  // namespace iqlh
