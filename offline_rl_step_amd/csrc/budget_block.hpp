// Block-level bodies of the gradient-budget passes and the flat clipped Adam,
// shared by their own launches and by the merged whole-step launches.  The
// method is described in budget.hip.  Every function takes its block index
// and the block count of its pass explicitly, so a merged launch can run it
// on any contiguous range of its blocks.
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

constexpr int kBT = 256;          // threads per block; each thread owns float4 quads
constexpr int kMaxBlocks = 2048;

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

// block_sum of k values per thread at once (one pair of barriers for all k);
// v[j] becomes the block sum of v[j], in block_sum's order.
IQLH_DEV void block_sum_k(float (&v)[kMaxSources], int k, float (*red)[kBT / kWave]) {
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j)
        if (j < k) v[j] = wave_sum(v[j]);
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j)
            if (j < k) red[j][w] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < kBT / kWave; ++i) t += j < k ? red[j][i] : 0.f;
        v[j] = t;
    }
}

// fold_partials of k consecutive sets of nb partials, all loads in flight
// together; out[j] equals fold_partials(p + j * nb, nb).
IQLH_DEV void fold_partials_k(const float* __restrict__ p, int nb, int k, float (&out)[kMaxSources],
                              float (*red)[kBT / kWave]) {
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j) out[j] = 0.f;
    for (int i = threadIdx.x; i < nb; i += kBT) {
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j)
            if (j < k) out[j] += p[(int64_t)j * nb + i];
    }
    block_sum_k(out, k, red);
}

// Thread t's share of block bx of nb of pass 1: the sums of squares of its
// quads of every source (the block then adds its threads with block_sum_k).
IQLH_DEV void norms_thread(const SourceSet& s, int64_t n, int vec, int bx, int nb, int t,
                           float (&acc)[kMaxSources]) {
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j) acc[j] = 0.f;
    const int64_t quads = (n + 3) / 4, stride = (int64_t)nb * kBT;
    for (int64_t qd = (int64_t)bx * kBT + t; qd < quads; qd += stride) {
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j) {
            if (j < s.k) {
                const f32x4 x = ld4(s.ptr[j], 4 * qd, n, vec);
                acc[j] = fmaf(x.x, x.x, fmaf(x.y, x.y, fmaf(x.z, x.z, fmaf(x.w, x.w, acc[j]))));
            }
        }
    }
}

// Pass 1 for block bx of nb: partial sums of squares of every source.
IQLH_DEV void norms_block(const SourceSet& s, int64_t n, int vec, float* __restrict__ partials, int bx,
                         int nb) {
    __shared__ float red[kMaxSources][kBT / kWave];
    float acc[kMaxSources];
    norms_thread(s, n, vec, bx, nb, threadIdx.x, acc);
    block_sum_k(acc, s.k, red);
    if (threadIdx.x == 0) {
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j)
            if (j < s.k) partials[(int64_t)j * nb + bx] = acc[j];
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

// Pass 2 for block bx of nb: clip scales, grad = sum_k c_k s_k, and the
// block's partial of ||grad||^2.
IQLH_DEV void saxpy_block(const SourceSet& s, int64_t n, int vec, float mgn, const float* __restrict__ partials,
                          float* __restrict__ grad, float* __restrict__ gpart, float* __restrict__ out_norms,
                          int32_t* __restrict__ adam_t, int bx, int nb) {
    __shared__ float red[kBT / kWave];
    __shared__ float redk[kMaxSources][kBT / kWave];
    // this thread's first quad of every source does not depend on the clip
    // scales: load it before folding the norm partials
    const int64_t quads = (n + 3) / 4, stride = (int64_t)nb * kBT;
    const int64_t q0 = (int64_t)bx * kBT + threadIdx.x;
    f32x4 pre[kMaxSources];
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j)
        pre[j] = (j < s.k && q0 < quads) ? ld4(s.ptr[j], 4 * q0, n, vec) : f32x4{0.f, 0.f, 0.f, 0.f};
    // every thread folds every source's partials (same value in all threads
    // and blocks) and derives the clip scales itself
    float c[kMaxSources];
    fold_partials_k(partials, nb, s.k, c, redk);
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j) {
        if (j < s.k) {
            const float nrm = sqrtf(c[j]);
            if (bx == 0 && threadIdx.x == 0 && out_norms) out_norms[j] = nrm;
            c[j] = s.alpha[j] * budget_scale(nrm, s.frac[j] * mgn);
        } else {
            c[j] = 0.f;
        }
    }
    if (bx == 0 && threadIdx.x == 0 && adam_t) *adam_t += 1;
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
    if (threadIdx.x == 0) gpart[bx] = t;
}

IQLH_DEV void norm_finalize_block(const float* __restrict__ p, int nb, float* __restrict__ out) {
    __shared__ float red[kBT / kWave];
    const float sq = fold_partials(p, nb, red);
    if (threadIdx.x == 0) *out = sqrtf(sq);
}

// Pass 3 for block bx of nbx: folds the nb grad partials into the norm and
// applies the clipped Adam update to the block's quads, zeroing grad.
IQLH_DEV void adam_flat_block(float* __restrict__ params, float* __restrict__ grad, float* __restrict__ m,
                              float* __restrict__ v, const int32_t* __restrict__ tptr,
                              const float* __restrict__ sq_part, int nb, int64_t n, int vec,
                              const AdamHyper& hp, float* __restrict__ out_norm, int32_t* __restrict__ flags,
                              int bx, int nbx) {
    // no contraction: the same roundings in every kernel this is inlined into
#pragma clang fp contract(off)
    __shared__ float red[kBT / kWave];
    const int64_t quads = (n + 3) / 4, stride = (int64_t)nbx * kBT;
    const int64_t q0 = (int64_t)bx * kBT + threadIdx.x;
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
    if (bx == 0 && threadIdx.x == 0 && out_norm) *out_norm = nrm;
    const float c = adam_clip(nrm, hp.max_grad_norm);
    const float tt = (float)(*tptr);
    const float bc1 = 1.f - powf(hp.beta1, tt);
    const float bc2 = 1.f - powf(hp.beta2, tt);
    const float decay = 1.f - hp.lr * hp.weight_decay;
    bool bad = false, bad_state = false;
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
            bad_state |= (i + e < n) && !(isfinite(p) && isfinite(mi) && isfinite(vi));
        }
        st4(params, i, n, vec, p4);
        st4(m, i, n, vec, m4);
        st4(v, i, n, vec, v4);
    }
    if (bad) set_flag(flags, 0x1);
    if (bad_state) set_flag(flags, 0x8);
}

}  // namespace iqlh
