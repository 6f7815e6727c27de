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

// Quad at element i (a multiple of 4 below n) with no lane-dependent branch:
// one 16-byte load when vec4 (every pointer 16-byte aligned and n a multiple
// of 4, the same for all lanes), else four element loads at clamped indices,
// zero past n.  A lane-dependent branch around a load makes the code after
// its end wait for every load in flight, which would serialise consecutive
// quads.
IQLH_DEV f32x4 ld4(const float* __restrict__ p, int64_t i, int64_t n, bool vec4) {
    if (vec4) return *(const f32x4*)(p + i);
    f32x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = keep_if(i + e < n, p[i + e < n ? i + e : n - 1]);
    return r;
}
// 16-byte quad loads are possible: aligned pointers and no partial last quad.
IQLH_DEV bool quads_vec(int vec, int64_t n) { return vec && (n & 3) == 0; }
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
// Every set's partial is loaded before any is added (at a clamped set index,
// so no branch separates the loads from each other), so one wait covers them.
IQLH_DEV void fold_partials_k(const float* __restrict__ p, int nb, int k, float (&out)[kMaxSources],
                              float (*red)[kBT / kWave]) {
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j) out[j] = 0.f;
    for (int i = threadIdx.x; i < nb; i += kBT) {
        float x[kMaxSources];
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j) x[j] = keep_if(j < k, p[(int64_t)(j < k ? j : k - 1) * nb + i]);
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j)
            if (j < k) out[j] += x[j];
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
    const bool vec4 = quads_vec(vec, n);
    for (int64_t qd = (int64_t)bx * kBT + t; qd < quads; qd += stride) {
        // every source's quad in flight before the first is used
        f32x4 x[kMaxSources];
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j)
            x[j] = j < s.k ? ld4(s.ptr[j], 4 * qd, n, vec4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j)
            if (j < s.k)
                acc[j] = fmaf(x[j].x, x[j].x, fmaf(x[j].y, x[j].y, fmaf(x[j].z, x[j].z, fmaf(x[j].w, x[j].w, acc[j]))));
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
template <bool PIPE = false>
IQLH_DEV void saxpy_block(const SourceSet& s, int64_t n, int vec, float mgn, const float* __restrict__ partials,
                          float* __restrict__ grad, float* __restrict__ gpart, float* __restrict__ out_norms, int bx,
                          int nb) {
    __shared__ float red[kBT / kWave];
    __shared__ float redk[kMaxSources][kBT / kWave];
    // this thread's first quad of every source does not depend on the clip
    // scales: load it before folding the norm partials
    const int64_t quads = (n + 3) / 4, stride = (int64_t)nb * kBT;
    const int64_t q0 = (int64_t)bx * kBT + threadIdx.x;
    const bool vec4 = quads_vec(vec, n);
    // (at a clamped quad, so that no lane-dependent branch surrounds the
    // loads; a thread past the last quad does not use them)
    const int64_t c0 = q0 < quads ? q0 : quads - 1;
    f32x4 pre[kMaxSources];
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j)
        pre[j] = (j < s.k && quads > 0) ? ld4(s.ptr[j], 4 * c0, n, vec4) : f32x4{0.f, 0.f, 0.f, 0.f};
    // every thread folds every source's partials (same value in all threads
    // and blocks) and derives the clip scales itself
    float c[kMaxSources], nrm[kMaxSources];
    fold_partials_k(partials, nb, s.k, c, redk);
#pragma unroll
    for (int j = 0; j < kMaxSources; ++j) {
        nrm[j] = sqrtf(c[j]);
        c[j] = j < s.k ? s.alpha[j] * budget_scale(nrm[j], s.frac[j] * mgn) : 0.f;
    }
    // PIPE: software-pipelined, the next quad's loads issued before this
    // quad's store, so that waiting for them never waits for the store as
    // well (vmcnt counts both, in order) -- for the standalone pass, whose
    // threads take many quads; it holds a second set of source quads, which
    // would lower the occupancy of the merged launch whose reduction blocks
    // share the kernel.  A thread's last iteration re-reads its own quad
    // (cached) rather than a common one: the same address from every thread
    // would queue on one L2 channel.  Same sums either way.
    float acc = 0.f;
    if constexpr (PIPE) {
        for (int64_t qd = q0; qd < quads; qd += stride) {
            const int64_t nx = qd + stride, nc = nx < quads ? nx : qd;
            f32x4 x[kMaxSources];
#pragma unroll
            for (int j = 0; j < kMaxSources; ++j)
                x[j] = j < s.k ? ld4(s.ptr[j], 4 * nc, n, vec4) : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kMaxSources; ++j)
                if (j < s.k) g += c[j] * pre[j];
            st4(grad, 4 * qd, n, vec, g);
            acc = fmaf(g.x, g.x, fmaf(g.y, g.y, fmaf(g.z, g.z, fmaf(g.w, g.w, acc))));
#pragma unroll
            for (int j = 0; j < kMaxSources; ++j) pre[j] = x[j];
        }
    } else {
        if (q0 < quads) {
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kMaxSources; ++j)
                if (j < s.k) g += c[j] * pre[j];
            st4(grad, 4 * q0, n, vec, g);
            acc = fmaf(g.x, g.x, fmaf(g.y, g.y, fmaf(g.z, g.z, fmaf(g.w, g.w, acc))));
        }
        for (int64_t qd = q0 + stride; qd < quads; qd += stride) {
            // every source's quad in flight before the first is used
            f32x4 x[kMaxSources];
#pragma unroll
            for (int j = 0; j < kMaxSources; ++j)
                x[j] = j < s.k ? ld4(s.ptr[j], 4 * qd, n, vec4) : f32x4{0.f, 0.f, 0.f, 0.f};
            f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kMaxSources; ++j)
                if (j < s.k) g += c[j] * x[j];
            st4(grad, 4 * qd, n, vec, g);
            acc = fmaf(g.x, g.x, fmaf(g.y, g.y, fmaf(g.z, g.z, fmaf(g.w, g.w, acc))));
        }
    }
    const float t = block_sum<kBT>(acc, red);
    if (threadIdx.x == 0) gpart[bx] = t;
    // block 0's norms last: a store issued earlier would make the wave's next
    // wait for a load wait for it as well
    if (bx == 0 && threadIdx.x == 0 && out_norms) {
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j)
            if (j < s.k) out_norms[j] = nrm[j];
    }
}

// The Adam step count of a pass-3 update: one thread increments t and stores
// the bias corrections 1 - beta1^t, 1 - beta2^t of the new count for the
// update blocks, so that they are computed once rather than by every wave.
// Runs in the launch before the update, in a block of its own.
IQLH_DEV void adam_count_block(int32_t* __restrict__ t, float* __restrict__ bc, float beta1, float beta2) {
    if (threadIdx.x == 0) {
        const int32_t tn = *t + 1;
        *t = tn;
        bc[0] = 1.f - powf(beta1, (float)tn);
        bc[1] = 1.f - powf(beta2, (float)tn);
    }
}

IQLH_DEV void norm_finalize_block(const float* __restrict__ p, int nb, float* __restrict__ out) {
    __shared__ float red[kBT / kWave];
    const float sq = fold_partials(p, nb, red);
    if (threadIdx.x == 0) *out = sqrtf(sq);
}

// One quad of pass 3: the clipped Adam update of elements i .. i+3 (those
// < n) from their loaded state, then every store of the quad (grad zeroed).
// The stores come after the arithmetic: a store issued between a load and
// its use would make the use wait for the store as well.
IQLH_DEV void adam_flat_quad(float* __restrict__ params, float* __restrict__ grad, float* __restrict__ m,
                             float* __restrict__ v, int64_t i, int64_t n, int vec, f32x4 g4, f32x4 m4, f32x4 v4,
                             f32x4 p4, float bc1, float bc2, float decay, const AdamHyper& hp, bool& bad,
                             bool& bad_state) {
    // no contraction: the same roundings in every kernel this is inlined into
#pragma clang fp contract(off)
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
    st4(grad, i, n, vec, f32x4{0.f, 0.f, 0.f, 0.f});
    st4(params, i, n, vec, p4);
    st4(m, i, n, vec, m4);
    st4(v, i, n, vec, v4);
}

// Pass 3 for block bx of nbx: folds the nb grad partials into the norm and
// applies the clipped Adam update to the block's quads, zeroing grad.
IQLH_DEV void adam_flat_block(float* __restrict__ params, float* __restrict__ grad, float* __restrict__ m,
                              float* __restrict__ v, const float* __restrict__ bcp,
                              const float* __restrict__ sq_part, int nb, int64_t n, int vec,
                              const AdamHyper& hp, float* __restrict__ out_norm, int32_t* __restrict__ flags,
                              int bx, int nbx) {
#pragma clang fp contract(off)
    __shared__ float red[kBT / kWave];
    const int64_t quads = (n + 3) / 4, stride = (int64_t)nbx * kBT;
    const int64_t q0 = (int64_t)bx * kBT + threadIdx.x;
    // The first quad's state does not depend on the norm: it is loaded before
    // the fold, at a clamped index so that no lane-dependent branch surrounds
    // the loads.
    const bool vec4 = quads_vec(vec, n), any = quads > 0;
    const int64_t c0 = q0 < quads ? q0 : quads - 1;
    const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};
    const f32x4 pg = any ? ld4(grad, 4 * c0, n, vec4) : z4, pm = any ? ld4(m, 4 * c0, n, vec4) : z4;
    const f32x4 pv = any ? ld4(v, 4 * c0, n, vec4) : z4, pp = any ? ld4(params, 4 * c0, n, vec4) : z4;
    const float bc1 = bcp[0], bc2 = bcp[1];
    const float sq = fold_partials(sq_part, nb, red);
    const float nrm = sqrtf(sq);
    const float c = adam_clip(nrm, hp.max_grad_norm);
    const float decay = 1.f - hp.lr * hp.weight_decay;
    bool bad = false, bad_state = false;
    // software-pipelined as in saxpy_block: the next quad's state is loaded
    // before this quad's stores (the last iteration re-reads its own quad)
    f32x4 cg = pg, cm = pm, cv = pv, cp = pp;
    for (int64_t qd = q0; qd < quads; qd += stride) {
        const int64_t nx = qd + stride, i1 = 4 * (nx < quads ? nx : qd);
        const f32x4 ng = ld4(grad, i1, n, vec4), nm = ld4(m, i1, n, vec4), nv = ld4(v, i1, n, vec4),
                    np = ld4(params, i1, n, vec4);
        adam_flat_quad(params, grad, m, v, 4 * qd, n, vec, cg * c, cm, cv, cp, bc1, bc2, decay, hp, bad, bad_state);
        cg = ng;
        cm = nm;
        cv = nv;
        cp = np;
    }
    // (stored last: a wave would wait for this store at its next use of a load)
    if (bx == 0 && threadIdx.x == 0 && out_norm) *out_norm = nrm;
    if (bad) set_flag(flags, 0x1);
    if (bad_state) set_flag(flags, 0x8);
}

}  // namespace iqlh
