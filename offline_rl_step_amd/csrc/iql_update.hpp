// Block-level bodies of the IQL gradient reduction and clipped Adam, shared
// by their own launches and by the merged whole-step launches.  The method is
// described in iql.hip.
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 master weight -> operand-typed shadow (bfloat16: round to nearest
// even, v_cvt_pk_bf16_f32)
template <typename T> IQLH_DEV T to_shadow(float x);
template <> IQLH_DEV float to_shadow<float>(float x) { return x; }
template <> IQLH_DEV uint16_t to_shadow<uint16_t>(float x) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x, 0.f}, b2)) & 0xFFFFu);
}

// Sums the per-workgroup partials of every parameter in a fixed order (slice
// sl of a block adds workgroups sl, sl + 8, ... in turn; the eight slice sums
// are then added in slice order), writes grad and per-block sums of squares,
// and, in block 0, the mean loss.  Each
// thread streams float4 quads of four parameters, all sixteen of a 128-row
// partial set in flight at once (in the whole-step launch, built with the
// ILP-first scheduler, unrolling by 16 measured faster than by 4 or 8).
constexpr int kRedLanes = 32;                 // threads per slice, 4 parameters each
constexpr int kRedSlices = 256 / kRedLanes;
constexpr int kRedParams = 4 * kRedLanes;     // parameters per block (divides 128)

// Block bx (of rb per group) of group g.
IQLH_DEV void iql_reduce_block(const float* __restrict__ part, const float* __restrict__ loss_part, int nwg,
                               int nloss, int64_t P, int64_t Pp, float invB, float* __restrict__ grad,
                               float* __restrict__ sq_part, int rb, float* __restrict__ out_loss,
                               int32_t* __restrict__ flags, int bx, int g) {
    __shared__ f32x4 red[kRedSlices][kRedLanes];
    __shared__ float wred[4];
    const int tid = threadIdx.x, q = tid % kRedLanes, sl = tid / kRedLanes;
    const int64_t p0 = (int64_t)bx * kRedParams + 4 * q;  // < Pp
    const float* src = part + (int64_t)g * nwg * Pp + p0;
    // block 0's share of the loss partials: the first one issued with the
    // gradient loads (at a clamped index, nloss >= 1, so that no lane-dependent
    // branch makes the gradient loads wait for it), any others after them
    float l0 = 0.f;
    if (bx == 0) l0 = loss_part[(int64_t)g * nloss + (tid < nloss ? tid : nloss - 1)];
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 16
    for (int w = sl; w < nwg; w += kRedSlices) acc += *(const f32x4*)(src + (int64_t)w * Pp);
    float l = 0.f + keep_if(tid < nloss, l0);
    if (bx == 0)
        for (int w = tid + 256; w < nloss; w += 256) l += loss_part[(int64_t)g * nloss + w];
    red[sl][q] = acc;
    __syncthreads();
    float sq = 0.f;
    if (sl == 0) {
        f32x4 s = red[0][q];
#pragma unroll
        for (int i = 1; i < kRedSlices; ++i) s += red[i][q];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (p0 + e < P) {
                grad[(int64_t)g * P + p0 + e] = s[e];
                sq = fmaf(s[e], s[e], sq);
            }
        }
    }
    sq = block_sum<256>(sq, wred);
    if (tid == 0) sq_part[(int64_t)g * rb + bx] = sq;
    if (bx == 0) {
        l = block_sum<256>(l, wred);
        if (tid == 0) {
            const float loss = l * invB;
            if (out_loss) out_loss[g] = loss;
            if (!isfinite(loss)) set_flag(flags, 0x4);
        }
    }
}

// The counters of group g's update, in a block of its own in the reduction's
// launch: t[g] and (group 0) the step counter are incremented, and the Adam
// bias corrections 1 - beta1^t, 1 - beta2^t of the new t are stored for the
// update blocks, which would otherwise each compute them in every wave.
IQLH_DEV void iql_count_block(int32_t* __restrict__ tcount, int64_t* __restrict__ step, float* __restrict__ bc,
                              float beta1, float beta2, int g) {
    if (threadIdx.x == 0) {
        const int32_t tn = tcount[g] + 1;
        tcount[g] = tn;
        if (g == 0) *step += 1;
        bc[2 * g] = 1.f - powf(beta1, (float)tn);
        bc[2 * g + 1] = 1.f - powf(beta2, (float)tn);
    }
}

// One parameter's clipped Adam update ("DQN Backward-Path NaN Audit -- SP1
// Phase A", section on iqn_adam_kernel): gi is the clipped gradient; returns
// false (state untouched) when gi is not finite.  Contraction is off so that
// every kernel this is inlined into rounds the same way (the compiler could
// otherwise fuse beta1 m + (1 - beta1) g into a multiply-add differently in
// each), which keeps the whole-step launch and the separate entry points
// equal bit for bit.
IQLH_DEV bool adam_elem(float gi, float& p, float& m, float& v, float bc1, float bc2, float decay,
                        const AdamHyper& hp) {
#pragma clang fp contract(off)
    if (!isfinite(gi)) return false;
    const float mi = hp.beta1 * m + (1.f - hp.beta1) * gi;
    const float vi = hp.beta2 * v + (1.f - hp.beta2) * gi * gi;
    const float mh = mi / bc1, vh = vi / bc2;
    if (hp.weight_decay != 0.f) p *= decay;
    p -= hp.lr * mh / (sqrtf(vh) + hp.eps);
    if (hp.clamp > 0.f) p = fminf(fmaxf(p, -hp.clamp), hp.clamp);
    m = mi;
    v = vi;
    return true;
}

// Operand-typed shadows of flat parameter i of one group (a group has fewer
// than 2^31 parameters, so the row / column split is a 32-bit division):
// W1 [H][SP], W2 [H2][H] and its transpose [H][H2].
template <typename T>
IQLH_DEV void iql_store_shadow(int64_t i, float p, int H, int H2, int S, int SP, T* w1s, T* w2s, T* w2ts) {
    const int64_t ow2 = (int64_t)H * S + H, ow2e = ow2 + (int64_t)H2 * H;
    if (i < (int64_t)H * S) {
        const uint32_t r = (uint32_t)i / (uint32_t)S, cc = (uint32_t)i - r * (uint32_t)S;
        w1s[(int64_t)r * SP + cc] = to_shadow<T>(p);
    } else if (i >= ow2 && i < ow2e) {
        const uint32_t q = (uint32_t)(i - ow2), r = q / (uint32_t)H, cc = q - r * (uint32_t)H;
        w2s[q] = to_shadow<T>(p);
        w2ts[cc * H2 + r] = to_shadow<T>(p);
    }
}

// One parameter of iql_adam_block from its loaded state (gradient already
// clipped): Adam, the fused target update and the shadows, then every store.
// The stores come after the arithmetic, so no store sits between a load and
// its use (the use would wait for the store too).
template <typename T>
IQLH_DEV void iql_adam_param(int64_t i, float gi, float p, float mi, float vi, float ti, float bc1, float bc2,
                             float decay, const AdamHyper& hp, int H, int H2, int S, int SP,
                             float* __restrict__ prm,
                             float* __restrict__ gr, float* __restrict__ m, float* __restrict__ v,
                             float* __restrict__ tg, T* w1s, T* w2s, T* w2ts, bool& bad, bool& bad_state) {
    const bool ok = adam_elem(gi, p, mi, vi, bc1, bc2, decay, hp);
    gr[i] = 0.f;
    if (ok) {
        prm[i] = p;
        m[i] = mi;
        v[i] = vi;
        bad_state |= !(isfinite(p) && isfinite(mi) && isfinite(vi));
    } else {
        bad = true;
    }
    // Polyak target with the step's parameters (unchanged ones when the
    // update was skipped): target += ema (p - target)
    if (hp.ema > 0.f) tg[i] = fmaf(hp.ema, p - ti, ti);
    iql_store_shadow<T>(i, p, H, H2, S, SP, w1s, w2s, w2ts);
}

// Clip and Adam over the parameters of group g, block bx of nbx; refreshes
// the operand-typed W1 / W2 / W2^T shadows of the updated weights and zeroes
// grad.
template <typename T>
IQLH_DEV void iql_adam_block(const IqlDims& d, const IqlBuffers& b, const AdamHyper& hp,
                             float* __restrict__ out_gnorm, int rb, int bx, int g, int nbx) {
    __shared__ float red[4];
    const int64_t P = d.P;
    const int H = d.H, H2 = d.H2, S = d.S, SP = d.S_pad;
    float* prm = b.params + (int64_t)g * P;
    float* gr = b.grad + (int64_t)g * P;
    float* m = b.m + (int64_t)g * P;
    float* v = b.v + (int64_t)g * P;
    float* tg = b.target + (int64_t)g * P;
    T* w1s = (T*)b.w1s + (int64_t)g * H * SP;
    T* w2s = (T*)b.w2s + (int64_t)g * H2 * H;
    T* w2ts = (T*)b.w2ts + (int64_t)g * H2 * H;
    // The first element's state does not depend on the norm: it is loaded
    // before the fold, at a clamped index (P >= 1) so that no lane-dependent
    // branch surrounds the loads.
    const int64_t i0 = (int64_t)bx * 256 + threadIdx.x, stride = (int64_t)nbx * 256;
    const int64_t j0 = i0 < P ? i0 : P - 1;
    const float pg = gr[j0], pp = prm[j0], pm = m[j0], pv = v[j0], pt = tg[j0];
    const float bc1 = b.bc[2 * g], bc2 = b.bc[2 * g + 1];
    float a = 0.f;
    for (int i = threadIdx.x; i < rb; i += 256) a += b.sq_part[(int64_t)g * rb + i];
    const float nrm = sqrtf(block_sum<256>(a, red));
    const float c = !isfinite(nrm) ? __int_as_float(0x7FC00000)
                                   : ((nrm > hp.max_grad_norm && nrm > 0.f) ? hp.max_grad_norm / nrm : 1.f);
    const float decay = 1.f - hp.lr * hp.weight_decay;
    bool bad = false, bad_state = false;
    // software-pipelined: the next parameter's state is loaded before this
    // parameter's stores, so waiting for it never waits for the stores as
    // well (vmcnt counts both, in order).  The last iteration re-reads the
    // thread's own element (cached): one common address for every thread
    // would queue on one L2 channel.
    float cg = pg, cp = pp, cm = pm, cv = pv, ct = pt;
    for (int64_t i = i0; i < P; i += stride) {
        const int64_t nx = i + stride, j1 = nx < P ? nx : i;
        const float ng = gr[j1], np = prm[j1], nm = m[j1], nv = v[j1], nt = tg[j1];
        iql_adam_param<T>(i, cg * c, cp, cm, cv, ct, bc1, bc2, decay, hp, H, H2, S, SP, prm, gr, m, v, tg, w1s, w2s,
                          w2ts, bad, bad_state);
        cg = ng;
        cp = np;
        cm = nm;
        cv = nv;
        ct = nt;
    }
    // (stored last: a wave would wait for this store at its next use of a load)
    if (bx == 0 && threadIdx.x == 0 && out_gnorm) out_gnorm[g] = nrm;
    if (bad) set_flag(b.flags, 0x1);
    if (bad_state) set_flag(b.flags, 0x8);
}

}  // namespace iqlh
