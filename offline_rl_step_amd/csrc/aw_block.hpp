// Block body of the streaming advantage-weighted policy
// pi = softmax(beta * clamp(Q - V, -10, 10)) ("GPU IQL + HER Porting Plan",
// section "Current State / IQL (CPU)", item "Advantage-weighted action
// selection"), shared by its own launch and by the wide-hidden weight-gradient
// launch, whose spare workgroups run it on compute units the gradient tiles
// leave idle.
//
// Action counts A = 4 LPR with LPR in {1, 2, 4, 8, 16} and 16-byte aligned
// rows: LPR lanes own one row, one float4 of four actions each, so a wave's
// load or store of 64 float4 covers 64 / LPR consecutive rows (1 KB
// contiguous).  The row maximum and sum are xor-shuffles among the row's
// lanes.  Each lane keeps kAwUnroll rows' loads in flight before it computes;
// block bid of nb strides over the rows.
#pragma once
#include "common.hpp"

namespace iqlh {

constexpr int kAwUnroll = 4;
typedef float aw_f4v __attribute__((ext_vector_type(4)));

template <int LPR, int NT>
IQLH_DEV void aw_vec_rows(const float4* __restrict__ q, const float* __restrict__ v, int G, int64_t B, float beta,
                          float4* __restrict__ pi, int64_t bid, int64_t nb) {
    constexpr int RPW = NT / LPR;  // rows per workgroup pass
    const int sub = threadIdx.x % LPR;
    const int64_t stride = nb * RPW * kAwUnroll;
    for (int64_t base = bid * RPW * kAwUnroll; base < B; base += stride) {
        float4 x[kAwUnroll];
        int64_t row[kAwUnroll];
#pragma unroll
        for (int u = 0; u < kAwUnroll; ++u) {
            row[u] = base + (int64_t)u * RPW + threadIdx.x / LPR;
            const int64_t rc = row[u] < B ? row[u] : B - 1;
            x[u] = q[rc * LPR + sub];
        }
        for (int g = 0; g < G; ++g) {
            float vv[kAwUnroll];
#pragma unroll
            for (int u = 0; u < kAwUnroll; ++u) vv[u] = v[(int64_t)g * B + (row[u] < B ? row[u] : B - 1)];
#pragma unroll
            for (int u = 0; u < kAwUnroll; ++u) {
                float e[4] = {x[u].x, x[u].y, x[u].z, x[u].w};
                float mx = -INFINITY;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    e[j] = beta * fminf(fmaxf(e[j] - vv[u], -10.f), 10.f);
                    mx = fmaxf(mx, e[j]);
                }
#pragma unroll
                for (int o = LPR / 2; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, LPR));
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    e[j] = expf(e[j] - mx);
                    s += e[j];
                }
#pragma unroll
                for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, LPR);
                // the policy is this call's output only: non-temporal stores
                // (measured 5 % faster on working sets beyond the caches)
                if (row[u] < B)
                    __builtin_nontemporal_store(aw_f4v{e[0] / s, e[1] / s, e[2] / s, e[3] / s},
                                                (aw_f4v*)&pi[((int64_t)g * B + row[u]) * LPR + sub]);
            }
        }
    }
}

// The lanes per row of the streaming form for A actions, 0 when A has none.
__host__ __device__ inline int aw_vec_lanes(int A) {
    return A == 4 ? 1 : A == 8 ? 2 : A == 16 ? 4 : A == 32 ? 8 : A == 64 ? 16 : 0;
}

}  // namespace iqlh
