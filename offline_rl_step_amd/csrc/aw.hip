// Advantage-weighted policy pi = softmax(beta * clamp(Q - V, -10, 10)), gfx950.
//
// Follows "GPU IQL + HER Porting Plan", section "Current State / IQL (CPU)",
// item "Advantage-weighted action selection": per-action advantage Q - V,
// clamp to [-10, 10], scale by the temperature beta, softmax over actions with
// the row maximum subtracted.
//
// HBM-bound.  Action counts of 4, 8, 16, 32 or 64 with 16-byte aligned rows
// take the streaming form (aw_block.hpp: float4 per lane, rows split over lanes).
// Any other A: a one-wave workgroup owns 64 consecutive rows (16384 rows give
// 256 workgroups, one per CU): the [64, A] slab of Q is read once with
// coalesced loads into LDS (padded to an odd row stride so the per-row reads
// are bank-conflict free), every group's policy is computed from that one
// copy, and each result slab is written back with coalesced stores.
#include "aw_block.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

constexpr int kAwRows = 64;

__global__ __launch_bounds__(kAwRows) void aw_policy_kernel(const float* __restrict__ q,
                                                         const float* __restrict__ v, int G, int B,
                                                         int A, float beta, float* __restrict__ pi) {
    extern __shared__ float lds[];
    const int AP = A | 1;  // odd stride
    float* sq = lds;                  // [kAwRows][AP]
    float* sp = lds + kAwRows * AP;   // [kAwRows][AP]
    const int64_t row0 = (int64_t)blockIdx.x * kAwRows;
    const int rows = (int)min<int64_t>(kAwRows, (int64_t)B - row0);
    const int cnt = rows * A;
    const float* qs = q + row0 * A;
    const int r = threadIdx.x;
    // every load is issued before any is consumed: the slab arrives in one
    // memory round trip (up to kStage values per thread; larger A loops)
    constexpr int kStage = 16;
    float stage[kStage];
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
        const int idx = threadIdx.x + k * kAwRows;
        stage[k] = idx < cnt ? qs[idx] : 0.f;
    }
    float vg[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) vg[g] = (g < G && r < rows) ? v[(int64_t)g * B + row0 + r] : 0.f;
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
        const int idx = threadIdx.x + k * kAwRows;
        if (idx < cnt) {
            const int rr = idx / A, c = idx - rr * A;
            sq[rr * AP + c] = stage[k];
        }
    }
    for (int idx = threadIdx.x + kStage * kAwRows; idx < cnt; idx += kAwRows) {
        const int rr = idx / A, c = idx - rr * A;
        sq[rr * AP + c] = qs[idx];
    }
    __syncthreads();
    for (int g = 0; g < G; ++g) {
        if (r < rows) {
            const float vv = g == 0 ? vg[0] : (g == 1 ? vg[1] : v[(int64_t)g * B + row0 + r]);
            const float* qr = sq + r * AP;
            float* pr = sp + r * AP;
            float mx = -INFINITY;
            for (int c = 0; c < A; ++c) {
                const float x = beta * fminf(fmaxf(qr[c] - vv, -10.f), 10.f);
                pr[c] = x;
                mx = fmaxf(mx, x);
            }
            float s = 0.f;
            for (int c = 0; c < A; ++c) {
                const float e = expf(pr[c] - mx);
                pr[c] = e;
                s += e;
            }
            for (int c = 0; c < A; ++c) pr[c] = pr[c] / s;
        }
        __syncthreads();
        float* ps = pi + ((int64_t)g * B + row0) * A;
        for (int idx = threadIdx.x; idx < cnt; idx += kAwRows) {
            const int rr = idx / A, c = idx - rr * A;
            ps[idx] = sp[rr * AP + c];
        }
        __syncthreads();
    }
}

// Streaming form (aw_block.hpp): 256-thread workgroups striding over the
// rows.
constexpr int kAwVecThreads = 256;

template <int LPR>
__global__ __launch_bounds__(kAwVecThreads) void aw_policy_vec_kernel(const float4* __restrict__ q,
                                                                   const float* __restrict__ v, int G, int64_t B,
                                                                   float beta, float4* __restrict__ pi) {
    aw_vec_rows<LPR, kAwVecThreads>(q, v, G, B, beta, pi, blockIdx.x, gridDim.x);
}

template <int LPR>
static hipError_t run_aw_vec(const float* q, const float* v, int G, int B, float beta, float* pi,
                             hipStream_t stream) {
    constexpr int RPW = kAwVecThreads / LPR;
    const int64_t need = ((int64_t)B + RPW * kAwUnroll - 1) / (RPW * kAwUnroll);
    const unsigned blocks = (unsigned)(need < 4096 ? need : 4096);
    hipLaunchKernelGGL(aw_policy_vec_kernel<LPR>, dim3(blocks), dim3(kAwVecThreads), 0, stream, (const float4*)q,
                       v, G, (int64_t)B, beta, (float4*)pi);
    return hipGetLastError();
}

hipError_t launch_aw_policy(const float* q, const float* v, int G, int B, int A, float beta,
                            float* pi, hipStream_t stream) {
    if (B <= 0) return hipSuccess;
    if (((uintptr_t)q & 15u) == 0 && ((uintptr_t)pi & 15u) == 0) {
        switch (A) {
            case 4: return run_aw_vec<1>(q, v, G, B, beta, pi, stream);
            case 8: return run_aw_vec<2>(q, v, G, B, beta, pi, stream);
            case 16: return run_aw_vec<4>(q, v, G, B, beta, pi, stream);
            case 32: return run_aw_vec<8>(q, v, G, B, beta, pi, stream);
            case 64: return run_aw_vec<16>(q, v, G, B, beta, pi, stream);
            default: break;
        }
    }
    const unsigned blocks = (unsigned)((B + kAwRows - 1) / kAwRows);
    const size_t lds = (size_t)2 * kAwRows * (A | 1) * sizeof(float);
    hipLaunchKernelGGL(aw_policy_kernel, dim3(blocks), dim3(kAwRows), lds, stream, q, v, G, B, A, beta, pi);
    return hipGetLastError();
}

}  // namespace iqlh
