// Prioritized-replay source sampling ("GPU IQL + HER Porting Plan", section
// "Current State": prefix sum of the priorities and a GPU search in it,
// indices and importance-sampling weights out; section "How HER Interacts
// with GPU PER": sample_indices for the HER sources).
//
// Row i is drawn with probability p_i / sum(p), independently, by inverse
// transform: u = U * total (U = 53 bits of Philox4x64-10 word 0 at counter
// (draw, step, 0, 0) under the key (seed, "PERdraws")), capped just below the
// total; the row is the first i whose inclusive prefix sum exceeds u.
// Weights are prioritized replay's (N P(i))^-beta over the batch maximum,
// i.e. (p_min / p_i)^beta with p_min the smallest drawn priority.
//
// MI355X layout, four launches on a caller workspace:
//   A  fp64 sum of each 2048-priority block (fixed order);
//   B  inclusive fp64 prefix of every row: each block folds the sums of the
//      blocks before it in a fixed order, then scans its own rows (thread
//      runs of 8, wave scan by DPP-free shuffles, waves through LDS);
//   C  one wave per draw: a 64-ary search (each lane probes one position, a
//      ballot picks the segment) -- about four dependent round trips over
//      2^20 rows instead of twenty; the smallest drawn priority by an
//      integer minimum on its bit pattern (order-independent);
//   D  the weights.
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

constexpr uint64_t kPerKey1 = 0x5045526472617773ull;  // "PERdraws"
constexpr int kPerBlock = 2048;                        // priorities per block of A and B

struct PerArgs {
    const float* p;
    int64_t size;
    int n;
    uint64_t seed;
    const int64_t* step;
    float beta;
    int32_t* idx;
    float* w;
    int32_t* flags;
    double* prefix;  // [size]
    double* bsum;    // [nb]
    uint32_t* pmin;  // [1]
    int nb;
};

IQLH_DEV bool bad_priority(float x) { return !(x >= 0.f) || !isfinite(x); }

__global__ __launch_bounds__(256) void per_block_sums_kernel(PerArgs a) {
    __shared__ double red[4];
    const int64_t base = (int64_t)blockIdx.x * kPerBlock + 8 * threadIdx.x;
    double s = 0.0;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int64_t i = base + k;
        const float x = i < a.size ? a.p[i] : 0.f;
        bad |= bad_priority(x);
        s += (double)x;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    if (__syncthreads_or(bad) && threadIdx.x == 0) set_flag(a.flags, 0x2);
    if (threadIdx.x == 0) a.bsum[blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void per_prefix_kernel(PerArgs a) {
    __shared__ double red[4], wtot[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    // offset = sum of the blocks before this one, in a fixed order
    double o = 0.0;
    for (int j = threadIdx.x; j < (int)blockIdx.x; j += 256) o += a.bsum[j];
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) o += __shfl_xor(o, s, 64);
    if (lane == 0) red[wv] = o;
    // this thread's run of 8
    const int64_t base = (int64_t)blockIdx.x * kPerBlock + 8 * threadIdx.x;
    double run[8];
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int64_t i = base + k;
        t += i < a.size ? (double)a.p[i] : 0.0;
        run[k] = t;
    }
    // inclusive scan of the run totals across the wave
    double incl = t;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const double y = __shfl_up(incl, s, 64);
        if (lane >= s) incl += y;
    }
    if (lane == 63) wtot[wv] = incl;
    __syncthreads();
    const double offset = (red[0] + red[1]) + (red[2] + red[3]);
    double before = offset + (incl - t);
    for (int w = 0; w < wv; ++w) before += wtot[w];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int64_t i = base + k;
        if (i < a.size) a.prefix[i] = before + run[k];
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.pmin = 0xFFFFFFFFu;
}

__global__ __launch_bounds__(256) void per_draw_kernel(PerArgs a) {
    const int lane = threadIdx.x & 63;
    const int k = blockIdx.x * 4 + (threadIdx.x >> 6);  // this wave's draw
    if (k >= a.n) return;                                // wave-uniform
    const uint64_t step = a.step ? (uint64_t)*a.step : 0ull;
    const uint64_t word = philox4x64_10(u64x4{(uint64_t)k, step, 0ull, 0ull}, a.seed, kPerKey1).x;
    const double total = a.prefix[a.size - 1];
    double u = (double)(word >> 11) * 0x1.0p-53 * total;
    const double cap = __longlong_as_double(__double_as_longlong(total) - 1);  // largest double below a positive total
    if (u > cap) u = cap;
    int32_t found = -1;
    if (total > 0.0 && isfinite(total)) {
        int64_t lo = 0, hi = a.size;  // answer in [lo, hi)
        for (int it = 0; it < 8 && hi - lo > 1; ++it) {
            const int64_t span = hi - lo;
            const int64_t stp = (span + 63) / 64;
            int64_t pos = lo + (int64_t)(lane + 1) * stp - 1;
            if (pos > hi - 1) pos = hi - 1;
            const bool gt = a.prefix[pos] > u;
            const uint64_t bal = __ballot(gt);
            if (!bal) { lo = hi; break; }  // cannot happen while u < prefix[size - 1]
            const int j = __builtin_ctzll(bal);
            const int64_t pj = __shfl(pos, j, 64);
            const int64_t pprev = j > 0 ? __shfl(pos, j - 1, 64) : lo - 1;
            hi = pj + 1;
            lo = pprev + 1;
        }
        if (hi - lo == 1) found = (int32_t)lo;
    }
    if (lane == 0) {
        a.idx[k] = found;
        if (found >= 0) atomicMin(a.pmin, __float_as_uint(a.p[found]));
        else set_flag(a.flags, 0x2);
    }
}

__global__ __launch_bounds__(256) void per_weight_kernel(PerArgs a) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= a.n) return;
    const int32_t i = a.idx[k];
    float w = 0.f;
    if (i >= 0) {
        const double pm = (double)__uint_as_float(*a.pmin), pi = (double)a.p[i];
        w = (float)pow(pm / pi, (double)a.beta);
    }
    a.w[k] = w;
}

size_t per_workspace_bytes_for(int64_t size) {
    const int64_t nb = (size + kPerBlock - 1) / kPerBlock;
    return (size_t)(8 * size + 8 * nb + 16 + 255) / 256 * 256;
}

hipError_t launch_per_sample(const float* p, int64_t size, int n, uint64_t seed, const int64_t* d_step, float beta,
                             int32_t* idx, float* w, int32_t* flags, void* workspace, hipStream_t stream) {
    PerArgs a{};
    a.p = p; a.size = size; a.n = n; a.seed = seed; a.step = d_step; a.beta = beta;
    a.idx = idx; a.w = w; a.flags = flags;
    a.nb = (int)((size + kPerBlock - 1) / kPerBlock);
    a.prefix = (double*)workspace;
    a.bsum = a.prefix + size;
    a.pmin = (uint32_t*)(a.bsum + a.nb);
    hipLaunchKernelGGL(per_block_sums_kernel, dim3(a.nb), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(per_prefix_kernel, dim3(a.nb), dim3(256), 0, stream, a);
    if (n > 0) {
        hipLaunchKernelGGL(per_draw_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, a);
        hipLaunchKernelGGL(per_weight_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace iqlh
