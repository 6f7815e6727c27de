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
//      blocks before it in a fixed order, then scans its own rows (runs of 8
//      per thread in registers, one wave scan by shuffles, waves through LDS);
//   C  one wave per draw, 64-ary searches (each lane probes one position,
//      a ballot picks the segment): first over the table of block ends,
//      staged in LDS once per workgroup, then inside the one 2048-row block
//      -- two rounds of global loads per draw instead of twenty; each
//      workgroup's smallest drawn priority (integer minimum on the bit
//      pattern: order-independent) to a slot of its own;
//   D  the weights, after every block folds the workgroup minima.
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
    double* bend;    // [nb] prefix at the last row of each block
    uint32_t* wgmin; // [nwg] smallest drawn priority (bit pattern) of each draw workgroup
    int vec;         // priorities 16-byte aligned
    int nb, nwg, dpw;  // blocks of A/B; draw workgroups; draws per wave
};

IQLH_DEV bool bad_priority(float x) { return !(x >= 0.f) || !isfinite(x); }

__global__ __launch_bounds__(256) void per_block_sums_kernel(PerArgs a) {
    __shared__ double red[4];
    const int64_t base = (int64_t)blockIdx.x * kPerBlock + threadIdx.x;
    double s = 0.0;
    bool bad = false;
#pragma unroll
    for (int k = 0; k < kPerBlock / 256; ++k) {
        const int64_t i = base + 256 * k;
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

// Inclusive prefix of one block's rows: each thread scans a run of 8 rows in
// registers (two 16-byte loads: a wave reads 2 KB contiguous), one wave scan
// of the run totals by shuffles, the totals of the waves before through LDS,
// 16-byte stores.
__global__ __launch_bounds__(256) void per_prefix_kernel(PerArgs a) {
    __shared__ double red[4], wtot[4];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int64_t base = (int64_t)blockIdx.x * kPerBlock + 8 * threadIdx.x;
    float x[8];
    if (a.vec && base + 8 <= a.size) {
        const float4 lo = *(const float4*)(a.p + base), hi = *(const float4*)(a.p + base + 4);
        x[0] = lo.x; x[1] = lo.y; x[2] = lo.z; x[3] = lo.w; x[4] = hi.x; x[5] = hi.y; x[6] = hi.z; x[7] = hi.w;
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = base + k < a.size ? a.p[base + k] : 0.f;
    }
    // offset = sum of the blocks before this one, in a fixed order
    double o = 0.0;
    for (int j = threadIdx.x; j < (int)blockIdx.x; j += 256) o += a.bsum[j];
#pragma unroll
    for (int s = 32; s > 0; s >>= 1) o += __shfl_xor(o, s, 64);
    if (lane == 0) red[wv] = o;
    double run[8];
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        t += (double)x[k];
        run[k] = t;
    }
    double incl = t;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const double y = __shfl_up(incl, s, 64);
        if (lane >= s) incl += y;
    }
    if (lane == 63) wtot[wv] = incl;
    __syncthreads();
    double before = ((red[0] + red[1]) + (red[2] + red[3])) + (incl - t);
    for (int w = 0; w < wv; ++w) before += wtot[w];
    double v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = before + run[k];
    const int64_t last = min((int64_t)(blockIdx.x + 1) * kPerBlock, a.size) - 1;
    if (base + 8 <= a.size) {
#pragma unroll
        for (int k = 0; k < 8; k += 2) *(double2*)(a.prefix + base + k) = double2{v[k], v[k + 1]};
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (base + k < a.size) a.prefix[base + k] = v[k];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
        if (base + k == last) a.bend[blockIdx.x] = v[k];
}

// First i in [lo, hi) with prefix[i] > u, given prefix[hi - 1] > u: each lane
// probes one of 64 evenly spaced positions and the ballot picks the segment.
template <typename Load>
IQLH_DEV int64_t search64(int64_t lo, int64_t hi, double u, Load&& at) {
    const int lane = threadIdx.x & 63;
    for (int it = 0; it < 8 && hi - lo > 1; ++it) {
        const int64_t stp = (hi - lo + 63) / 64;
        int64_t pos = lo + (int64_t)(lane + 1) * stp - 1;
        if (pos > hi - 1) pos = hi - 1;
        const uint64_t bal = __ballot(at(pos) > u);
        if (!bal) return -1;  // cannot happen while at(hi - 1) > u
        const int j = __builtin_ctzll(bal);
        const int64_t pj = __shfl(pos, j, 64);
        const int64_t pprev = j > 0 ? __shfl(pos, j - 1, 64) : lo - 1;
        hi = pj + 1;
        lo = pprev + 1;
    }
    return hi - lo == 1 ? lo : -1;
}

constexpr int kPerMaxWg = 1024;  // workgroups of the draw pass (each wave takes ceil(n / 4096) draws)
constexpr int kPerTable = 8192;  // block ends staged in LDS (at most 64 KB): up to 2^24 rows

// Draws of one wave: the block of the row from the table of block ends
// (binary64 prefix at the last row of every 2048-row block, staged in LDS
// once per workgroup), then the row inside that block -- two rounds of
// global loads per draw.
__global__ __launch_bounds__(256) void per_draw_kernel(PerArgs a) {
    extern __shared__ double tbl[];  // [nb] when staged
    const int lane = threadIdx.x & 63;
    const bool staged = a.nb <= kPerTable;
    if (staged)
        for (int j = threadIdx.x; j < a.nb; j += 256) tbl[j] = a.bend[j];
    __syncthreads();
    const uint64_t step = a.step ? (uint64_t)*a.step : 0ull;
    const double total = a.prefix[a.size - 1];
    const double cap = __longlong_as_double(__double_as_longlong(total) - 1);  // largest double below a positive total
    const bool ok = total > 0.0 && isfinite(total);
    const int k0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * a.dpw;
    uint32_t wmin = 0xFFFFFFFFu;  // smallest drawn priority of this wave (bit pattern: p >= 0)
    for (int kk = 0; kk < a.dpw; ++kk) {
        const int k = k0 + kk;
        if (k >= a.n) break;  // wave-uniform
        const uint64_t word = philox4x64_10(u64x4{(uint64_t)k, step, 0ull, 0ull}, a.seed, kPerKey1).x;
        double u = (double)(word >> 11) * 0x1.0p-53 * total;
        if (u > cap) u = cap;
        int64_t found = -1;
        if (ok) {
            if (staged) {
                const int64_t blk = search64(0, a.nb, u, [&](int64_t i) { return tbl[i]; });
                if (blk >= 0) {
                    const int64_t lo = blk * kPerBlock, hi = min(lo + kPerBlock, a.size);
                    found = search64(lo, hi, u, [&](int64_t i) { return a.prefix[i]; });
                }
            } else {
                found = search64(0, a.size, u, [&](int64_t i) { return a.prefix[i]; });
            }
        }
        if (lane == 0) {
            a.idx[k] = (int32_t)found;
            if (found >= 0) wmin = min(wmin, __float_as_uint(a.p[found]));
            else set_flag(a.flags, 0x2);
        }
    }
    // the workgroup's minimum to its own slot (no atomics: same-address
    // atomics serialise in L2); the weight pass folds the slots
    __shared__ uint32_t smin[4];
    if (lane == 0) smin[threadIdx.x >> 6] = wmin;
    __syncthreads();
    if (threadIdx.x == 0) a.wgmin[blockIdx.x] = min(min(smin[0], smin[1]), min(smin[2], smin[3]));
}

__global__ __launch_bounds__(256) void per_weight_kernel(PerArgs a) {
    __shared__ uint32_t red[4];
    uint32_t mn = 0xFFFFFFFFu;
    for (int j = threadIdx.x; j < a.nwg; j += 256) mn = min(mn, a.wgmin[j]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mn;
    __syncthreads();
    mn = min(min(red[0], red[1]), min(red[2], red[3]));
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= a.n) return;
    const int32_t i = a.idx[k];
    float w = 0.f;
    if (i >= 0) {
        const double pm = (double)__uint_as_float(mn), pi = (double)a.p[i];
        w = (float)pow(pm / pi, (double)a.beta);
    }
    a.w[k] = w;
}

size_t per_workspace_bytes_for(int64_t size) {
    const int64_t nb = (size + kPerBlock - 1) / kPerBlock;
    return (size_t)(8 * size + 16 * nb + 4 * kPerMaxWg + 255) / 256 * 256;
}

hipError_t launch_per_sample(const float* p, int64_t size, int n, uint64_t seed, const int64_t* d_step, float beta,
                             int32_t* idx, float* w, int32_t* flags, void* workspace, hipStream_t stream) {
    PerArgs a{};
    a.p = p; a.size = size; a.n = n; a.seed = seed; a.step = d_step; a.beta = beta;
    a.idx = idx; a.w = w; a.flags = flags;
    a.nb = (int)((size + kPerBlock - 1) / kPerBlock);
    a.vec = ((uintptr_t)p & 15u) == 0;
    a.prefix = (double*)workspace;
    a.bsum = a.prefix + size;
    a.bend = a.bsum + a.nb;
    a.wgmin = (uint32_t*)(a.bend + a.nb);
    hipLaunchKernelGGL(per_block_sums_kernel, dim3(a.nb), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(per_prefix_kernel, dim3(a.nb), dim3(256), 0, stream, a);
    if (n > 0) {
        a.dpw = (n + 4 * kPerMaxWg - 1) / (4 * kPerMaxWg);
        const int waves = (n + a.dpw - 1) / a.dpw;
        a.nwg = (waves + 3) / 4;
        const size_t lds = a.nb <= kPerTable ? (size_t)a.nb * sizeof(double) : 0;
        hipLaunchKernelGGL(per_draw_kernel, dim3(a.nwg), dim3(256), lds, stream, a);
        hipLaunchKernelGGL(per_weight_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace iqlh
