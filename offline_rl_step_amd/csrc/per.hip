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
// MI355X layout, three launches on a caller workspace; the prefix sums are
// never stored whole:
//   A  fp64 sums of every 256-row sub-block and of every 2048-row block (the
//      block sum adds its eight sub-block sums in order), and the draws'
//      counter words, one per lane, parked in the index and weight outputs;
//   D  each workgroup scans the block sums into a table of block ends in LDS
//      (fixed order); one wave per draw: a 64-ary search of the table (each
//      lane probes one position, a ballot picks the segment), then the
//      block's eight sub-block sums (one load round), then the 256 rows of
//      the sub-block, scanned in registers (the second round).  Two rounds of
//      global loads per draw, and no 8-byte-per-row prefix array to write and
//      read.  The block, sub-block and row prefixes are formed in different
//      orders, so at a boundary they may disagree by a rounding; the draw
//      then takes the last row of positive priority before that boundary,
//      a row on one side of it.  Each workgroup's smallest drawn priority
//      (integer minimum on the bit pattern: order-independent) goes to a slot
//      of its own;
//   W  the weights, from the drawn priorities the draws leave in the weight
//      output, after every block folds the workgroup minima.
// For more than 8192 blocks (2^24 rows) the table does not fit in LDS; a
// one-workgroup launch T then writes it to the workspace and the draws search
// it there.
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

constexpr uint64_t kPerKey1 = 0x5045526472617773ull;  // "PERdraws"
constexpr int kPerBlock = 2048;                        // rows per block of the table
constexpr int kPerSub = 256;                           // rows per sub-block (one wave scans one)
constexpr int kPerSubs = kPerBlock / kPerSub;
constexpr int kPerMaxWg = 2048;  // workgroups of the draw pass (each wave takes ceil(n / 8192) draws)
constexpr int kPerTable = 8192;  // block ends kept in LDS (64 KB): up to 2^24 rows

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
    double* bsum;    // [nb] block sums
    double* ssum;    // [nb][8] sub-block sums
    double* bend;    // [nb] inclusive prefix at each block end (only when nb > kPerTable)
    uint32_t* wgmin; // [nwg] smallest drawn priority (bit pattern) of each draw workgroup
    int vec;         // priorities 16-byte aligned, a whole number of quads
    int nb, nwg, dpw;  // blocks; draw workgroups; draws per wave
};

IQLH_DEV bool bad_priority(float x) { return !(x >= 0.f) || !isfinite(x); }

// One 2048-row block per workgroup: wave w sums sub-blocks w and w + 4, four
// consecutive rows per lane (one 16-byte load when the priorities are
// aligned whole quads), each lane's four in a fixed order and then the 64
// lanes by a butterfly; the block sum adds the eight sub-block sums in order.
// While the rows load, workgroup b evaluates the counter words of draws b,
// b + nb, b + 2 nb, ... one per lane, and parks each in the draw's outputs
// (low half in idx, high half in w), which the draw pass reads and
// overwrites: lane-parallel, instead of every lane of a draw's wave
// evaluating the same word.
__global__ __launch_bounds__(256) void per_block_sums_kernel(PerArgs a) {
    __shared__ double red[kPerSubs];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    float x[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t r0 = (int64_t)blockIdx.x * kPerBlock + (int64_t)(wv + 4 * h) * kPerSub + 4 * lane;
        if (a.vec) {  // uniform: the rows past the end are whole quads
            const float4 v = *(const float4*)(a.p + (r0 < a.size ? r0 : 0));
            x[h][0] = v.x; x[h][1] = v.y; x[h][2] = v.z; x[h][3] = v.w;
#pragma unroll
            for (int e = 0; e < 4; ++e) x[h][e] = keep_if(r0 < a.size, x[h][e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t i = r0 + e;
                x[h][e] = keep_if(i < a.size, a.p[i < a.size ? i : a.size - 1]);
            }
        }
    }
    if (a.n > 0) {
        const uint64_t step = a.step ? (uint64_t)*a.step : 0ull;
        for (int64_t k = (int64_t)threadIdx.x * a.nb + blockIdx.x; k < a.n; k += (int64_t)256 * a.nb) {
            const uint64_t word = philox4x64_10(u64x4{(uint64_t)k, step, 0ull, 0ull}, a.seed, kPerKey1).x;
            a.idx[k] = (int32_t)(uint32_t)word;
            a.w[k] = __uint_as_float((uint32_t)(word >> 32));
        }
    }
    double s[2];
    bool bad = false;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int e = 0; e < 4; ++e) bad |= bad_priority(x[h][e]);
        s[h] = ((double)x[h][0] + (double)x[h][1]) + ((double)x[h][2] + (double)x[h][3]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        s[0] += __shfl_xor(s[0], o, 64);
        s[1] += __shfl_xor(s[1], o, 64);
    }
    if (lane == 0) {
        red[wv] = s[0];
        red[wv + 4] = s[1];
    }
    if (__syncthreads_or(bad) && threadIdx.x == 0) set_flag(a.flags, 0x2);
    if (threadIdx.x < kPerSubs) a.ssum[(int64_t)blockIdx.x * kPerSubs + threadIdx.x] = red[threadIdx.x];
    if (threadIdx.x == 0) {
        double t = 0.0;
#pragma unroll
        for (int k = 0; k < kPerSubs; ++k) t += red[k];
        a.bsum[blockIdx.x] = t;
    }
}

// Inclusive prefix of the nb block sums into out (LDS or global), by the 256
// threads of one workgroup in a fixed order: thread t scans its run of
// ceil(nb / 256) sums sequentially; the run totals are scanned across the
// wave by shuffles and across the waves in order; each value is the run's
// offset plus its running sum.  The first four sums of a run are loaded
// together (adding the zeros past a short run changes no sum).
IQLH_DEV void per_table_scan(const double* __restrict__ bsum, int nb, double* out) {
    __shared__ double wtot[4];
    constexpr int PF = 4;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int run = (nb + 255) / 256, j0 = threadIdx.x * run, j1 = min(j0 + run, nb);
    double pf[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        const double x = bsum[min(j0 + i, nb - 1)];
        pf[i] = j0 + i < j1 ? x : 0.0;
    }
    double t = 0.0;
#pragma unroll
    for (int i = 0; i < PF; ++i) t += pf[i];
    for (int j = j0 + PF; j < j1; ++j) t += bsum[j];
    double incl = t;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const double y = __shfl_up(incl, s, 64);
        if (lane >= s) incl += y;
    }
    if (lane == 63) wtot[wv] = incl;
    __syncthreads();
    double off = __shfl_up(incl, 1, 64);
    if (lane == 0) off = 0.0;
    for (int w = 0; w < wv; ++w) off += wtot[w];
    double r = 0.0;
#pragma unroll
    for (int i = 0; i < PF; ++i) {
        if (j0 + i < j1) {
            r += pf[i];
            out[j0 + i] = off + r;
        }
    }
    for (int j = j0 + PF; j < j1; ++j) {
        r += bsum[j];
        out[j] = off + r;
    }
}

__global__ __launch_bounds__(256) void per_table_kernel(PerArgs a) { per_table_scan(a.bsum, a.nb, a.bend); }

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
        // lane j's and lane j - 1's probe positions, recomputed (uniform)
        // rather than fetched by shuffles
        const int j = __builtin_ctzll(bal);
        const int64_t pj = min(lo + (int64_t)(j + 1) * stp - 1, hi - 1);
        const int64_t pprev = j > 0 ? min(lo + (int64_t)j * stp - 1, hi - 1) : lo - 1;
        hi = pj + 1;
        lo = pprev + 1;
    }
    return hi - lo == 1 ? lo : -1;
}

// The row of one draw inside block blk (its prefix before the block is off):
// the sub-block from the eight sub-block sums, then the row from the
// sub-block's 256 priorities scanned in registers (four rows per lane).
// Returns the row and, in every lane, its priority; u = +inf gives the
// block's last row of positive priority.  Returns -2 for a block of zero sum
// (chosen only at a rounding boundary of the table).
IQLH_DEV int64_t per_find_row(const PerArgs& a, int64_t blk, double off, double u, float& prow) {
    const int lane = threadIdx.x & 63;
    double sv[kPerSubs];
    bool any = false;
#pragma unroll
    for (int k = 0; k < kPerSubs; ++k) {
        sv[k] = a.ssum[blk * kPerSubs + k];
        any |= sv[k] > 0.0;
    }
    if (!any) return -2;  // wave-uniform
    // the sub-block: first whose end prefix exceeds u, else (a rounding
    // boundary) the last of positive sum
    int j = -1, jpos = 0;
    double r = 0.0, rbefore = 0.0;
#pragma unroll
    for (int k = 0; k < kPerSubs; ++k) {
        const double rk = r + sv[k];
        if (j < 0 && sv[k] > 0.0 && off + rk > u) { j = k; rbefore = r; }
        if (sv[k] > 0.0) jpos = k;
        r = rk;
    }
    if (j < 0) {
        j = jpos;
        rbefore = 0.0;
        for (int k = 0; k < j; ++k) rbefore += sv[k];
    }
    const double soff = off + rbefore;
    const int64_t base = blk * kPerBlock + (int64_t)j * kPerSub + 4 * lane;
    float x[4];
    if (a.vec && base + 4 <= a.size) {
        const float4 v4 = *(const float4*)(a.p + base);
        x[0] = v4.x; x[1] = v4.y; x[2] = v4.z; x[3] = v4.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = keep_if(base + e < a.size, a.p[base + e < a.size ? base + e : a.size - 1]);
    }
    double c[4], t = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) { t += (double)x[e]; c[e] = t; }
    double incl = t;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        const double y = __shfl_up(incl, s, 64);
        if (lane >= s) incl += y;
    }
    double ex = __shfl_up(incl, 1, 64);
    if (lane == 0) ex = 0.0;
    // the first row of positive priority whose prefix soff + (ex + c)
    // exceeds u (the lane prefixes are tree sums, so a lane of zero rows may
    // sit an ulp above its predecessor: only lanes with a positive row
    // qualify), else the last row of positive priority
    const bool lpos = x[0] > 0.f || x[1] > 0.f || x[2] > 0.f || x[3] > 0.f;
    const uint64_t above = __ballot(lpos && soff + (ex + c[3]) > u);
    const uint64_t pos = __ballot(lpos);
    int L, e = 3;
    if (above) {
        L = __builtin_ctzll(above);
        int mine = 3;
#pragma unroll
        for (int k = 3; k >= 0; --k)
            if (x[k] > 0.f && soff + (ex + c[k]) > u) mine = k;
        e = __shfl(mine, L, 64);
    } else {
        L = 63 - __builtin_clzll(pos);  // pos != 0: the sub-block's sum is positive
        int mine = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (x[k] > 0.f) mine = k;
        e = __shfl(mine, L, 64);
    }
    const float xs = e == 0 ? x[0] : e == 1 ? x[1] : e == 2 ? x[2] : x[3];
    prow = __shfl(xs, L, 64);
    return blk * kPerBlock + (int64_t)j * kPerSub + 4 * L + e;
}

// Draws of one wave (dpw per wave, four waves per workgroup).
__global__ __launch_bounds__(256, 8) void per_draw_kernel(PerArgs a) {
    extern __shared__ double tbl[];  // [nb] when the table fits in LDS
    const int lane = threadIdx.x & 63;
    const bool staged = a.nb <= kPerTable;
    const int k0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * a.dpw;
    // the draws' counter words, parked in their outputs by the block-sums pass
    auto draw_word = [&](int k) {
        return ((uint64_t)__float_as_uint(a.w[k]) << 32) | (uint64_t)(uint32_t)a.idx[k];
    };
    const uint64_t word0 = draw_word(min(k0, a.n - 1));
    if (staged) per_table_scan(a.bsum, a.nb, tbl);
    __syncthreads();
    const double* gtab = a.bend;
    const double total = staged ? tbl[a.nb - 1] : gtab[a.nb - 1];
    const double cap = __longlong_as_double(__double_as_longlong(total) - 1);  // largest double below a positive total
    const bool ok = total > 0.0 && isfinite(total);
    uint32_t wmin = 0xFFFFFFFFu;  // smallest drawn priority of this wave (bit pattern: p >= 0)
    for (int kk = 0; kk < a.dpw; ++kk) {
        const int k = k0 + kk;
        if (k >= a.n) break;  // wave-uniform
        const uint64_t word = kk == 0 ? word0 : draw_word(k);
        double u = (double)(word >> 11) * 0x1.0p-53 * total;
        if (u > cap) u = cap;
        int64_t found = -1;
        float pf = 0.f;
        if (ok) {
            const int64_t blk = staged ? search64(0, a.nb, u, [&](int64_t i) { return tbl[i]; })
                                       : search64(0, a.nb, u, [&](int64_t i) { return gtab[i]; });
            if (blk >= 0) {
                const double off = blk == 0 ? 0.0 : (staged ? tbl[blk - 1] : gtab[blk - 1]);
                found = per_find_row(a, blk, off, u, pf);
                if (found == -2) {
                    // a block of zero sum: u lies within a rounding of the
                    // boundary before it, so the draw takes the last row of
                    // positive priority before the boundary (a positive block
                    // precedes: the table exceeds u >= 0 at blk, and sums of
                    // zeros are exactly zero)
                    int64_t b = blk - 1;
                    while (b >= 0 && a.bsum[b] == 0.0) --b;  // wave-uniform
                    found = b >= 0 ? per_find_row(a, b, 0.0, INFINITY, pf) : -1;
                }
            }
        }
        if (lane == 0) {
            a.idx[k] = (int32_t)found;
            a.w[k] = found >= 0 ? pf : 0.f;  // the drawn priority, turned into the weight by W
            if (found >= 0) wmin = min(wmin, __float_as_uint(pf));
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

// Weights from the drawn priorities the draw pass left in w, loaded with the
// workgroup minima in one round.
__global__ __launch_bounds__(256) void per_weight_kernel(PerArgs a) {
    __shared__ uint32_t red[4];
    const int k = blockIdx.x * 256 + threadIdx.x;
    const int kc = k < a.n ? k : a.n - 1;
    const int32_t i = a.idx[kc];
    const float pi = a.w[kc];
    uint32_t mn = 0xFFFFFFFFu;
    for (int j = threadIdx.x; j < a.nwg; j += 256) mn = min(mn, a.wgmin[j]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mn;
    __syncthreads();
    mn = min(min(red[0], red[1]), min(red[2], red[3]));
    if (k >= a.n) return;
    float w = 0.f;
    if (i >= 0) w = (float)pow((double)__uint_as_float(mn) / (double)pi, (double)a.beta);
    a.w[k] = w;
}

size_t per_workspace_bytes_for(int64_t size) {
    const int64_t nb = (size + kPerBlock - 1) / kPerBlock;
    return (size_t)(8 * nb * (2 + kPerSubs) + 4 * kPerMaxWg + 255) / 256 * 256;
}

hipError_t launch_per_sample(const float* p, int64_t size, int n, uint64_t seed, const int64_t* d_step, float beta,
                             int32_t* idx, float* w, int32_t* flags, void* workspace, hipStream_t stream) {
    PerArgs a{};
    a.p = p; a.size = size; a.n = n; a.seed = seed; a.step = d_step; a.beta = beta;
    a.idx = idx; a.w = w; a.flags = flags;
    a.nb = (int)((size + kPerBlock - 1) / kPerBlock);
    a.vec = ((uintptr_t)p & 15u) == 0 && size % 4 == 0;
    a.bsum = (double*)workspace;
    a.ssum = a.bsum + a.nb;
    a.bend = a.ssum + (int64_t)a.nb * kPerSubs;
    a.wgmin = (uint32_t*)(a.bend + a.nb);
    hipLaunchKernelGGL(per_block_sums_kernel, dim3(a.nb), dim3(256), 0, stream, a);
    if (n > 0) {
        if (a.nb > kPerTable) hipLaunchKernelGGL(per_table_kernel, dim3(1), dim3(256), 0, stream, a);
        a.dpw = (n + 4 * kPerMaxWg - 1) / (4 * kPerMaxWg);
        const int waves = (n + a.dpw - 1) / a.dpw;
        a.nwg = (waves + 3) / 4;
        const size_t lds = a.nb <= kPerTable ? (size_t)a.nb * sizeof(double) : 0;
        // the staged table takes up to 64 KB of dynamic LDS (plus the
        // kernel's few static words): raise the kernel's limit to that once
        static bool attr_set = false;
        if (!attr_set) {
            const hipError_t e = hipFuncSetAttribute((const void*)per_draw_kernel,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)(kPerTable * sizeof(double)));
            if (e != hipSuccess) return e;
            attr_set = true;
        }
        hipLaunchKernelGGL(per_draw_kernel, dim3(a.nwg), dim3(256), lds, stream, a);
        hipLaunchKernelGGL(per_weight_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace iqlh
