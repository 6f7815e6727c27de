// Measurement probes behind design decisions of the forward/backward launch.
// They are not part of the step: bench.py runs them (`--probe NAME`) so that
// the figures quoted for these decisions can be reproduced.  Built into their
// own library, libiqlh_probes.so.
//
// team_fold: whether the split-K gradient partials of the forward/backward
//   launch could be summed inside that launch instead of by the next one.
//   256 workgroups of 1024 threads, each holding 150 KB of LDS (one per CU,
//   like the forward/backward kernel), each write one partial row of PP
//   floats.  Three variants:
//     base     rows only; a separate launch sums the 128 rows of each group
//              in the reduction's order (slice sl adds rows sl, sl + 8, ...,
//              the eight slice sums are then added in slice order);
//     fold_all rows, then a team of the 16 workgroups whose rows one slice
//              adds (same group, tile index = x mod 8) meet at a counter:
//              each thread releases at agent scope, one thread of each
//              workgroup arrives and waits (bounded); member m then adds
//              its 1/16 of the team's rows in the slice's order, and the
//              next launch adds the eight team rows in slice order;
//     fold_t0  as fold_all with one agent-scope release per workgroup.
//   The three sums are compared bit for bit.
// xcc_map: the XCC (XCD) each block of a launch runs on, from the hardware
//   register, for a launch of the forward/backward kernel's shape.
// stream_sum: sums of squares of four float arrays of n elements (a read-only
//   streaming reduction, the gradient budget's first pass) with three ways of
//   cutting the work into 256-thread blocks: a persistent grid of nb blocks
//   striding over the arrays (block b, thread t takes quads b 256 + t +
//   i nb 256); the same grid with each block owning one contiguous range;
//   and one block per 8 KB of each array (no loop).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <vector>

namespace {

constexpr int kNwg = 256, kG = 2, kTiles = 128, kPP = 33280, kTeam = 16, kTeams = kG * 8;
constexpr int kLds = 150 * 1024;
typedef float f4 __attribute__((ext_vector_type(4)));

// block -> (group, tile) as in the forward/backward launch: tiles 64..127
// first, then 0..63; runs of 8 tiles take 16 blocks, group-major
__device__ void map_block(int L, int& g, int& wg) {
    const int first = L < kNwg / 2;
    const int h = first ? L : L - kNwg / 2, t0 = first ? kTiles / 2 : 0;
    const int run = h / 16, r = h % 16;
    g = r / 8;
    wg = t0 + 8 * run + r % 8;
}

__device__ __forceinline__ float row_value(int row, int i) {
    return (float)((row * 7 + i * 13) % 1000) * 1e-3f - 0.5f;
}

__device__ void write_row(float* rows, int row) {
    extern __shared__ float lds[];
    f4* dst = (f4*)(rows + (int64_t)row * kPP);
    for (int i = threadIdx.x; i < kPP / 4; i += 1024)
        dst[i] = f4{row_value(row, 4 * i), row_value(row, 4 * i + 1), row_value(row, 4 * i + 2),
                    row_value(row, 4 * i + 3)};
    if (threadIdx.x == 0) lds[0] = 0.f;  // the LDS is held, not used
}

__global__ __launch_bounds__(1024) void probe_write_kernel(float* rows) {
    int g, wg;
    map_block(blockIdx.x, g, wg);
    write_row(rows, g * kTiles + wg);
}

// counters: [kTeams] arrivals, [kTeams] departures, [1] timed-out flag.  The
// last member to depart resets its team's two counters, so every launch
// starts from zero; a member that waits longer than `limit` ticks of the
// 100 MHz clock skips its share and raises the flag.
template <bool ALL_RELEASE>
__global__ __launch_bounds__(1024) void probe_write_fold_kernel(float* rows, float* team_rows, int* cnt,
                                                                long long limit) {
    __shared__ int s_ok;
    int g, wg;
    map_block(blockIdx.x, g, wg);
    write_row(rows, g * kTiles + wg);
    const int x = wg % 8, member = wg / 8, team = g * 8 + x;
    if (ALL_RELEASE) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    if (threadIdx.x == 0) {
        if (!ALL_RELEASE) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        __hip_atomic_fetch_add(cnt + team, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const long long t0 = __builtin_amdgcn_s_memrealtime();
        int ok = 1;
        while (__hip_atomic_load(cnt + team, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < kTeam) {
            if (__builtin_amdgcn_s_memrealtime() - t0 > limit) {
                ok = 0;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        s_ok = ok;
    }
    __syncthreads();
    if (s_ok) {
        constexpr int per = kPP / 4 / kTeam;  // quads per member
        for (int i = threadIdx.x; i < per; i += 1024) {
            const int64_t c = (int64_t)member * per + i;
            f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < kTeam; ++k) acc += ((const f4*)(rows + (int64_t)(g * kTiles + x + 8 * k) * kPP))[c];
            ((f4*)(team_rows + (int64_t)team * kPP))[c] = acc;
        }
    } else if (threadIdx.x == 0) {
        __hip_atomic_store(cnt + 2 * kTeams, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int d = __hip_atomic_fetch_add(cnt + kTeams + team, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == kTeam - 1) {
            __hip_atomic_store(cnt + team, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(cnt + kTeams + team, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <bool TEAM>
__global__ __launch_bounds__(256) void probe_sum_kernel(const float* rows, const float* team_rows, float* out) {
    __shared__ f4 red[8][32];
    const int g = blockIdx.y, tid = threadIdx.x, q = tid % 32, sl = tid / 32;
    const int64_t p = (int64_t)blockIdx.x * 128 + 4 * q;
    f4 acc = {0.f, 0.f, 0.f, 0.f};
    if (TEAM) {
        acc = *(const f4*)(team_rows + (int64_t)(g * 8 + sl) * kPP + p);
    } else {
#pragma unroll 16
        for (int w = sl; w < kTiles; w += 8) acc += *(const f4*)(rows + (int64_t)(g * kTiles + w) * kPP + p);
    }
    red[sl][q] = acc;
    __syncthreads();
    if (sl == 0) {
        f4 s = red[0][q];
#pragma unroll
        for (int i = 1; i < 8; ++i) s += red[i][q];
        *(f4*)(out + (int64_t)g * kPP + p) = s;
    }
}

__global__ __launch_bounds__(1024) void probe_xcc_kernel(int* out) {
    extern __shared__ float lds[];
    if (threadIdx.x == 0) {
        unsigned v;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
        out[blockIdx.x] = (int)(v & 15u);
        lds[0] = 0.f;
    }
}

// four arrays, n a multiple of 4 * 256 * nb
__global__ __launch_bounds__(256) void probe_sum_stride_kernel(const float* const* a, int64_t quads, float* out) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < quads; q += stride) {
        f4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = ((const f4*)a[j])[q];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += x[j].x * x[j].x + x[j].y * x[j].y + x[j].z * x[j].z + x[j].w * x[j].w;
    }
    if (acc[0] + acc[1] + acc[2] + acc[3] == -1.f) out[0] = 1.f;  // keeps the loads
}
__global__ __launch_bounds__(256) void probe_sum_chunk_kernel(const float* const* a, int64_t quads, float* out) {
    const int64_t chunk = quads / gridDim.x, q0 = (int64_t)blockIdx.x * chunk;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t q = q0 + threadIdx.x; q < q0 + chunk; q += 256) {
        f4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = ((const f4*)a[j])[q];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += x[j].x * x[j].x + x[j].y * x[j].y + x[j].z * x[j].z + x[j].w * x[j].w;
    }
    if (acc[0] + acc[1] + acc[2] + acc[3] == -1.f) out[0] = 1.f;
}
// one block per 512 quads of one array (blockIdx.y = the array)
__global__ __launch_bounds__(256) void probe_sum_piece_kernel(const float* const* a, int64_t quads, float* out) {
    const f4* p = (const f4*)a[blockIdx.y] + (int64_t)blockIdx.x * 512;
    const f4 x0 = p[threadIdx.x], x1 = p[threadIdx.x + 256];
    const float acc = x0.x * x0.x + x0.y * x0.y + x0.z * x0.z + x0.w * x0.w + x1.x * x1.x + x1.y * x1.y +
                      x1.z * x1.z + x1.w * x1.w;
    if (acc == -1.f) out[0] = 1.f;
}

#define PCK(x)                                   \
    do {                                         \
        hipError_t e_ = (x);                     \
        if (e_ != hipSuccess) return (int)e_;    \
    } while (0)

}  // namespace

extern "C" {

// out_us[0..8]: for base, fold_all, fold_t0 in turn, the mean time (us) of
// the row launch alone, of the sum launch alone, and of the pair, each over
// `reps` back-to-back launches.  out_equal[0..1]: fold_all's and fold_t0's sums
// equal base's bit for bit.  out_timeouts: waits that hit the limit.
int iqlh_probe_team_fold(int reps, double* out_us, int* out_equal, int* out_timeouts) {
    if (reps < 1 || !out_us || !out_equal || !out_timeouts) return -1;
    float *rows = nullptr, *team_rows = nullptr, *sum[3] = {nullptr, nullptr, nullptr};
    int* cnt = nullptr;
    PCK(hipMalloc(&rows, sizeof(float) * kG * kTiles * kPP));
    PCK(hipMalloc(&team_rows, sizeof(float) * kTeams * kPP));
    for (auto& s : sum) PCK(hipMalloc(&s, sizeof(float) * kG * kPP));
    PCK(hipMalloc(&cnt, sizeof(int) * (2 * kTeams + 1)));
    PCK(hipMemset(cnt, 0, sizeof(int) * (2 * kTeams + 1)));
    PCK(hipFuncSetAttribute((const void*)probe_write_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kLds));
    PCK(hipFuncSetAttribute((const void*)probe_write_fold_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kLds));
    PCK(hipFuncSetAttribute((const void*)probe_write_fold_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kLds));
    const long long limit = 200000;  // 2 ms
    auto first = [&](int v) {
        if (v == 0) hipLaunchKernelGGL(probe_write_kernel, dim3(kNwg), dim3(1024), kLds, 0, rows);
        else if (v == 1)
            hipLaunchKernelGGL(probe_write_fold_kernel<true>, dim3(kNwg), dim3(1024), kLds, 0, rows, team_rows, cnt,
                               limit);
        else
            hipLaunchKernelGGL(probe_write_fold_kernel<false>, dim3(kNwg), dim3(1024), kLds, 0, rows, team_rows, cnt,
                               limit);
    };
    auto second = [&](int v) {
        if (v == 0) hipLaunchKernelGGL(probe_sum_kernel<false>, dim3(kPP / 128, kG), dim3(256), 0, 0, rows, team_rows,
                                       sum[0]);
        else hipLaunchKernelGGL(probe_sum_kernel<true>, dim3(kPP / 128, kG), dim3(256), 0, 0, rows, team_rows, sum[v]);
    };
    hipEvent_t e0, e1;
    PCK(hipEventCreate(&e0));
    PCK(hipEventCreate(&e1));
    auto timed = [&](int v, int what, double* us) -> int {
        for (int i = 0; i < 3; ++i) {  // warm-up
            if (what != 1) first(v);
            if (what != 0) second(v);
        }
        PCK(hipEventRecord(e0, 0));
        for (int i = 0; i < reps; ++i) {
            if (what != 1) first(v);
            if (what != 0) second(v);
        }
        PCK(hipEventRecord(e1, 0));
        PCK(hipEventSynchronize(e1));
        float ms = 0.f;
        PCK(hipEventElapsedTime(&ms, e0, e1));
        *us = 1e3 * ms / reps;
        return 0;
    };
    for (int v = 0; v < 3; ++v) {
        // the sum launch alone re-reads what the last row launch left
        for (int what = 0; what < 3; ++what) {
            const int r = timed(v, what, out_us + 3 * v + what);
            if (r) return r;
        }
    }
    PCK(hipDeviceSynchronize());
    std::vector<float> a((size_t)kG * kPP), b((size_t)kG * kPP);
    PCK(hipMemcpy(a.data(), sum[0], a.size() * sizeof(float), hipMemcpyDeviceToHost));
    for (int v = 1; v < 3; ++v) {
        PCK(hipMemcpy(b.data(), sum[v], b.size() * sizeof(float), hipMemcpyDeviceToHost));
        out_equal[v - 1] = memcmp(a.data(), b.data(), a.size() * sizeof(float)) == 0;
    }
    PCK(hipMemcpy(out_timeouts, cnt + 2 * kTeams, sizeof(int), hipMemcpyDeviceToHost));
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    hipFree(rows);
    hipFree(team_rows);
    for (auto& s : sum) hipFree(s);
    hipFree(cnt);
    return 0;
}

// out_us[0..2]: mean time of the strided, chunked and per-piece sums of four
// arrays of n floats (n a multiple of 2^21), each over `reps` back-to-back
// launches after one warm-up; nb = blocks of the first two.
int iqlh_probe_stream_sum(int64_t n, int nb, int reps, double* out_us) {
    if (n < (1 << 21) || (n & ((1 << 21) - 1)) || nb < 1 || nb > 8192 || reps < 1 || !out_us) return -1;
    const int64_t quads = n / 4;
    if (quads % ((int64_t)nb * 256) != 0) return -1;
    float* arr[4] = {nullptr, nullptr, nullptr, nullptr};
    float* out = nullptr;
    const float** dptr = nullptr;
    for (auto& x : arr) {
        PCK(hipMalloc(&x, sizeof(float) * n));
        PCK(hipMemset(x, 0, sizeof(float) * n));
    }
    PCK(hipMalloc(&out, sizeof(float)));
    PCK(hipMalloc(&dptr, sizeof(arr)));
    PCK(hipMemcpy(dptr, arr, sizeof(arr), hipMemcpyHostToDevice));
    hipEvent_t e0, e1;
    PCK(hipEventCreate(&e0));
    PCK(hipEventCreate(&e1));
    for (int v = 0; v < 3; ++v) {
        auto launch = [&]() {
            if (v == 0) hipLaunchKernelGGL(probe_sum_stride_kernel, dim3(nb), dim3(256), 0, 0, dptr, quads, out);
            else if (v == 1) hipLaunchKernelGGL(probe_sum_chunk_kernel, dim3(nb), dim3(256), 0, 0, dptr, quads, out);
            else hipLaunchKernelGGL(probe_sum_piece_kernel, dim3((unsigned)(quads / 512), 4), dim3(256), 0, 0, dptr,
                                    quads, out);
        };
        launch();
        PCK(hipEventRecord(e0, 0));
        for (int i = 0; i < reps; ++i) launch();
        PCK(hipEventRecord(e1, 0));
        PCK(hipEventSynchronize(e1));
        float ms = 0.f;
        PCK(hipEventElapsedTime(&ms, e0, e1));
        out_us[v] = 1e3 * ms / reps;
    }
    hipEventDestroy(e0);
    hipEventDestroy(e1);
    for (auto& x : arr) hipFree(x);
    hipFree(out);
    hipFree(dptr);
    return 0;
}

// out_xcc[b] = the XCC that block b of a launch of `blocks` blocks of 1024
// threads with `lds_bytes` of dynamic LDS ran on.
int iqlh_probe_xcc_map(int blocks, int lds_bytes, int* out_xcc) {
    if (blocks < 1 || blocks > 65536 || lds_bytes < 4 || lds_bytes > 160 * 1024 || !out_xcc) return -1;
    int* d = nullptr;
    PCK(hipMalloc(&d, sizeof(int) * blocks));
    PCK(hipFuncSetAttribute((const void*)probe_xcc_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes));
    hipLaunchKernelGGL(probe_xcc_kernel, dim3(blocks), dim3(1024), lds_bytes, 0, d);
    PCK(hipGetLastError());
    PCK(hipMemcpy(out_xcc, d, sizeof(int) * blocks, hipMemcpyDeviceToHost));
    hipFree(d);
    return 0;
}

}  // extern "C"
