// HER goal relabelling with sparse-reward recomputation, gfx950.
//
// Follows "GPU IQL + HER Porting Plan": section "CUDA Kernel:
// her_relabel_kernel.cu" (copy s and s' of the source, overwrite the goal
// entries of both with the donor's next-state goal, copy action and done,
// reward from the Euclidean goal distance against the threshold) and section
// "Donor Index Generation" (final / future / random donors).
//
// MI355X layout: one wave64 per relabelled row.  The wave finds the source's
// episode with a 64-ary search (each lane probes one position, a ballot picks
// the segment), so a 16k-episode table takes three dependent loads instead of
// fourteen; the row copy is a coalesced 64-lane sweep; the relabelled state is
// written straight into the caller's merged batch (bf16 or f32), which removes
// the page's staging buffers and the D2D concatenation.
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

constexpr uint64_t kHerKey1 = 0x484552646F6E6F72ull;

// First e in [0, E) with ends[e] > src, or -1.  All 64 lanes call it with the
// same arguments; every branch is wave-uniform.
//
// Round 0 probes the 64 episodes around the interpolation guess
// src * E / buffer_size; when the answer lies strictly inside that window it
// is found in one memory round trip (always, for equal-length episodes).
// Otherwise the window's ballot still narrows the range before the 64-ary
// search continues.
IQLH_DEV int find_episode(const int32_t* __restrict__ ends, int E, int64_t src, int64_t size,
                          int lane) {
    int lo = 0, hi = E - 1;  // answer in [lo, hi] if one exists
    {
        int64_t gs = (src * (int64_t)E) / (size > 0 ? size : 1) - 31;
        if (gs > (int64_t)E - 64) gs = (int64_t)E - 64;
        if (gs < 0) gs = 0;
        const int p = (int)gs + lane;
        const bool pred = p < E && (int64_t)ends[p < E ? p : E - 1] > src;
        const uint64_t m = __ballot(pred);
        const int c = __popcll(~m & (E - (int)gs >= 64 ? ~0ull : ((1ull << (E - (int)gs)) - 1ull)));
        // lanes [0, c) hold ends <= src, lanes [c, ...) ends > src
        if (c > 0) lo = (int)gs + c;          // ends[gs + c - 1] <= src
        if ((int)gs + c < E && c < 64) hi = (int)gs + c;  // ends[gs + c] > src
        if (c == 0) hi = (int)gs;
        if (lo > hi) lo = hi;  // source past the last end: checked below
    }
    for (int it = 0; it < 64 && lo < hi; ++it) {
        const int64_t span = (int64_t)(hi - lo) + 1;
        const int p = lo + (int)((span * lane) >> 6);
        const bool pred = (int64_t)ends[p] > src;
        const uint64_t m = __ballot(pred);
        const int c = 64 - __popcll(m);  // lanes whose probe is still <= src
        if (c == 0) {
            hi = lo;
        } else {
            const int nlo = lo + (int)((span * (c - 1)) >> 6) + 1;
            if (c < 64) hi = lo + (int)((span * c) >> 6);
            lo = nlo;
        }
    }
    if (lo >= E || (int64_t)ends[lo] <= src || (lo > 0 && (int64_t)ends[lo - 1] > src)) return -1;
    return lo;
}

constexpr int kRowRegs = 4;  // source-row columns held per lane (S <= 256)

__global__ __launch_bounds__(256) void her_relabel_kernel(HerArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= a.n) return;  // wave-uniform
    const int S = a.S, G = a.G;
    const uint64_t step = a.d_step ? (uint64_t)(*a.d_step) : 0ull;
    const int64_t src = a.source_idx[i];
    bool ok = src >= 0 && src < a.buffer_size;
    const float* __restrict__ s_src = a.states + (ok ? src : 0) * S;
    const float* __restrict__ n_src = a.next_states + (ok ? src : 0) * S;
    // The source row does not depend on the donor: issue its loads first so
    // they overlap the random draw and the episode search.
    float sv[kRowRegs], nv[kRowRegs];
#pragma unroll
    for (int r = 0; r < kRowRegs; ++r) {
        const int d = lane + 64 * r;
        sv[r] = (ok && d < S) ? s_src[d] : 0.f;
        nv[r] = (ok && d < S) ? n_src[d] : 0.f;
    }
    const int32_t act = (ok && a.out_actions) ? a.actions[src] : 0;
    const float done = (ok && a.out_dones) ? a.dones[src] : 0.f;
    int64_t donor = -1;
    if (ok) {
        uint64_t r = 0;
        if (a.strategy != 0) {  // future and random draw one word
            u64x4 c = philox4x64_10(u64x4{(uint64_t)i, step, 0ull, 0ull}, a.seed, kHerKey1);
            r = c.x;
        }
        if (a.strategy == 2) {
            donor = uniform_index(r, 0, (uint64_t)a.buffer_size);
        } else {
            const int e = find_episode(a.episode_ends, a.num_episodes, src, a.buffer_size, lane);
            if (e < 0) {
                ok = false;
            } else {
                const int64_t end = a.episode_ends[e];
                if (a.strategy == 0) {
                    donor = end - 1;
                } else {
                    const int64_t span = end - src - 1;
                    donor = span > 0 ? uniform_index(r, src + 1, (uint64_t)span) : src;
                }
            }
        }
        if (donor < 0 || donor >= a.buffer_size) ok = false;
    }

    const int64_t ld = a.out_ld;
    if (!ok) {
        for (int d = lane; d < S; d += 64) {
            if (a.out_bf16) ((uint16_t*)a.out_states)[i * ld + d] = 0;
            else ((float*)a.out_states)[i * ld + d] = 0.f;
            if (a.out_next_states) a.out_next_states[i * S + d] = 0.f;
        }
        if (lane == 0) {
            if (a.donor_out) a.donor_out[i] = -1;
            if (a.out_actions) a.out_actions[i] = 0;
            if (a.out_dones) a.out_dones[i] = 0.f;
            a.out_rewards[i] = 0.f;
            set_flag(a.flags, 0x2);
        }
        return;
    }

    const float* __restrict__ n_don = a.next_states + donor * S;
    const float dg = lane < G ? n_don[lane] : 0.f;  // donor goal, column = lane
    auto put = [&](int d, float vs, float vn) {
        if (a.out_bf16) ((uint16_t*)a.out_states)[i * ld + d] = f2bf(vs);
        else ((float*)a.out_states)[i * ld + d] = vs;
        if (a.out_next_states) a.out_next_states[i * S + d] = vn;
    };
#pragma unroll
    for (int r = 0; r < kRowRegs; ++r) {
        const int d = lane + 64 * r;
        if (d < S) {
            const float gv = d < G ? (r == 0 ? dg : n_don[d]) : 0.f;
            put(d, d < G ? gv : sv[r], d < G ? gv : nv[r]);
        }
    }
    for (int d = lane + 64 * kRowRegs; d < S; d += 64) {
        const float gv = d < G ? n_don[d] : 0.f;
        put(d, d < G ? gv : s_src[d], d < G ? gv : n_src[d]);
    }
    // Binary32 sum of squares in goal order, no contraction, correctly rounded
    // square root, strict comparison.  Goal d < 64 sits in lane d.
    float acc = 0.f;
    for (int d = 0; d < G; ++d) {
        const float x = d < 64 ? __shfl(nv[0], d, 64) : n_src[d];
        const float y = d < 64 ? __shfl(dg, d, 64) : n_don[d];
        const float diff = __fsub_rn(x, y);
        acc = __fadd_rn(acc, __fmul_rn(diff, diff));
    }
    if (lane == 0) {
        const float dist = __fsqrt_rn(acc);
        a.out_rewards[i] = dist < a.threshold ? a.reward_hit : a.reward_miss;
        if (a.donor_out) a.donor_out[i] = (int32_t)donor;
        if (a.out_actions) a.out_actions[i] = act;
        if (a.out_dones) a.out_dones[i] = done;
    }
}

hipError_t launch_her_relabel(const HerArgs& a, hipStream_t stream) {
    if (a.n <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((a.n + 3) / 4);
    hipLaunchKernelGGL(her_relabel_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace iqlh
