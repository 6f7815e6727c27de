// Block-level body of the HER relabelling kernel, shared by its own launch
// and by the merged whole-step launches.  The description of the method and
// of the MI355X layout is in her.hip.
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

constexpr uint64_t kHerKey1 = 0x484552646F6E6F72ull;
constexpr int kHerRows = 32;

// First e in [0, E) with ends[e] > src, or -1 (src past the last end).
IQLH_DEV int find_episode(const int32_t* __restrict__ ends, int E, int64_t src, int64_t size) {
    int64_t e = (src * (int64_t)E) / (size > 0 ? size : 1);
    if (e > E - 1) e = E - 1;
    if (e < 0) e = 0;
    const int64_t hv = ends[e];
    const int64_t lv = e > 0 ? (int64_t)ends[e - 1] : INT64_MIN;
    if (hv > src && lv <= src) return (int)e;
    // binary search for the first end > src in [lo, hi)
    int lo = 0, hi = E;
    if (hv <= src) lo = (int)e + 1;
    else hi = (int)e;
    for (int it = 0; it < 40 && lo < hi; ++it) {
        const int mid = lo + ((hi - lo) >> 1);
        if ((int64_t)ends[mid] > src) hi = mid;
        else lo = mid + 1;
    }
    return lo < E ? lo : -1;
}

constexpr int kHerItems = 8;    // row quads prefetched per thread (S <= 256)
constexpr int kHerGoalLds = 64;  // goal entries staged per row (G <= 64)

// Relabels rows 32 blk .. 32 blk + 31; every thread of a 256-thread block
// takes part.
IQLH_DEV void her_block(const HerArgs& a, int64_t blk) {
    __shared__ int64_t s_don[kHerRows];  // donor row, -1 marks a zeroed row
    __shared__ float s_goal[kHerRows][kHerGoalLds];
    const int tid = threadIdx.x;
    const int64_t row0 = blk * kHerRows;
    const int S = a.S, G = a.G;
    const int nrows = (int)min<int64_t>(kHerRows, a.n - row0);
    const int C4 = (S + 3) / 4;  // column quads per row
    const int items = nrows * C4;
    const bool vec = (S % 4) == 0 && ((uintptr_t)a.states & 15u) == 0 &&
                     ((uintptr_t)a.next_states & 15u) == 0;

    // ---- phase A, every thread: its row quads of s and s' do not depend on
    // the donor, so they are loaded while phase 1 finds it
    float vs[kHerItems][4], vn[kHerItems][4];
#pragma unroll
    for (int k = 0; k < kHerItems; ++k) {
        const int w = tid + 256 * k;
#pragma unroll
        for (int e = 0; e < 4; ++e) vs[k][e] = vn[k][e] = 0.f;
        if (w < items) {
            const int rr = w / C4, c = (w - rr * C4) * 4;
            const int64_t src = a.source_idx[row0 + rr];
            if (src >= 0 && src < a.buffer_size) {
                const float* s_row = a.states + src * S + c;
                const float* n_row = a.next_states + src * S + c;
                if (vec) {
                    const float4 x = *(const float4*)s_row, y = *(const float4*)n_row;
                    vs[k][0] = x.x; vs[k][1] = x.y; vs[k][2] = x.z; vs[k][3] = x.w;
                    vn[k][0] = y.x; vn[k][1] = y.y; vn[k][2] = y.z; vn[k][3] = y.w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        vs[k][e] = c + e < S ? s_row[e] : 0.f;
                        vn[k][e] = c + e < S ? n_row[e] : 0.f;
                    }
                }
            }
        }
    }

    // ---- phase 1, one thread per row: donor, reward, action, done
    if (tid < kHerRows) {
        const int64_t i = row0 + tid;
        int64_t src = -1, donor = -1;
        if (i < a.n) {
            src = a.source_idx[i];
            bool ok = src >= 0 && src < a.buffer_size;
            int32_t act = 0;
            float done = 0.f;
            if (ok) {
                if (a.out_actions) act = a.actions[src];
                if (a.out_dones) done = a.dones[src];
                uint64_t r = 0;
                if (a.strategy != 0) {  // future and random draw one word
                    const uint64_t step = a.d_step ? (uint64_t)(*a.d_step) : 0ull;
                    r = philox4x64_10(u64x4{(uint64_t)i, step, 0ull, 0ull}, a.seed, kHerKey1).x;
                }
                if (a.strategy == 2) {
                    donor = uniform_index(r, 0, (uint64_t)a.buffer_size);
                } else {
                    const int e = find_episode(a.episode_ends, a.num_episodes, src, a.buffer_size);
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
            if (ok) {
                const float* ns = a.next_states + src * S;
                const float* nd = a.next_states + donor * S;
                // both goals in flight at once, then the binary32 sum of
                // squares in goal order (no contraction), correctly rounded
                // square root, strict comparison
                float gs[16], gd[16];
#pragma unroll
                for (int d = 0; d < 16; ++d) {
                    gs[d] = d < G ? ns[d] : 0.f;
                    gd[d] = d < G ? nd[d] : 0.f;
                }
                float acc = 0.f;
#pragma unroll
                for (int d = 0; d < 16; ++d) {
                    if (d < G) {
                        const float diff = __fsub_rn(gs[d], gd[d]);
                        acc = __fadd_rn(acc, __fmul_rn(diff, diff));
                    }
                }
                for (int d = 16; d < G; ++d) {
                    const float diff = __fsub_rn(ns[d], nd[d]);
                    acc = __fadd_rn(acc, __fmul_rn(diff, diff));
                }
#pragma unroll
                for (int d = 0; d < 16; ++d)
                    if (d < G) s_goal[tid][d] = gd[d];
                for (int d = 16; d < G && d < kHerGoalLds; ++d) s_goal[tid][d] = nd[d];
                const float dist = __fsqrt_rn(acc);
                a.out_rewards[i] = dist < a.threshold ? a.reward_hit : a.reward_miss;
                if (a.donor_out) a.donor_out[i] = (int32_t)donor;
                if (a.out_actions) a.out_actions[i] = act;
                if (a.out_dones) a.out_dones[i] = done;
            } else {
                src = -1;
                donor = -1;
                a.out_rewards[i] = 0.f;
                if (a.donor_out) a.donor_out[i] = -1;
                if (a.out_actions) a.out_actions[i] = 0;
                if (a.out_dones) a.out_dones[i] = 0.f;
                set_flag(a.flags, 0x2);
            }
        }
        s_don[tid] = donor < 0 ? -1 : donor;
    }
    __syncthreads();

    // ---- phase B: goal replacement and stores
    const int64_t ld = a.out_ld;
    auto emit = [&](int w, float* xs, float* xn) {
        const int rr = w / C4, c = (w - rr * C4) * 4;
        const int64_t i = row0 + rr, don = s_don[rr];
        if (don < 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[e] = xn[e] = 0.f;
        } else if (c < G) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = c + e;
                if (d < G) xs[e] = xn[e] = d < kHerGoalLds ? s_goal[rr][d] : a.next_states[don * S + d];
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (c + e < S) {
                if (a.out_bf16) ((uint16_t*)a.out_states)[i * ld + c + e] = f2bf(xs[e]);
                else ((float*)a.out_states)[i * ld + c + e] = xs[e];
                if (a.out_next_states) a.out_next_states[i * S + c + e] = xn[e];
            }
        }
    };
#pragma unroll
    for (int k = 0; k < kHerItems; ++k) {
        const int w = tid + 256 * k;
        if (w < items) emit(w, vs[k], vn[k]);
    }
    // rows wider than the prefetch (S > 256): remaining quads, loaded here
    for (int w = tid + 256 * kHerItems; w < items; w += 256) {
        const int rr = w / C4, c = (w - rr * C4) * 4;
        const int64_t src = a.source_idx[row0 + rr];
        float xs[4] = {0.f, 0.f, 0.f, 0.f}, xn[4] = {0.f, 0.f, 0.f, 0.f};
        if (src >= 0 && src < a.buffer_size) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xs[e] = c + e < S ? a.states[src * S + c + e] : 0.f;
                xn[e] = c + e < S ? a.next_states[src * S + c + e] : 0.f;
            }
        }
        emit(w, xs, xn);
    }
}

}  // namespace iqlh
