// Block-level body of the HER relabelling kernel, shared by its own launch
// and by the merged whole-step launches.  The description of the method and
// of the MI355X layout is in her.hip.
#pragma once
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

constexpr uint64_t kHerKey1 = 0x484552646F6E6F72ull;
constexpr int kHerRows = 32;

// Episode lookup in two halves, so that its loads can be issued early and
// consumed late: the probe at the interpolation guess src * E / size (two
// loads; it hits at once for equal-length episodes), then the resolution
// (a bounded binary search when the probe missed).
struct EpisodeProbe {
    int64_t e;
    int32_t hv, lv;  // raw ends[e] and ends[max(e - 1, 0)]: consumed only when resolving
};
IQLH_DEV EpisodeProbe probe_episode(const int32_t* __restrict__ ends, int E, int64_t src, int64_t size) {
    // the guess need not be exact (resolution is), so a double product
    // replaces the 64-bit integer division
    int64_t e = (int64_t)((double)src * (double)E / (double)(size > 0 ? size : 1));
    if (e > E - 1) e = E - 1;
    if (e < 0) e = 0;
    EpisodeProbe p;
    p.e = e;
    p.hv = ends[e];
    p.lv = ends[e > 0 ? e - 1 : 0];
    return p;
}
// First e in [0, E) with ends[e] > src, or -1 (src past the last end).
IQLH_DEV int resolve_episode(const int32_t* __restrict__ ends, int E, int64_t src, const EpisodeProbe& p) {
    const int64_t hv = p.hv, lv = p.e > 0 ? (int64_t)p.lv : INT64_MIN;
    if (hv > src && lv <= src) return (int)p.e;
    int lo = 0, hi = E;
    if (hv <= src) lo = (int)p.e + 1;
    else hi = (int)p.e;
    for (int it = 0; it < 40 && lo < hi; ++it) {
        const int mid = lo + ((hi - lo) >> 1);
        if ((int64_t)ends[mid] > src) hi = mid;
        else lo = mid + 1;
    }
    return lo < E ? lo : -1;
}

constexpr int kHerItems = 8;    // row quads prefetched per thread (S <= 256)
constexpr int kHerGoalLds = 64;  // goal entries staged per row (G <= 64)

// The random word of relabelled row i: word 0 of Philox4x64-10 at counter
// (i, step, 0, 0) under the key (seed, kHerKey1); 0 for "final", which draws
// nothing.  It does not depend on the source row, so callers compute it
// while the source index is still in flight.
IQLH_DEV uint64_t her_draw(const HerArgs& a, int64_t i, uint64_t step) {
    if (a.strategy == 0) return 0ull;
    return philox4x64_10(u64x4{(uint64_t)i, step, 0ull, 0ull}, a.seed, kHerKey1).x;
}

// The step word of the draws (the device step counter, 0 without one).
IQLH_DEV uint64_t her_step_word(const HerArgs& a) { return a.d_step ? (uint64_t)(*a.d_step) : 0ull; }

// Donor of a relabelled row whose source src lies in [0, buffer_size), from
// its random word r and its episode probe (unused by "random"): "final"
// takes the last transition of src's episode, "future" a uniform draw from
// the transitions after src in its episode (src itself when there is none),
// "random" a uniform draw from the whole buffer.  False when the episode
// lookup fails or the donor falls outside the buffer (malformed episode
// ends).
IQLH_DEV bool her_donor(const HerArgs& a, int64_t src, uint64_t r, const EpisodeProbe& p, int64_t& donor) {
    if (a.strategy == 2) {
        donor = uniform_index(r, 0, (uint64_t)a.buffer_size);
    } else {
        const int e = resolve_episode(a.episode_ends, a.num_episodes, src, p);
        if (e < 0) return false;
        const int64_t end = e == p.e ? (int64_t)p.hv : (int64_t)a.episode_ends[e];
        if (a.strategy == 0) {
            donor = end - 1;
        } else {
            const int64_t span = end - src - 1;
            donor = span > 0 ? uniform_index(r, src + 1, (uint64_t)span) : src;
        }
    }
    return donor >= 0 && donor < a.buffer_size;
}

// Probe of src's episode (src clamped into the buffer: the result of an
// invalid source is never used).  "random" needs no episode and may come
// without episode ends: its probe reads a word of the source indices
// instead and ignores it, so the loads never sit behind a branch.
IQLH_DEV EpisodeProbe her_probe(const HerArgs& a, int64_t src) {
    const bool episodes = a.strategy != 2 && a.episode_ends != nullptr;  // uniform
    const int32_t* ends = episodes ? a.episode_ends : a.source_idx;
    const int E = episodes ? a.num_episodes : 1;
    const int64_t s = src >= 0 && src < a.buffer_size ? src : 0;
    return probe_episode(ends, E, episodes ? s : 0, episodes ? a.buffer_size : 1);
}

// Goal distance of the sparse reward: binary32 sum of squared differences of
// the first G entries of two next states, in goal order (no contraction),
// then the correctly rounded square root (0 for an empty goal).  gs and gd
// hold the first 16 entries of both goals; entries past 16 are loaded here.
IQLH_DEV float her_distance_loaded(const float* __restrict__ ns, const float* __restrict__ nd, int G,
                                   const float (&gs)[16], const float (&gd)[16]) {
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
    return __fsqrt_rn(acc);
}
// The same with the first 16 entries of both goals loaded together (clamped
// indexes, no branch around a load); the donor's are returned in gd for
// callers that stage them.
IQLH_DEV float her_distance(const float* __restrict__ ns, const float* __restrict__ nd, int G, float (&gd)[16]) {
    if (G <= 0) {
#pragma unroll
        for (int d = 0; d < 16; ++d) gd[d] = 0.f;
        return 0.f;  // empty goal: the square root of an empty sum
    }
    float gs[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) {
        const int dd = min(d, G - 1);
        gs[d] = ns[dd];
        gd[d] = nd[dd];
    }
    return her_distance_loaded(ns, nd, G, gs, gd);
}

// Donor guessed before the episode ends arrive, so that its goal can be
// loaded with them: episodes of equal length size / E put the end of the
// probe's guess e at (e + 1) size / E; "random" needs no episode, so its
// guess is exact.  Clamped into the buffer (the caller loads its goal
// unconditionally and keeps it only when the resolved donor equals it).
IQLH_DEV int64_t her_guess_donor(const HerArgs& a, int64_t src, uint64_t r, const EpisodeProbe& p) {
    int64_t donor;
    if (a.strategy == 2) {
        donor = uniform_index(r, 0, (uint64_t)a.buffer_size);
    } else {
        const int E = a.num_episodes > 0 ? a.num_episodes : 1;
        const int64_t end = (p.e + 1) * a.buffer_size / E;
        if (a.strategy == 0) {
            donor = end - 1;
        } else {
            const int64_t span = end - src - 1;
            donor = span > 0 ? uniform_index(r, src + 1, (uint64_t)span) : src;
        }
    }
    return max<int64_t>(0, min<int64_t>(donor, a.buffer_size - 1));
}

// Relabels rows 32 blk .. 32 blk + 31; every thread of a 256-thread block
// takes part.  A wave waits for a load by draining every load it issued
// before it, so each thread issues its loads in the order it consumes them:
// the source of its lead row (threads 0..31 lead one row each), the sources
// of its row quads, the episode probe, the row quads themselves, then the
// goals; the Philox draw runs while the first loads are in flight.
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

    // (1) the lead row's source
    const bool lead = tid < nrows;
    const int64_t i = row0 + tid;
    const int64_t src = lead ? (int64_t)a.source_idx[i] : -1;
    // (2) the sources of this thread's row quads (indexes clamped: no
    // lane-dependent branch around a load, unused values replaced afterwards;
    // slots beyond the block's quads, as at S = 128, are skipped uniformly)
    int64_t srck[kHerItems];
#pragma unroll
    for (int k = 0; k < kHerItems; ++k)
        srck[k] = 256 * k < items ? a.source_idx[row0 + min(tid + 256 * k, items - 1) / C4] : 0;
    // (3) the draw, while those are in flight
    const uint64_t r = lead ? her_draw(a, i, her_step_word(a)) : 0ull;
    // (4) the lead row's episode probe, action and done
    bool ok = lead && src >= 0 && src < a.buffer_size;
    const EpisodeProbe probe = her_probe(a, lead ? src : 0);
    const int64_t sc = ok ? src : 0;
    const int32_t act = a.out_actions ? a.actions[sc] : 0;  // uniform conditions
    const float done = a.out_dones ? a.dones[sc] : 0.f;
    // (5) the row quads of s and s' (they do not depend on the donor)
    float vs[kHerItems][4], vn[kHerItems][4];
#pragma unroll
    for (int k = 0; k < kHerItems; ++k) {
        if (256 * k >= items) {  // uniform: a slot no quad of this block fills
#pragma unroll
            for (int e = 0; e < 4; ++e) vs[k][e] = vn[k][e] = 0.f;
            continue;
        }
        const int w = tid + 256 * k;
        const int wc = min(w, items - 1);
        const int rr = wc / C4, c = (wc - rr * C4) * 4;
        const bool use = w < items && srck[k] >= 0 && srck[k] < a.buffer_size;
        const int64_t sk = use ? srck[k] : 0;
        const float* s_row = a.states + sk * S;
        const float* n_row = a.next_states + sk * S;
        float x[4], y[4];
        if (vec) {  // uniform
            const float4 x4 = *(const float4*)(s_row + c), y4 = *(const float4*)(n_row + c);
            x[0] = x4.x; x[1] = x4.y; x[2] = x4.z; x[3] = x4.w;
            y[0] = y4.x; y[1] = y4.y; y[2] = y4.z; y[3] = y4.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[e] = s_row[min(c + e, S - 1)];
                y[e] = n_row[min(c + e, S - 1)];
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vs[k][e] = (use && c + e < S) ? x[e] : 0.f;
            vn[k][e] = (use && c + e < S) ? y[e] : 0.f;
        }
    }
    // (6) donor, goals, reward of the lead row
    if (lead) {
        int64_t donor = -1;
        if (ok) ok = her_donor(a, src, r, probe, donor);
        if (ok) {
            const float* ns = a.next_states + src * S;
            const float* nd = a.next_states + donor * S;
            float gd[16];
            const float dist = her_distance(ns, nd, G, gd);
#pragma unroll
            for (int d = 0; d < 16; ++d)
                if (d < G) s_goal[tid][d] = gd[d];
            for (int d = 16; d < G && d < kHerGoalLds; ++d) s_goal[tid][d] = nd[d];
            a.out_rewards[i] = dist < a.threshold ? a.reward_hit : a.reward_miss;
            if (a.donor_out) a.donor_out[i] = (int32_t)donor;
            if (a.out_actions) a.out_actions[i] = act;
            if (a.out_dones) a.out_dones[i] = done;
            if (a.out_isw) a.out_isw[i] = 1.f;
        } else {
            donor = -1;
            a.out_rewards[i] = 0.f;
            if (a.donor_out) a.donor_out[i] = -1;
            if (a.out_actions) a.out_actions[i] = 0;
            if (a.out_dones) a.out_dones[i] = 0.f;
            if (a.out_isw) a.out_isw[i] = 0.f;
            set_flag(a.flags, 0x2);
        }
        s_don[tid] = donor;
    }
    __syncthreads();

    // ---- goal replacement and stores
    const int64_t ld = a.out_ld;
    const bool lds_goals = G <= kHerGoalLds;  // uniform: no global load below
    // whole quads leave as one store per output row (8 bytes of bf16 or 16 of
    // f32 for the state, 16 for s'), not as four element stores each
    const uintptr_t oal = (uintptr_t)a.out_states;
    const bool wide = vec && ld % 4 == 0 && (a.out_bf16 ? (oal & 7u) == 0 : (oal & 15u) == 0) &&
                      ((uintptr_t)a.out_next_states & 15u) == 0;
    auto emit = [&](int w, float* xs, float* xn, bool from_lds) {
        const int rr = w / C4, c = (w - rr * C4) * 4;
        const int64_t row = row0 + rr, don = s_don[rr];
        if (don < 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[e] = xn[e] = 0.f;
        } else if (c < G) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int d = c + e;
                if (d < G) {
                    if (from_lds) xs[e] = xn[e] = s_goal[rr][d];
                    else xs[e] = xn[e] = d < kHerGoalLds ? s_goal[rr][d] : a.next_states[don * S + d];
                }
            }
        }
        if (wide) {  // uniform; S % 4 == 0, so the quad is whole
            if (a.out_bf16)
                *(uint2*)((uint16_t*)a.out_states + row * ld + c) =
                    uint2{pack_bf2(xs[0], xs[1]), pack_bf2(xs[2], xs[3])};
            else
                *(float4*)((float*)a.out_states + row * ld + c) = float4{xs[0], xs[1], xs[2], xs[3]};
            if (a.out_next_states) *(float4*)(a.out_next_states + row * S + c) = float4{xn[0], xn[1], xn[2], xn[3]};
            return;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (c + e < S) {
                if (a.out_bf16) ((uint16_t*)a.out_states)[row * ld + c + e] = f2bf(xs[e]);
                else ((float*)a.out_states)[row * ld + c + e] = xs[e];
                if (a.out_next_states) a.out_next_states[row * S + c + e] = xn[e];
            }
        }
    };
    if (lds_goals) {
#pragma unroll
        for (int k = 0; k < kHerItems; ++k) {
            const int w = tid + 256 * k;
            if (w < items) emit(w, vs[k], vn[k], true);
        }
    } else {
#pragma unroll
        for (int k = 0; k < kHerItems; ++k) {
            const int w = tid + 256 * k;
            if (w < items) emit(w, vs[k], vn[k], false);
        }
    }
    // rows wider than the prefetch (S > 256): remaining quads, loaded here
    for (int w = tid + 256 * kHerItems; w < items; w += 256) {
        const int rr = w / C4, c = (w - rr * C4) * 4;
        const int64_t sk = a.source_idx[row0 + rr];
        float xs[4] = {0.f, 0.f, 0.f, 0.f}, xn[4] = {0.f, 0.f, 0.f, 0.f};
        if (sk >= 0 && sk < a.buffer_size) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xs[e] = c + e < S ? a.states[sk * S + c + e] : 0.f;
                xn[e] = c + e < S ? a.next_states[sk * S + c + e] : 0.f;
            }
        }
        emit(w, xs, xn, false);
    }
}

}  // namespace iqlh
