// IQL value-network forward/backward for wide hidden layers (bf16 operands,
// hidden 256 or 512, state_dim a multiple of 32), e.g. batch 65536, state 256,
// hidden 512.  Same arithmetic as the fused kernel ("GPU IQL + HER Porting
// Plan", section "Current State / IQL (CPU)"; the backward products of "Phase
// 2: Multi-Stream Graph Parallelism", section "2C. Grouped GEMM for IQL"):
//
//   fwd2   for all H features of a 128-sample block: h1 = relu(W1 s + b1),
//          kept in LDS (and stored -> H1 [B][H] bf16 for wgrad) with
//          relu'(z1) as bits; z2 = W2 h1 + b2 from that tile, then in the
//          epilogue v = w3 . relu(z2) + b3, the expectile loss, dv,
//          dz2 = dv w3 relu'(z2) -> DZ2 [B][H] bf16, and the block's sums of
//          dz2 (db2), dv relu(z2) (dw3) and dv (db3); in training the same
//          workgroup goes on with dh1 = W2^T dz2 from its dz2 tile in LDS,
//          dz1 = dh1 relu'(z1) -> DZ1 [B][H] bf16 and the block's db1 sums
//   wgrad  dW2 = dz2^T h1, dW1 = dz1^T s over chunks of samples, one fp32
//          partial row per chunk; the jobs of a chunk also add its block
//          sums (db2, dw3, db3, db1) into the same row
//
// then the fixed-order partial reduction and Adam shared with the other
// paths (no float atomics anywhere).
//
// MI355X design.  Every product runs on v_mfma_f32_16x16x32_bf16, with
// eight waves per workgroup (two per SIMD, so that one wave's dependent
// epilogue arithmetic and LDS round trips overlap the other's MFMAs) and
// one workgroup per CU: wgrad splits its 256 x 256 tile into 128 x 64 wave
// tiles, fwd2 its H x 128 tile into H / 8 features per wave.  Streamed
// operands go HBM -> LDS with global_load_lds_dwordx4 (no register staging)
// through a ring of 32-k stages; each stage ends in one s_barrier after the
// wave's own vmcnt wait, and the fragments of the next stage are read from
// LDS while the current stage's MFMAs run.  The products whose B operand is
// a tile already in LDS (z2 = W2 h1, dh1 = W2^T dz2) take their A operand
// (weights, L2-resident) straight from global memory into registers, one
// k-step ahead.  Activations are row-major [sample][feature]:
//   * in the ring's forward product k is the feature (contiguous): LDS rows
//     of 32 k (64 bytes), the 16-byte unit u of row r stored at
//     u ^ ((r >> 1) & 3), read with ds_read_b128 (conflict-free);
//   * in the weight gradients k is the sample: LDS keeps the natural
//     [sample][feature] rows (512 bytes), unit v of sample s stored at
//     v ^ (2 (s & 3)), and the MFMA operands are read with the LDS transpose
//     load ds_read_b64_tr_b16, so no transposed copy of an activation is
//     ever written.
// The product orientation is D[feature][sample], so a lane ends with four
// consecutive features of one sample: bias, ReLU masks and the bf16 stores
// work on 8-byte runs of a row.
#include "aw_block.hpp"
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace iqlh {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float bf2f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
#define IQLH_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int kThreads = 256;
constexpr int kBK = 32;           // k per stage
constexpr int kFwd2Samples = 128; // samples per fwd2 block (the loss blocks)
constexpr int kFwd2Waves = 8;     // waves of a fwd2 workgroup (two per SIMD)
constexpr int kTile = 256;        // wgrad output tile edge
constexpr int kWgradStages = 5;   // ring depth of wgrad (5 x 32 KB)
constexpr int kWgradWaves = 8;    // waves of a wgrad workgroup (two per SIMD)
// entries of a loss block's sums: db2 [H], dw3 [H], db3, db1 [H]
__host__ __device__ constexpr int spart_w(int H) { return 3 * H + 1; }

IQLH_DEV f4 mma(bf16x8 a, bf16x8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }

// s_waitcnt on vmcnt only (expcnt and lgkmcnt fields at their maxima)
template <int N>
IQLH_DEV void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt on lgkmcnt only: this wave's LDS operations are complete
IQLH_DEV void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Workgroup barrier without a memory fence: the global->LDS copies of the
// stages in flight must stay in flight across it (a fenced barrier would wait
// for all of them).  The empty asm keeps the compiler from moving LDS
// accesses across it.
IQLH_DEV void bar() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

IQLH_DEV uint32_t cvt2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(bf2f32x2{lo, hi}, bf16x2v));
}
IQLH_DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
IQLH_DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// sum over the four 16-lane groups (lanes l, l^16, l^32, l^48); every lane gets it
IQLH_DEV float sum_groups(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// sum over the 16 lanes of a row (lanes 16g .. 16g + 15); every lane gets it
IQLH_DEV float sum_row16(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x128, 0xF, 0xF, false);  // row_ror:8
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x124, 0xF, 0xF, false);  // row_ror:4
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x122, 0xF, 0xF, false);  // row_ror:2
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x121, 0xF, 0xF, false);  // row_ror:1
    return x;
}

// Scheduling hint for one stage: the next stage's NR LDS fragment reads
// spread between this stage's NM MFMAs, so the reads complete under the
// matrix work (with one wave per SIMD nothing else would hide them).
template <int NR, int NM, int I = 0>
IQLH_DEV void reads_among_mfma() {
    if constexpr (I < NR) {
        __builtin_amdgcn_sched_group_barrier(0x008, NM * (I + 1) / NR - NM * I / NR, 0);  // MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                                   // one DS read
        reads_among_mfma<NR, NM, I + 1>();
    }
}

// vmcnt wait leaving min(K, ahead) stages of LPT copies in flight (K <= 3
// known at compile time; written as compares on ahead alone, which the
// compiler keeps scalar)
template <int K, int LPT>
IQLH_DEV void wait_ahead(int ahead) {
    static_assert(K >= 0 && K <= 3, "stages in flight");
    if (K >= 3 && ahead >= 3) wait_vm<(K >= 3 ? 3 : 0) * LPT>();
    else if (K >= 2 && ahead >= 2) wait_vm<(K >= 2 ? 2 : 0) * LPT>();
    else if (K >= 1 && ahead >= 1) wait_vm<(K >= 1 ? 1 : 0) * LPT>();
    else wait_vm<0>();
}

// ---------------------------------------------------------------- K-loop
// Stage s of nsl goes to ring buffer s % NST; NST - 1 stages are issued
// ahead.  LPT = copies each thread issues per stage.  The product supplies
// issue(slice, buf) (global -> LDS copies of a stage), mma(p) (the MFMAs of
// the stage held in fragment set p), load(buf, p) (LDS -> fragment set p),
// and pre(), run once after the first stages are issued (work whose memory
// latency then overlaps theirs).  p is 0 or 1 as a type
// (std::integral_constant), so the fragment sets stay in registers.
//
// Each step runs the MFMAs of stage s and reads the fragments of stage s + 1
// into the other set; the product's scheduling hint spreads the reads among
// the MFMAs.  A fragment used by one row of MFMAs only may be read into the
// same registers once that row is done (the reads follow the MFMAs in
// program order), so only the operand every row uses needs two sets.
//
// Buffer reuse: stage s + NST - 1 is issued into the buffer of stage s - 1
// after the barrier of step s; every wave reaches that barrier after its
// MFMAs of stage s - 1, i.e. after its reads of that buffer completed.
template <int V>
using Set = std::integral_constant<int, V>;
template <int NST, int LPT, class Issue, class Load, class Mma, class Pre>
IQLH_DEV void kloop(int nsl, Issue&& issue, Load&& load, Mma&& mma, Pre&& pre) {
    static_assert(NST >= 2 && NST <= 5, "ring depth");
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nsl) issue(s, s);
    pre();
    // stage 0 landed: stages 1 .. min(NST - 2, nsl - 1) may stay in flight
    wait_ahead<NST - 2, LPT>(nsl - 1);
    bar();
    load(0, Set<0>{});
    auto step = [&](int s, auto cur, auto nxt) __attribute__((always_inline)) {
        if (s + 1 < nsl) {
            // issued so far: stages 0 .. min(s + NST - 2, nsl - 1); stage s + 1
            // must have landed, stages s + 2 .. of those may stay in flight
            wait_ahead<NST - 3, LPT>(nsl - 2 - s);
            bar();
            if (s + NST - 1 < nsl) issue(s + NST - 1, (s + NST - 1) % NST);
        }
        mma(cur);
        // the last step re-reads its own (valid) stage: no branch around the
        // reads, so they stay in the MFMAs' basic block
        load((s + 1 < nsl ? s + 1 : s) % NST, nxt);
    };
    // pairs of steps, so that set 0 holds the current fragments at the top
    // of every iteration; an odd last step after the loop
    int s = 0;
    for (; s + 2 <= nsl; s += 2) {
        step(s, Set<0>{}, Set<1>{});
        step(s + 1, Set<1>{}, Set<0>{});
    }
    if (s < nsl) step(s, Set<0>{}, Set<1>{});
}
constexpr auto no_pre = [] {};

// The same ring with one fragment set: every step reads its own stage's
// fragments and then runs its MFMAs (for a product whose epilogue leaves no
// registers for a second set).
template <int NST, int LPT, class Issue, class Compute, class Pre>
IQLH_DEV void kloop1(int nsl, Issue&& issue, Compute&& compute, Pre&& pre) {
    static_assert(NST >= 2 && NST <= 5, "ring depth");
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nsl) issue(s, s);
    pre();
    for (int s = 0; s < nsl; ++s) {
        // issued so far: stages 0 .. min(s + NST - 2, nsl - 1); stage s must
        // have landed, stages s + 1 .. of those may stay in flight
        wait_ahead<NST - 2, LPT>(nsl - 1 - s);
        bar();
        if (s + NST - 1 < nsl) issue(s + NST - 1, (s + NST - 1) % NST);
        compute(s % NST);
    }
}

// Scheduling hint for kloop1: the NR fragment reads first, then the NM MFMAs
// (the compiler otherwise sinks each read to its first use).
template <int NR, int NM>
IQLH_DEV void reads_then_mfma() {
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);  // MFMA
}

// ----------------------------------------------- K-contiguous operand tiles
// Rows [0, R) of a row-major operand (k contiguous), k in [k0, k0 + 32):
// LDS chunk c (16 bytes) holds row c >> 2, k unit (c & 3) ^ ((row >> 1) & 3).
// Rows at or past rmax re-read row rmax - 1 (their products are discarded).
template <int R, int NT = kThreads>
IQLH_DEV void dma_kc(const uint16_t* g, int64_t ld, int rmax, int k0, uint16_t* lds) {
    static_assert((R * 4) % NT == 0, "chunks per thread");
    const int tid = threadIdx.x, wbase = tid & ~63;
#pragma unroll
    for (int i = 0; i < R * 4 / NT; ++i) {
        const int c = i * NT + tid;
        const int r = c >> 2, u = (c & 3) ^ ((r >> 1) & 3);
        const int gr = r < rmax ? r : rmax - 1;
        __builtin_amdgcn_global_load_lds((const void*)(g + (int64_t)gr * ld + k0 + 8 * u),
                                         IQLH_LDS(lds + (i * NT + wbase) * 8), 16, 0, 0);
    }
}
// this lane's element offset of its fragment in row tile 0 of a K-contiguous
// tile (row tile t adds 512 elements)
IQLH_DEV int kc_lane() {
    const int l = threadIdx.x & 63, l16 = l & 15, q = l >> 4;
    return l16 * kBK + 8 * (q ^ ((l16 >> 1) & 3));
}

// --------------------------------------------------- natural operand tiles
// A row of zeros in device memory: the copies of samples past the end of a
// chunk read it, so that those samples contribute nothing to the products.
__device__ __align__(16) const uint16_t kZeroRow[kTile] = {};

// Samples [0, 32) x features [f0, f0 + 256) of a row-major [sample][feature]
// activation: LDS chunk c holds sample c >> 5, feature unit (c & 31) ^ (2 (s & 3)).
// Samples at or past smax read zeros (ZERO) or re-read sample smax - 1 (their
// products are then discarded or multiplied by zeros); features at or past
// fmax re-read feature 0 of the row (those columns are discarded).
template <bool ZERO, int NT = kThreads>
IQLH_DEV void dma_nat(const uint16_t* g, int64_t ld, int smax, int f0, int fmax, uint16_t* lds) {
    const int tid = threadIdx.x, wbase = tid & ~63;
#pragma unroll
    for (int i = 0; i < 1024 / NT; ++i) {
        const int c = i * NT + tid;
        const int s = c >> 5, v = (c & 31) ^ (2 * (s & 3));
        const int gs = s < smax ? s : smax - 1;
        const int f = f0 + 8 * v;
        const int gf = f < fmax ? f : 0;
        const uint16_t* src = g + (int64_t)gs * ld + gf;
        if (ZERO) src = s < smax ? src : kZeroRow + 8 * v;
        __builtin_amdgcn_global_load_lds((const void*)src, IQLH_LDS(lds + (i * NT + wbase) * 8), 16, 0, 0);
    }
}
IQLH_DEV u32x2 ld_tr(const uint16_t* p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
    return __builtin_bit_cast(u32x2, r);
}
// Transpose-load addressing of a natural tile: the operand of feature tile c
// (features 16c .. 16c + 15) over the 32 samples is two loads at
// base[h][c & 3] + 16 (c & ~3); this lane addresses sample 8 (l >> 4) +
// ((l >> 2) & 3) + 4h, features 16c + 4 (l & 3).
struct NatBase {
    int b[2][4];
};
IQLH_DEV NatBase nat_base() {
    const int l = threadIdx.x & 63, g = l >> 4, e = (l >> 2) & 3, i = l & 3;
    NatBase nb;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            nb.b[h][c] = (8 * g + e + 4 * h) * kTile + 16 * (c ^ e) + 8 * (i >> 1) + 4 * (i & 1);
    return nb;
}
IQLH_DEV bf16x8 nat_frag(const uint16_t* tile, const NatBase& nb, int c) {
    const int off = 16 * (c & ~3);
    const u32x2 lo = ld_tr(tile + nb.b[0][c & 3] + off);
    const u32x2 hi = ld_tr(tile + nb.b[1][c & 3] + off);
    return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
}

// ---------------------------------------------------- staged epilogues
// A workgroup's bf16 results go to LDS as [sample][feature] rows of NF
// features, the 16-byte unit u of row s at u ^ (s & 7), and leave as 16-byte
// stores covering whole rows (coalesced), not as the 8-byte pieces of the
// MFMA layout.
template <int NF>
IQLH_DEV int stage_off(int s, int f) { return s * NF + ((((f >> 3) ^ (s & 7)) << 3) | (f & 7)); }

// threadIdx.x through an empty asm statement: address arithmetic on it
// cannot be hoisted above this point (so it is not held in registers across
// an earlier loop).
IQLH_DEV int opaque_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Rows [0, ns) of the staged tile to dst rows (row stride ld), columns
// [0, NF).
template <int NF, int NS, int NT = kThreads>
IQLH_DEV void stage_out(const uint16_t* lds, uint16_t* dst, int64_t ld, int ns, int tid = threadIdx.x) {
    constexpr int UPR = NF / 8;  // 16-byte units per row
#pragma unroll 4
    for (int c = tid; c < NS * UPR; c += NT) {
        const int r = c / UPR, u = c - r * UPR;
        if (r >= ns) break;
        *(u32x4*)(dst + (int64_t)r * ld + 8 * u) = *(const u32x4*)(lds + r * NF + ((u ^ (r & 7)) << 3));
    }
}

struct BigArgs {
    const uint16_t* x;      // [B][ldx] batch rows
    int64_t ldx;
    const uint16_t* w1s;    // [G][H][S_pad] W1 shadow
    int64_t ldw1;
    const uint16_t* w2s;    // [G][H][H] W2 shadow
    const uint16_t* w2ts;   // [G][H][H] W2^T shadow
    const float* params;    // [G][P]
    const float* q;         // [B]
    uint16_t* h1;           // [G][B][H]
    uint16_t* dz2;          // [G][B][H]
    uint16_t* dz1;          // [G][B][H]
    float* spart;           // [G][nblk][3H + 1]: db2, dw3, db3 and db1 of each 128-sample block
    float* loss_part;       // [G][nblk]
    float* out_v;           // [G][B] or null
    float* part;            // [G][nchunk][Pp]
    int64_t P, Pp;
    int64_t off_b1, off_w2, off_b2, off_w3, off_b3;
    float tau0, tau1, invB;
    int B, S, H, chunk, nchunk, nblk;
    int fwd_only;  // 1: V (and the bootstrap target) only
    ValueOut vo;
    // advantage-weighted policy run by the weight-gradient launch's spare
    // workgroups: grid columns pol_x0 .. pol_x0 + pol_nx - 1 of every group
    // row; pol_lpr = 0 when the launch does not run it
    const float4* pol_q;  // [B][A]
    float4* pol_pi;       // [G][B][A]
    float pol_beta;
    int pol_lpr, pol_x0, pol_nx;
};

// A spare workgroup of the weight-gradient launch: its share of the policy of
// every group from V, which fwd2 completed before this launch started.
IQLH_DEV void big_policy_block(const BigArgs& a) {
    constexpr int NT = 64 * kWgradWaves;
    const int64_t bid = (int64_t)blockIdx.y * a.pol_nx + ((int)blockIdx.x - a.pol_x0);
    const int64_t nb = (int64_t)gridDim.y * a.pol_nx;
    const int G = (int)gridDim.y;
    switch (a.pol_lpr) {
        case 1: aw_vec_rows<1, NT>(a.pol_q, a.out_v, G, a.B, a.pol_beta, a.pol_pi, bid, nb); break;
        case 2: aw_vec_rows<2, NT>(a.pol_q, a.out_v, G, a.B, a.pol_beta, a.pol_pi, bid, nb); break;
        case 4: aw_vec_rows<4, NT>(a.pol_q, a.out_v, G, a.B, a.pol_beta, a.pol_pi, bid, nb); break;
        case 8: aw_vec_rows<8, NT>(a.pol_q, a.out_v, G, a.B, a.pol_beta, a.pol_pi, bid, nb); break;
        default: aw_vec_rows<16, NT>(a.pol_q, a.out_v, G, a.B, a.pol_beta, a.pol_pi, bid, nb); break;
    }
}


// Workgroup id -> (tile, group): consecutive ids go to different XCDs, so the
// ids of one sample range are spread as id = xcd + 8 k; this picks the tiles
// of one sample range for the ids of one XCD.  nper = tiles per range.
IQLH_DEV void xcd_map(int id, int nranges, int nper, int& range, int& job) {
    const int full = (nranges / 8) * 8;  // ranges mapped XCD-locally
    if (id < full * nper) {
        const int xcd = id & 7, k = id >> 3;
        range = xcd + 8 * (k / nper);
        job = k % nper;
    } else {
        const int r = id - full * nper;
        range = full + r / nper;
        job = r % nper;
    }
}

// First k-slice of this workgroup's product, of nks: the workgroups of one
// XCD (ids xcd + 8 k) start at different slices, so that they do not all
// read the same weight rows from their shared L2 at the same time.  Each
// workgroup still adds every slice once, in a fixed order (deterministic).
IQLH_DEV int k_rotation(int nks) { return (int)((blockIdx.x >> 3) % (unsigned)nks); }

// ------------------------------------------------- dh1 inside fwd2's workgroup
// dh1[f][s] = sum_k W2^T[f][k] dz2[s][k] for the H features of this wave's
// rows ((H / NW) w + 16 i + .., NW waves) and the block's 128 samples, K = H.  The B
// operand is the dz2 tile staged in LDS ([sample][feature], 16-byte unit u of
// row s at u ^ (s & 7)); the A operand comes from the W2^T shadow in global
// memory (L2-resident after the first blocks), 16 bytes per lane, loaded one
// k-step ahead.  Then dz1 = dh1 relu'(z1) from the forward's mask bits, the block's
// db1 sums from dz1 as stored, and dz1 staged and stored as whole rows.
template <int H, int NW>
IQLH_DEV const uint16_t* w2t_lane(const BigArgs& a, int g, int wv, int l16, int q) {
    return a.w2ts + (int64_t)g * H * H + (int64_t)((H / NW) * wv + l16) * H + 8 * q;
}
// the first k-step's W2^T fragments (issued before the dz2 stores, so that
// waiting for them does not wait for the stores)
template <int H, int MT>
IQLH_DEV void w2t_frags(const uint16_t* At, int kt, bf16x8 (&f)[MT]) {
#pragma unroll
    for (int i = 0; i < MT; ++i) f[i] = *(const bf16x8*)(At + (int64_t)16 * i * H + kBK * kt);
}
// acc[i][j] = sum_k A[f_i][k] Bt[s_j][k] over k = 0 .. H - 1, in the k-step
// order rotated by krot: A row-major in global memory (At = this lane's row
// and k-offset, 16-byte fragments loaded one k-step ahead, the first step's
// in fa0 already), Bt the [sample][k] tile staged in LDS (stage_off<H>).
template <int H, int MT>
IQLH_DEV void lds_b_product(const uint16_t* At, const uint16_t* smem, f4 (&acc)[MT][8], bf16x8 (&fa0)[MT], int krot,
                            int l16, int q) {
    constexpr int NK = H / kBK;
    static_assert(NK % 2 == 0, "k-steps in pairs");
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    bf16x8 fa1[MT], fb[8];
    auto load_a = [&](int kt, bf16x8 (&f)[MT]) __attribute__((always_inline)) { w2t_frags<H, MT>(At, kt, f); };
    auto step = [&](int kt, bf16x8 (&cur)[MT], bf16x8 (&nxt)[MT]) __attribute__((always_inline)) {
        if (kt + 1 < NK) load_a((kt + 1 + krot) & (NK - 1), nxt);
        // the next step's loads stay ahead of this step's MFMAs (the
        // scheduler would otherwise sink each load to its first use)
        __builtin_amdgcn_sched_barrier(0);
        const int kk = (kt + krot) & (NK - 1);
#pragma unroll
        for (int j = 0; j < 8; ++j) fb[j] = *(const bf16x8*)(smem + stage_off<H>(16 * j + l16, kBK * kk + 8 * q));
#pragma unroll
        for (int i = 0; i < MT; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = mma(cur[i], fb[j], acc[i][j]);
    };
#pragma unroll
    for (int kt = 0; kt < NK; kt += 2) {
        step(kt, fa0, fa1);
        step(kt + 1, fa1, fa0);
    }
}

template <int H, int MT, int NW>
IQLH_DEV void backward_h1(const BigArgs& a, uint16_t* smem, f4 (&acc)[MT][8], bf16x8 (&fa0)[MT], int g, int blk,
                          int s0, int srows, int wv, int l, int l16, int q, int krot, const uint32_t* smask) {
    // (l16 and q are formed again from the thread index before the epilogue)
    static_assert(MT * 16 * NW == H, "row tiles");
    const uint16_t* At = w2t_lane<H, NW>(a, g, wv, l16, q);
    // this lane's relu'(z1) words, left in LDS by the forward product
    uint32_t mb[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) mb[i] = smask[i * (64 * NW) + (int)threadIdx.x];
    lds_b_product<H, MT>(At, smem, acc, fa0, krot, l16, q);
    __syncthreads();  // every wave is done with the dz2 tile
    // lane coordinates formed again here (opaque_tid): otherwise the compiler
    // keeps the epilogue's LDS and store addresses, equal to or derived from
    // the dz2 epilogue's, live across the loop above, and spills them
    const int tid2 = opaque_tid();
    l16 = tid2 & 15;
    q = (tid2 & 63) >> 4;
    float* db1 = a.spart + ((int64_t)g * a.nblk + blk) * spart_w(H) + 2 * H + 1;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int f = (H / NW) * wv + 16 * i + 4 * q;
        float cs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int sl = 16 * j + l16;
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = (mb[i] >> (4 * j + r)) & 1u ? acc[i][j][r] : 0.f;
            const u32x2 pk = u32x2{cvt2(y[0], y[1]), cvt2(y[2], y[3])};
            if (sl < srows) {
                cs[0] += bf_lo(pk.x);
                cs[1] += bf_hi(pk.x);
                cs[2] += bf_lo(pk.y);
                cs[3] += bf_hi(pk.y);
            }
            *(u32x2*)(smem + stage_off<H>(sl, f)) = pk;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) cs[r] = sum_row16(cs[r]);
        if (l16 == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) db1[f + r] = cs[r];
        }
    }
    __syncthreads();
    stage_out<H, kFwd2Samples, 64 * NW>(smem, a.dz1 + ((int64_t)g * a.B + s0) * H, H, srows, opaque_tid());
}

// v's partial dot products of the NW waves for sample sl, added pairwise in a
// fixed order
template <int NW>
IQLH_DEV float wave_parts_sum(const float* svp, int sl) {
    static_assert(NW == 4 || NW == 8, "waves");
    const float a = (svp[sl] + svp[kFwd2Samples + sl]) + (svp[2 * kFwd2Samples + sl] + svp[3 * kFwd2Samples + sl]);
    if constexpr (NW == 4) return a;
    const float b = (svp[4 * kFwd2Samples + sl] + svp[5 * kFwd2Samples + sl]) +
                    (svp[6 * kFwd2Samples + sl] + svp[7 * kFwd2Samples + sl]);
    return a + b;
}

// --------------------------------------------------------------- fwd2
// All H features of 128 samples: z1 = W1 s through the ring, h1 =
// relu(z1 + b1) to LDS, z2 = W2 h1 + b2 from it, and the loss epilogue.
// Wave w of NW owns features (H / NW) w .. + H / NW - 1 (MT row tiles of 16)
// of every layer, so the mask bits of relu'(z1) sit in the lanes that form
// dh1 for the same features and samples.
// With BWD, the same workgroup then forms dh1 = W2^T dz2 for its samples from
// the dz2 tile still staged in LDS, and dz1 = dh1 relu'(z1) with the block's
// db1 sums, so dz2 is never read back from memory for it.
template <int H, bool BWD, int NW>
__global__ __launch_bounds__(64 * NW) void big_fwd2_kernel(BigArgs a) {
    extern __shared__ __align__(16) uint16_t smem[];
    constexpr int NT = 64 * NW, MT = H / (16 * NW), NST = 3, STG = (H + kFwd2Samples) * kBK;
    constexpr int LPT = (H + kFwd2Samples) * 4 / NT;
    const int g = blockIdx.y, blk = blockIdx.x;
    const int B = a.B, s0 = blk * kFwd2Samples;
    // the ring's product: z1 = W1 s over the state's k-slices
    const uint16_t* A = a.w1s + (int64_t)g * H * a.ldw1;
    const int64_t lda = a.ldw1;
    const uint16_t* Bm = a.x + (int64_t)s0 * a.ldx;
    const int64_t ldb = a.ldx;
    const int nks = a.S / kBK;
    const int srows = B - s0;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lo = kc_lane();
    constexpr int RING = NST * STG, STAGE = kFwd2Samples * H;
    float* svp = (float*)(smem + (RING > STAGE ? RING : STAGE));  // [NW][128] V partials of each wave
    float* sq = svp + NW * kFwd2Samples;                            // [128] q of the block's samples
    float* sb2 = sq + kFwd2Samples;                                 // [H] b2
    float* sw3 = sb2 + H;                                           // [H] w3
    float* sb1 = sw3 + H;                                           // [H] b1
    uint32_t* smask = (uint32_t*)(sb1 + H);                         // [MT][NT] relu'(z1) words
    const float* prm = a.params + (int64_t)g * a.P;
    // q, b2 and w3 to LDS while the first stages are in flight, so that the
    // epilogue reads them without a memory round trip
    auto pre = [&] {
        const int t = threadIdx.x;
        if (t < kFwd2Samples) sq[t] = (!a.fwd_only && t < srows) ? a.q[s0 + t] : 0.f;
        for (int f = t; f < H; f += NT) {
            sb2[f] = prm[a.off_b2 + f];
            sw3[f] = prm[a.off_w3 + f];
            sb1[f] = prm[a.off_b1 + f];
        }
        wait_lgkm0();  // the stores are complete before the loop's first barrier
    };

    f4 acc[MT][8];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    const int krot = k_rotation(H / kBK), krot1 = k_rotation(nks);
    auto issue = [&](int s, int buf) {
        uint16_t* st_ = smem + buf * STG;
        const int k0 = ((s + krot1) % nks) * kBK;
        dma_kc<H, NT>(A, lda, H, k0, st_);
        dma_kc<kFwd2Samples, NT>(Bm, ldb, srows, k0, st_ + H * kBK);
    };
    if constexpr (H == 512) {
        // no registers for a second fragment set next to this epilogue
        kloop1<NST, LPT>(nks, issue, [&](int buf) {
            const uint16_t* ta = smem + buf * STG + ((H / NW) * wv) * kBK + lo;
            const uint16_t* tb = smem + buf * STG + H * kBK + lo;
            bf16x8 fa[MT], fb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) fb[j] = *(const bf16x8*)(tb + j * 16 * kBK);
#pragma unroll
            for (int i = 0; i < MT; ++i) fa[i] = *(const bf16x8*)(ta + i * 16 * kBK);
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = mma(fa[i], fb[j], acc[i][j]);
            reads_then_mfma<8 + MT, 8 * MT>();
        }, pre);
    } else {
        bf16x8 fa[MT], fb[2][8];  // fa: one set, re-read row by row (see kloop)
        kloop<NST, LPT>(
            nks, issue,
            [&](int buf, auto p) {
                constexpr int P = decltype(p)::value;
                const uint16_t* ta = smem + buf * STG + ((H / NW) * wv) * kBK + lo;
                const uint16_t* tb = smem + buf * STG + H * kBK + lo;
#pragma unroll
                for (int j = 0; j < 8; ++j) fb[P][j] = *(const bf16x8*)(tb + j * 16 * kBK);
#pragma unroll
                for (int i = 0; i < MT; ++i) fa[i] = *(const bf16x8*)(ta + i * 16 * kBK);
            },
            [&](auto p) {
                constexpr int P = decltype(p)::value;
#pragma unroll
                for (int i = 0; i < MT; ++i)
#pragma unroll
                    for (int j = 0; j < 8; ++j) acc[i][j] = mma(fa[i], fb[P][j], acc[i][j]);
                reads_among_mfma<8 + MT, 8 * MT>();
            },
            pre);
    }

    {
        // lane coordinates formed afresh in each phase (opaque_tid), so that
        // no phase's addresses are held across another phase's loop
        const int ta1 = opaque_tid(), l16a = ta1 & 15, fb0a = (H / NW) * wv + 4 * ((ta1 & 63) >> 4);
        // h1 = relu(z1 + b1) to the LDS tile ([sample][feature], the layout
        // the dz2 tile takes below) and relu'(z1) as bits, bit 4 j + r of
        // word i for this lane's feature 16 i + r and sample 16 j + l16 --
        // the accumulator layout the dh1 product ends with
        __syncthreads();  // every wave is done with the ring
#pragma unroll
        for (int i = 0; i < MT; ++i) {
            uint32_t bits = 0u;
            float b1[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) b1[r] = sb1[fb0a + 16 * i + r];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float y[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // relu as an integer max on the bit pattern (negative
                    // values and -0 become +0), the bit from the result
                    const int zb = max(__float_as_int(acc[i][j][r] + b1[r]), 0);
                    y[r] = __int_as_float(zb);
                    bits |= min((uint32_t)zb, 1u) << (4 * j + r);
                }
                *(u32x2*)(smem + stage_off<H>(16 * j + l16a, fb0a + 16 * i)) = u32x2{cvt2(y[0], y[1]), cvt2(y[2], y[3])};
            }
            smask[i * NT + ta1] = bits;
        }
        // z2 = W2 h1 from the tile: W2's rows from global memory, h1 from
        // LDS; h1 leaves for the weight gradients after the product, so that
        // no wait for W2's fragments inside it waits for those stores too
        const int ta2 = opaque_tid(), l16b = ta2 & 15, qb = (ta2 & 63) >> 4;
        const uint16_t* A2 = a.w2s + (int64_t)g * H * H + (int64_t)((H / NW) * wv + l16b) * H + 8 * qb;
        bf16x8 fz[MT];
        w2t_frags<H, MT>(A2, krot, fz);
        __syncthreads();
        lds_b_product<H, MT>(A2, smem, acc, fz, krot, l16b, qb);
        if (!a.fwd_only) stage_out<H, kFwd2Samples, NT>(smem, a.h1 + ((int64_t)g * B + s0) * H, H, srows, opaque_tid());
    }
    const int l = opaque_tid() & 63, l16 = l & 15, q = l >> 4;
    const int fb0 = (H / NW) * wv + 4 * q;
    // z2 = acc + b2 (formed again in each pass below, so the accumulators
    // are only read); this wave's part of v for each of its 8 samples
    float vp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vp[j] = 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int f = fb0 + 16 * i + r;
            const float b2 = sb2[f], w3 = sw3[f];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float z = acc[i][j][r] + b2;
                vp[j] = fmaf(w3, z > 0.f ? z : 0.f, vp[j]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float t = sum_groups(vp[j]);
        if (q == 0) svp[wv * kFwd2Samples + 16 * j + l16] = t;
    }
    __syncthreads();
    const float b3 = prm[a.off_b3];
    if (a.fwd_only) {
        if (wv == 0 && q == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int sl = 16 * j + l16, s = s0 + sl;
                const float v = wave_parts_sum<NW>(svp, sl) + b3;
                if (s < B) write_value(a.vo, g, B, s, v);
            }
        }
        return;
    }
    const float tau = g == 0 ? a.tau0 : a.tau1;
    float dv[8], lsum = 0.f, dsum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int sl = 16 * j + l16, s = s0 + sl;
        const float v = wave_parts_sum<NW>(svp, sl) + b3;
        dv[j] = 0.f;
        if (s < B) {
            const float diff = sq[sl] - v;
            const float w = diff >= 0.f ? tau : 1.f - tau;
            dv[j] = -2.f * w * diff * a.invB;
            lsum += w * diff * diff;
            dsum += dv[j];
            if (wv == 0 && q == 0 && a.out_v) a.out_v[(int64_t)g * B + s] = v;
        }
    }
    float* sp = a.spart + ((int64_t)g * a.nblk + blk) * spart_w(H);
    if (wv == 0) {
        lsum = sum_row16(lsum);
        dsum = sum_row16(dsum);
        if (l == 0) {
            a.loss_part[(int64_t)g * a.nblk + blk] = lsum;
            sp[2 * H] = dsum;
        }
    }
    // dz2 = dv w3 relu'(z2) -> DZ2; block sums of dz2 and dv relu(z2)
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        float db2[4] = {0.f, 0.f, 0.f, 0.f}, dw3[4] = {0.f, 0.f, 0.f, 0.f}, b2[4], w3[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            b2[r] = sb2[fb0 + 16 * i + r];
            w3[r] = sw3[fb0 + 16 * i + r];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float d[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float z = acc[i][j][r] + b2[r];
                d[r] = z > 0.f ? dv[j] * w3[r] : 0.f;
                dw3[r] = fmaf(dv[j], z > 0.f ? z : 0.f, dw3[r]);
            }
            // db2 sums dz2 as stored (bf16), as the products that read it do
            const u32x2 pk = u32x2{cvt2(d[0], d[1]), cvt2(d[2], d[3])};
            db2[0] += bf_lo(pk.x);
            db2[1] += bf_hi(pk.x);
            db2[2] += bf_lo(pk.y);
            db2[3] += bf_hi(pk.y);
            *(u32x2*)(smem + stage_off<H>(16 * j + l16, fb0 + 16 * i)) = pk;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            db2[r] = sum_row16(db2[r]);
            dw3[r] = sum_row16(dw3[r]);
        }
        if (l16 == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                sp[fb0 + 16 * i + r] = db2[r];
                sp[H + fb0 + 16 * i + r] = dw3[r];
            }
        }
    }
    bf16x8 fa0[MT];
    if constexpr (BWD) w2t_frags<H, MT>(w2t_lane<H, NW>(a, g, wv, l16, q), krot, fa0);
    __syncthreads();
    stage_out<H, kFwd2Samples, NT>(smem, a.dz2 + ((int64_t)g * B + s0) * H, H, srows);
    if constexpr (BWD) backward_h1<H, MT, NW>(a, smem, acc, fa0, g, blk, s0, srows, wv, l, l16, q, krot, smask);
}

// --------------------------------------------------------------- wgrad
// Per (chunk, job): job < n2 -> a 256 x 256 tile of dW2 = dz2^T h1; else a
// tile of dW1 = dz1^T s.  Job j of a chunk also adds the chunk's block sums
// (db2, dw3, db3, db1, all from fwd2) for its share of the entries, so that
// no workgroup exists for that small sum alone.
__global__ __launch_bounds__(64 * kWgradWaves) void big_wgrad_kernel(BigArgs a) {
    extern __shared__ __align__(16) uint16_t smem[];
    // wave w: rows 128 (w & 1) .. + 127 and columns (256 / NC) (w >> 1) .. of
    // the 256 x 256 tile, NC = waves / 2 column groups of JT feature tiles
    constexpr int NT = 64 * kWgradWaves, NC = kWgradWaves / 2, JT = 16 / NC;
    constexpr int NST = kWgradStages, STG = 2 * kBK * kTile;
    if (a.pol_lpr && (int)blockIdx.x >= a.pol_x0) {  // uniform per workgroup, before any barrier
        big_policy_block(a);
        return;
    }
    const int g = blockIdx.y;
    const int H = a.H, S = a.S, B = a.B;
    const int nth = H / kTile, nts = (S + kTile - 1) / kTile;
    const int n2 = nth * nth, n1 = nth * nts, njob = n2 + n1;
    int c, job;
    xcd_map(blockIdx.x, a.nchunk, njob, c, job);
    const int b0 = c * a.chunk;
    const int len = min(a.chunk, B - b0);
    float* part = a.part + ((int64_t)g * a.nchunk + c) * a.Pp;
    const int tid = threadIdx.x;

    const uint16_t* A;
    const uint16_t* Bm;
    int64_t ldb;
    int fa0, fb0, fbmax, ldo;
    float* dst;
    if (job < n2) {
        const int mt = job / nth, nt = job % nth;
        A = a.dz2 + ((int64_t)g * B + b0) * H;
        Bm = a.h1 + ((int64_t)g * B + b0) * H;
        ldb = H; fa0 = kTile * mt; fb0 = kTile * nt; fbmax = H;
        dst = part + a.off_w2; ldo = H;
    } else {
        const int jj = job - n2, mt = jj / nts, nt = jj % nts;
        A = a.dz1 + ((int64_t)g * B + b0) * H;
        Bm = a.x + (int64_t)b0 * a.ldx;
        ldb = a.ldx; fa0 = kTile * mt; fb0 = kTile * nt; fbmax = S;
        dst = part; ldo = S;  // dW1 sits at offset 0
    }
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv & 1, wn = wv >> 1;
    const NatBase nb = nat_base();

    f4 acc[8][JT];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < JT; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    const int nsl = (len + kBK - 1) / kBK;

    // this job's share of the chunk's block sums, in block order, while the
    // first stages are in flight
    auto pre = [&] {
        const int ne = spart_w(H), per = (ne + njob - 1) / njob;
        const int k0 = b0 / kFwd2Samples, k1 = (b0 + len + kFwd2Samples - 1) / kFwd2Samples;
        const float* sp = a.spart + (int64_t)g * a.nblk * ne;
        for (int t = tid; t < per; t += NT) {
            const int e = job * per + t;
            if (e >= ne) break;
            float s = 0.f;
#pragma unroll 8
            for (int k = k0; k < k1; ++k) s += sp[(int64_t)k * ne + e];
            const int64_t off = e < H ? a.off_b2 + e
                                      : (e < 2 * H ? a.off_w3 + (e - H) : (e == 2 * H ? a.off_b3 : a.off_b1 + (e - 2 * H - 1)));
            part[off] = s;
        }
    };
    bf16x8 fa[8], fb[2][JT];  // fa: one set, re-read row by row (see kloop)
    kloop<NST, 2 * 1024 / NT>(
        nsl,
        [&](int s, int buf) {
            uint16_t* st_ = smem + buf * STG;
            const int sm = len - s * kBK;
            dma_nat<true, NT>(A + (int64_t)s * kBK * H, H, sm, fa0, H, st_);
            dma_nat<false, NT>(Bm + (int64_t)s * kBK * ldb, ldb, sm, fb0, fbmax, st_ + kBK * kTile);
        },
        [&](int buf, auto p) {
            constexpr int P = decltype(p)::value;
            const uint16_t* ta = smem + buf * STG;
            const uint16_t* tb = ta + kBK * kTile;
#pragma unroll
            for (int j = 0; j < JT; ++j) fb[P][j] = nat_frag(tb, nb, JT * wn + j);
#pragma unroll
            for (int i = 0; i < 8; ++i) fa[i] = nat_frag(ta, nb, 8 * wm + i);
        },
        [&](auto p) {
            constexpr int P = decltype(p)::value;
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < JT; ++j) acc[i][j] = mma(fa[i], fb[P][j], acc[i][j]);
            reads_among_mfma<2 * (8 + JT), 8 * JT>();
        },
        pre);

    const int l = tid & 63, l16 = l & 15, q = l >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int m = fa0 + 128 * wm + 16 * i + 4 * q;
#pragma unroll
        for (int j = 0; j < JT; ++j) {
            const int n = fb0 + 16 * (JT * wn + j) + l16;
            if (n < fbmax) {
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(int64_t)(m + r) * ldo + n] = acc[i][j][r];
            }
        }
    }

}

constexpr size_t ring_lds_bytes(int nst) { return (size_t)nst * 2 * kTile * kBK * 2; }
template <int H>
constexpr size_t fwd2_lds_bytes() {
    return (size_t)(3 * (H + kFwd2Samples) * kBK > kFwd2Samples * H ? 3 * (H + kFwd2Samples) * kBK : kFwd2Samples * H) * 2 +
           ((kFwd2Waves + 1) * kFwd2Samples + 3 * H + (H / (16 * kFwd2Waves)) * 64 * kFwd2Waves) * sizeof(float);
}

template <typename K>
hipError_t allow_lds(K kern, size_t bytes) {
    return hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

bool iql_big_supported(int dtype, int S, int H) {
    return dtype == 1 && (H == 256 || H == 512) && S >= kBK && S % kBK == 0 && S <= 4096;
}
int iql_big_blocks(int B) { return (B + kFwd2Samples - 1) / kFwd2Samples; }
int iql_big_spart_width(int H) { return spart_w(H); }
static int big_tiles(int S, int H) {
    const int nth = H / kTile, nts = (S + kTile - 1) / kTile;
    return nth * nth + nth * nts;
}
// chunks of one trainer: at most one weight-gradient tile per CU over all
// trainers (256 CUs), so the launch runs as one round
int iql_big_max_chunks(int S, int H) { return 256 / big_tiles(S, H) > 1 ? 256 / big_tiles(S, H) : 1; }
// samples per weight-gradient chunk for a batch of B rows and G trainers: a
// multiple of the fwd2 block, so every block's sums belong to exactly one chunk
int iql_big_chunk(int S, int H, int G, int B) {
    const int per = 256 / (big_tiles(S, H) * G);
    const int target = per > 1 ? per : 1;
    int c = (B + target - 1) / target;
    c = (c + kFwd2Samples - 1) / kFwd2Samples * kFwd2Samples;
    return c < kFwd2Samples ? kFwd2Samples : c;
}

struct BigPolicy {
    const float* q_all;
    int A;
    float beta;
    float* out_pi;
};

static hipError_t big_launch(const IqlDims& d, const IqlBuffers& b, const float* tau, const void* states, int64_t ld,
                             const float* q, int B, float* out_v, const ValueOut* vo, const BigPolicy* pol,
                             hipStream_t stream);

// Grid columns of the weight-gradient launch that run the policy: the compute
// units its tiles leave idle (256 - tiles x groups; one workgroup per CU), per
// group row, in whole multiples of 8 so that the tiles keep their XCD
// placement, and at least 8; 0 when the policy cannot run there (no streaming
// form for A, unaligned rows, too few idle CUs).
static int big_policy_cols(const IqlDims& d, int B, int A, const void* q_all, const void* out_pi) {
    if (!d.big || B <= 0 || aw_vec_lanes(A) == 0 || (((uintptr_t)q_all | (uintptr_t)out_pi) & 15u)) return 0;
    const int chunk = iql_big_chunk(d.S, d.H, d.G, B);
    const int tiles = ((B + chunk - 1) / chunk) * big_tiles(d.S, d.H);
    const int idle = 256 - tiles * d.G;
    const int px = idle > 0 ? idle / d.G / 8 * 8 : 0;
    return px >= 8 ? px : 0;
}

bool iql_big_policy_ok(const IqlDims& d, int B, int A, const void* q_all, const void* out_pi) {
    return q_all && out_pi && big_policy_cols(d, B, A, q_all, out_pi) > 0;
}

hipError_t launch_iql_big_fwd_bwd(const IqlDims& d, const IqlBuffers& b, const float* tau, const void* states,
                                  int64_t ld, const float* q, int B, float* out_v, hipStream_t stream,
                                  const float* q_all, int A, float beta, float* out_pi) {
    if (!out_pi) return big_launch(d, b, tau, states, ld, q, B, out_v, nullptr, nullptr, stream);
    if (!out_v || !iql_big_policy_ok(d, B, A, q_all, out_pi)) return hipErrorInvalidValue;
    const BigPolicy pol{q_all, A, beta, out_pi};
    return big_launch(d, b, tau, states, ld, q, B, out_v, nullptr, &pol, stream);
}

hipError_t launch_iql_big_forward(const IqlDims& d, const IqlBuffers& b, const void* states, int64_t ld, int B,
                                  const ValueOut& vo, hipStream_t stream) {
    const float tau[2] = {0.f, 0.f};
    return big_launch(d, b, tau, states, ld, nullptr, B, nullptr, &vo, nullptr, stream);
}

static hipError_t big_launch(const IqlDims& d, const IqlBuffers& b, const float* tau, const void* states, int64_t ld,
                             const float* q, int B, float* out_v, const ValueOut* vo, const BigPolicy* pol,
                             hipStream_t stream) {
    const int G = d.G, S = d.S, H = d.H;
    BigArgs a{};
    a.x = (const uint16_t*)states; a.ldx = ld;
    a.w1s = (const uint16_t*)b.w1s; a.ldw1 = d.S_pad;
    a.w2s = (const uint16_t*)b.w2s; a.w2ts = (const uint16_t*)b.w2ts;
    a.params = b.params; a.q = q;
    a.h1 = (uint16_t*)b.act_h1; a.dz2 = (uint16_t*)b.act_dz2; a.dz1 = (uint16_t*)b.act_dz1;
    a.spart = b.big_spart; a.loss_part = b.loss_part; a.out_v = out_v; a.part = b.part;
    a.P = d.P; a.Pp = d.Pp;
    a.off_b1 = (int64_t)H * S; a.off_w2 = a.off_b1 + H; a.off_b2 = a.off_w2 + (int64_t)H * H;
    a.off_w3 = a.off_b2 + H; a.off_b3 = a.off_w3 + H;
    a.tau0 = tau[0]; a.tau1 = tau[G > 1 ? 1 : 0]; a.invB = 1.f / (float)B;
    a.B = B; a.S = S; a.H = H;
    a.chunk = iql_big_chunk(S, H, G, B);
    a.nchunk = (B + a.chunk - 1) / a.chunk;
    a.nblk = iql_big_blocks(B);
    if (vo) {
        a.fwd_only = 1;
        a.vo = *vo;
    }

    static bool attr = false;
    if (!attr) {
        hipError_t e = allow_lds(big_wgrad_kernel, ring_lds_bytes(kWgradStages));
        if (e == hipSuccess) e = allow_lds(big_fwd2_kernel<256, false, kFwd2Waves>, fwd2_lds_bytes<256>());
        if (e == hipSuccess) e = allow_lds(big_fwd2_kernel<512, false, kFwd2Waves>, fwd2_lds_bytes<512>());
        if (e == hipSuccess) e = allow_lds(big_fwd2_kernel<256, true, kFwd2Waves>, fwd2_lds_bytes<256>());
        if (e == hipSuccess) e = allow_lds(big_fwd2_kernel<512, true, kFwd2Waves>, fwd2_lds_bytes<512>());
        if (e != hipSuccess) return e;
        attr = true;
    }
    const dim3 g2(a.nblk, G), t2(64 * kFwd2Waves);
    if (vo) {
        if (H == 512)
            hipLaunchKernelGGL((big_fwd2_kernel<512, false, kFwd2Waves>), g2, t2, fwd2_lds_bytes<512>(), stream, a);
        else
            hipLaunchKernelGGL((big_fwd2_kernel<256, false, kFwd2Waves>), g2, t2, fwd2_lds_bytes<256>(), stream, a);
        return hipGetLastError();
    }
    if (H == 512)
        hipLaunchKernelGGL((big_fwd2_kernel<512, true, kFwd2Waves>), g2, t2, fwd2_lds_bytes<512>(), stream, a);
    else
        hipLaunchKernelGGL((big_fwd2_kernel<256, true, kFwd2Waves>), g2, t2, fwd2_lds_bytes<256>(), stream, a);
    const int xw = a.nchunk * big_tiles(S, H);
    int px = 0;
    if (pol) {
        px = big_policy_cols(d, B, pol->A, pol->q_all, pol->out_pi);
        if (px <= 0) return hipErrorInvalidValue;
        a.pol_q = (const float4*)pol->q_all;
        a.pol_pi = (float4*)pol->out_pi;
        a.pol_beta = pol->beta;
        a.pol_lpr = aw_vec_lanes(pol->A);
        a.pol_x0 = xw;
        a.pol_nx = px;
    }
    const dim3 gw(xw + px, G);
    hipLaunchKernelGGL(big_wgrad_kernel, gw, dim3(64 * kWgradWaves), ring_lds_bytes(kWgradStages), stream, a);
    return hipGetLastError();
}

}  // namespace iqlh
