// IQL value-network forward/backward for wide hidden layers (bf16 operands,
// hidden 256 or 512, state_dim a multiple of 32), e.g. batch 65536, state 256,
// hidden 512.  Same arithmetic as the fused kernel ("GPU IQL + HER Porting
// Plan", section "Current State / IQL (CPU)"; the backward products of "Phase
// 2: Multi-Stream Graph Parallelism", section "2C. Grouped GEMM for IQL"):
//
//   fwd1   h1 = relu(W1 s + b1)                         -> H1  [B][H] bf16
//   fwd2   z2 = W2 h1 + b2 over all H features of a 128-sample block, then in
//          the epilogue v = w3 . relu(z2) + b3, the expectile loss, dv,
//          dz2 = dv w3 relu'(z2) -> DZ2 [B][H] bf16, and the block's sums of
//          dz2 (db2), dv relu(z2) (dw3) and dv (db3)
//   bwd1   dz1 = (W2^T dz2) * relu'(z1)                  -> DZ1 [B][H] bf16
//   wgrad  dW2 = dz2^T h1, dW1 = dz1^T s (with db1 = column sums of dz1)
//          over chunks of samples, one fp32 partial row per chunk; a small job
//          per chunk adds the fwd2 block sums of the chunk into the same row
//
// then the fixed-order partial reduction and Adam shared with the other
// paths (no float atomics anywhere).
//
// MI355X design.  Every product runs on v_mfma_f32_16x16x32_bf16 with a
// 128 x 128 output tile per wave (8 x 8 MFMA tiles, 256 accumulators), four
// waves per workgroup.  Operands stream HBM -> LDS with global_load_lds_dwordx4
// (no register staging) through a ring of 3-4 stages of 32 k each, so two or
// three stages are in flight while one is consumed; each stage ends in one
// s_barrier after the wave's own vmcnt wait.  Activations are row-major
// [sample][feature]:
//   * in the forward products k is the feature (contiguous): LDS rows of 32 k
//     (64 bytes), the 16-byte unit u of row r stored at u ^ ((r >> 1) & 3),
//     read with ds_read_b128 (conflict-free);
//   * in the weight gradients k is the sample: LDS keeps the natural
//     [sample][feature] rows (512 bytes), unit v of sample s stored at
//     v ^ (2 (s & 3)), and the MFMA operands are read with the LDS transpose
//     load ds_read_b64_tr_b16 (conflict-free), so no transposed copy of an
//     activation is ever written.
// The product orientation is D[feature][sample], so a lane ends with four
// consecutive features of one sample: bias, ReLU masks and the bf16 stores
// work on 8-byte runs of a row.
#include "common.hpp"
#include "launch.hpp"

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
constexpr int kTile = 256;        // fwd1 / bwd1 / wgrad output tile edge

IQLH_DEV f4 mma(bf16x8 a, bf16x8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0); }

// s_waitcnt on vmcnt only (expcnt and lgkmcnt fields at their maxima)
template <int N>
IQLH_DEV void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
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

// Scheduling hint for one stage: the NR LDS reads of the fragments first, then
// the NM MFMAs (the compiler otherwise sinks each read to its first use, and
// with one wave per SIMD every such read waits out the LDS latency).
template <int NR, int NM>
IQLH_DEV void reads_then_mfma() {
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // DS reads
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);  // MFMA
}

// ---------------------------------------------------------------- K-loop
// Stage s of nsl goes to ring buffer s % NST; NST - 1 stages are issued
// ahead.  LPT = copies each thread issues per stage.  issue(slice, buf) and
// compute(slice, buf) are the product's own.
template <int NST, int LPT, class Issue, class Compute>
IQLH_DEV void kloop(int nsl, Issue&& issue, Compute&& compute) {
    static_assert(NST >= 2 && NST <= 4, "ring depth");
#pragma unroll
    for (int s = 0; s < NST - 1; ++s)
        if (s < nsl) issue(s, s);
    for (int s = 0; s < nsl; ++s) {
        // slices after s already issued: min(NST - 2, nsl - 1 - s)
        const int ahead = nsl - 1 - s;
        if (NST >= 4 && ahead >= 2) wait_vm<(NST >= 4 ? 2 : 0) * LPT>();
        else if (NST >= 3 && ahead >= 1) wait_vm<LPT>();
        else wait_vm<0>();
        bar();
        if (s + NST - 1 < nsl) issue(s + NST - 1, (s + NST - 1) % NST);
        compute(s, s % NST);
    }
}

// ----------------------------------------------- K-contiguous operand tiles
// Rows [0, R) of a row-major operand (k contiguous), k in [k0, k0 + 32):
// LDS chunk c (16 bytes) holds row c >> 2, k unit (c & 3) ^ ((row >> 1) & 3).
// Rows at or past rmax re-read row rmax - 1 (their products are discarded).
template <int R>
IQLH_DEV void dma_kc(const uint16_t* g, int64_t ld, int rmax, int k0, uint16_t* lds) {
    static_assert((R * 4) % kThreads == 0, "chunks per thread");
    const int tid = threadIdx.x, wbase = tid & ~63;
#pragma unroll
    for (int i = 0; i < R * 4 / kThreads; ++i) {
        const int c = i * kThreads + tid;
        const int r = c >> 2, u = (c & 3) ^ ((r >> 1) & 3);
        const int gr = r < rmax ? r : rmax - 1;
        __builtin_amdgcn_global_load_lds((const void*)(g + (int64_t)gr * ld + k0 + 8 * u),
                                         IQLH_LDS(lds + (i * kThreads + wbase) * 8), 16, 0, 0);
    }
}
// this lane's element offset of its fragment in row tile 0 of a K-contiguous
// tile (row tile t adds 512 elements)
IQLH_DEV int kc_lane() {
    const int l = threadIdx.x & 63, l16 = l & 15, q = l >> 4;
    return l16 * kBK + 8 * (q ^ ((l16 >> 1) & 3));
}

// --------------------------------------------------- natural operand tiles
// Samples [0, 32) x features [f0, f0 + 256) of a row-major [sample][feature]
// activation: LDS chunk c holds sample c >> 5, feature unit (c & 31) ^ (2 (s & 3)).
// Samples at or past smax re-read sample smax - 1, features at or past fmax
// re-read feature 0 of the row (a ragged sample slice is zeroed afterwards;
// columns past fmax are discarded).
IQLH_DEV void dma_nat(const uint16_t* g, int64_t ld, int smax, int f0, int fmax, uint16_t* lds) {
    const int tid = threadIdx.x, wbase = tid & ~63;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = i * kThreads + tid;
        const int s = c >> 5, v = (c & 31) ^ (2 * (s & 3));
        const int gs = s < smax ? s : smax - 1;
        const int f = f0 + 8 * v;
        const int gf = f < fmax ? f : 0;
        __builtin_amdgcn_global_load_lds((const void*)(g + (int64_t)gs * ld + gf), IQLH_LDS(lds + (i * kThreads + wbase) * 8),
                                         16, 0, 0);
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

// Rows [0, ns) of the staged tile to dst rows (row stride ld), columns
// [0, NF).  With mask, an element is zeroed where the same element of mask
// is zero (dz1 = dh1 relu'(z1), read from h1 = relu(z1) as stored).
template <int NF, int NS>
IQLH_DEV void stage_out(const uint16_t* lds, uint16_t* dst, int64_t ld, int ns, const uint16_t* mask) {
    constexpr int UPR = NF / 8;  // 16-byte units per row
#pragma unroll 4
    for (int c = threadIdx.x; c < NS * UPR; c += kThreads) {
        const int r = c / UPR, u = c - r * UPR;
        if (r >= ns) break;
        u32x4 v = *(const u32x4*)(lds + r * NF + ((u ^ (r & 7)) << 3));
        if (mask) {
            const u32x4 h = *(const u32x4*)(mask + (int64_t)r * ld + 8 * u);
            v.x &= (h.x & 0xFFFFu ? 0xFFFFu : 0u) | (h.x >> 16 ? 0xFFFF0000u : 0u);
            v.y &= (h.y & 0xFFFFu ? 0xFFFFu : 0u) | (h.y >> 16 ? 0xFFFF0000u : 0u);
            v.z &= (h.z & 0xFFFFu ? 0xFFFFu : 0u) | (h.z >> 16 ? 0xFFFF0000u : 0u);
            v.w &= (h.w & 0xFFFFu ? 0xFFFFu : 0u) | (h.w >> 16 ? 0xFFFF0000u : 0u);
        }
        *(u32x4*)(dst + (int64_t)r * ld + 8 * u) = v;
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
    float* spart;           // [G][nblk][2H + 1]: db2, dw3, db3 of each 128-sample block
    float* loss_part;       // [G][nblk]
    float* out_v;           // [G][B] or null
    float* part;            // [G][nchunk][Pp]
    int64_t P, Pp;
    int64_t off_b1, off_w2, off_b2, off_w3, off_b3;
    float tau0, tau1, invB;
    int B, S, H, chunk, nchunk, nblk;
    int fwd_only;  // 1: V (and the bootstrap target) only
    ValueOut vo;
};

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

// ---------------------------------------------------- fwd1 / bwd1 products
// D[f][s] = sum_k A[f][k] Bm[s][k] over a 256-feature x 256-sample tile.
// MODE 0 (fwd1): A = W1 rows, Bm = batch rows, H1 = relu(D + b1).
// MODE 1 (bwd1): A = W2^T rows, Bm = dz2 rows, DZ1 = D * (H1 > 0).
template <int MODE>
__global__ __launch_bounds__(kThreads) void big_tile_kernel(BigArgs a) {
    extern __shared__ __align__(16) uint16_t smem[];
    constexpr int NST = 4, STG = 2 * kTile * kBK;  // elements per stage
    const int g = blockIdx.y;
    const int H = a.H, B = a.B;
    const int nft = H / kTile, nst = (B + kTile - 1) / kTile;
    int st, ft;
    xcd_map(blockIdx.x, nst, nft, st, ft);
    const int f0 = ft * kTile, s0 = st * kTile;
    const uint16_t* A;
    int64_t lda;
    const uint16_t* Bm;
    int64_t ldb;
    int K;
    if (MODE == 0) {
        A = a.w1s + (int64_t)g * H * a.ldw1 + (int64_t)f0 * a.ldw1; lda = a.ldw1;
        Bm = a.x + (int64_t)s0 * a.ldx; ldb = a.ldx; K = a.S;
    } else {
        A = a.w2ts + (int64_t)g * H * H + (int64_t)f0 * H; lda = H;
        Bm = a.dz2 + ((int64_t)g * B + s0) * H; ldb = H; K = H;
    }
    const int srows = B - s0;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wv & 1, wn = wv >> 1;
    const int lo = kc_lane();

    f4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    kloop<NST, 8>(
        K / kBK,
        [&](int s, int buf) {
            uint16_t* st_ = smem + buf * STG;
            dma_kc<kTile>(A, lda, kTile, s * kBK, st_);
            dma_kc<kTile>(Bm, ldb, srows, s * kBK, st_ + kTile * kBK);
        },
        [&](int, int buf) {
            const uint16_t* ta = smem + buf * STG + (128 * wm) * kBK + lo;
            const uint16_t* tb = smem + buf * STG + kTile * kBK + (128 * wn) * kBK + lo;
            bf16x8 fa[8], fb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) fb[j] = *(const bf16x8*)(tb + j * 16 * kBK);
#pragma unroll
            for (int i = 0; i < 8; ++i) fa[i] = *(const bf16x8*)(ta + i * 16 * kBK);
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = mma(fa[i], fb[j], acc[i][j]);
            reads_then_mfma<16, 64>();
        });

    // epilogue: lane holds features 128 wm + 16 i + 4 q + r of samples
    // 128 wn + 16 j + l16 (tile-local); staged as [sample][feature] rows
    const int l = threadIdx.x & 63, l16 = l & 15, q = l >> 4;
    const float* bias = a.params + (int64_t)g * a.P + a.off_b1 + f0;
    __syncthreads();  // every wave is done with the last stage
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int f = 128 * wm + 16 * i + 4 * q;
        float bb[4] = {0.f, 0.f, 0.f, 0.f};
        if (MODE == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) bb[r] = bias[f + r];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int sl = 128 * wn + 16 * j + l16;
            float y[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float z = acc[i][j][r] + bb[r];
                y[r] = MODE == 0 ? (z > 0.f ? z : 0.f) : z;
            }
            *(u32x2*)(smem + stage_off<kTile>(sl, f)) = u32x2{cvt2(y[0], y[1]), cvt2(y[2], y[3])};
        }
    }
    __syncthreads();
    const int64_t o = ((int64_t)g * B + s0) * H + f0;
    if (MODE == 0) stage_out<kTile, kTile>(smem, a.h1 + o, H, srows, nullptr);
    else stage_out<kTile, kTile>(smem, a.dz1 + o, H, srows, a.h1 + o);
}

// --------------------------------------------------------------- fwd2
// All H features of 128 samples: z2 = W2 h1 + b2 and the loss epilogue.
// Wave w owns features (H / 4) w .. + H / 4 - 1 (MT row tiles of 16).
template <int H>
__global__ __launch_bounds__(kThreads) void big_fwd2_kernel(BigArgs a) {
    extern __shared__ __align__(16) uint16_t smem[];
    constexpr int MT = H / 64, NST = 3, STG = (H + kFwd2Samples) * kBK;
    constexpr int LPT = (H + kFwd2Samples) * 4 / kThreads;
    const int g = blockIdx.y, blk = blockIdx.x;
    const int B = a.B, s0 = blk * kFwd2Samples;
    const uint16_t* A = a.w2s + (int64_t)g * H * H;
    const uint16_t* Bm = a.h1 + ((int64_t)g * B + s0) * H;
    const int srows = B - s0;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lo = kc_lane();
    constexpr int RING = NST * STG, STAGE = kFwd2Samples * H;
    float* svp = (float*)(smem + (RING > STAGE ? RING : STAGE));  // [4][128] V partials of each wave

    f4 acc[MT][8];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};

    kloop<NST, LPT>(
        H / kBK,
        [&](int s, int buf) {
            uint16_t* st_ = smem + buf * STG;
            dma_kc<H>(A, H, H, s * kBK, st_);
            dma_kc<kFwd2Samples>(Bm, H, srows, s * kBK, st_ + H * kBK);
        },
        [&](int, int buf) {
            const uint16_t* ta = smem + buf * STG + ((H / 4) * wv) * kBK + lo;
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
        });

    const int l = threadIdx.x & 63, l16 = l & 15, q = l >> 4;
    const float* prm = a.params + (int64_t)g * a.P;
    const int fb0 = (H / 4) * wv + 4 * q;
    // z2 = acc + b2; this wave's part of v for each of its 8 samples
    float w3v[MT][4];
    float vp[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) vp[j] = 0.f;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int f = fb0 + 16 * i + r;
            const float b2 = prm[a.off_b2 + f];
            w3v[i][r] = prm[a.off_w3 + f];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float z = acc[i][j][r] + b2;
                acc[i][j][r] = z;
                vp[j] = fmaf(w3v[i][r], z > 0.f ? z : 0.f, vp[j]);
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
                const float v = ((svp[sl] + svp[kFwd2Samples + sl]) +
                                 (svp[2 * kFwd2Samples + sl] + svp[3 * kFwd2Samples + sl])) + b3;
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
        const float v = ((svp[sl] + svp[kFwd2Samples + sl]) + (svp[2 * kFwd2Samples + sl] + svp[3 * kFwd2Samples + sl])) + b3;
        dv[j] = 0.f;
        if (s < B) {
            const float diff = a.q[s] - v;
            const float w = diff >= 0.f ? tau : 1.f - tau;
            dv[j] = -2.f * w * diff * a.invB;
            lsum += w * diff * diff;
            dsum += dv[j];
            if (wv == 0 && q == 0 && a.out_v) a.out_v[(int64_t)g * B + s] = v;
        }
    }
    float* sp = a.spart + ((int64_t)g * a.nblk + blk) * (2 * H + 1);
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
        float db2[4] = {0.f, 0.f, 0.f, 0.f}, dw3[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float d[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float z = acc[i][j][r];
                d[r] = z > 0.f ? dv[j] * w3v[i][r] : 0.f;
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
    __syncthreads();
    stage_out<H, kFwd2Samples>(smem, a.dz2 + ((int64_t)g * B + s0) * H, H, srows, nullptr);
}

// --------------------------------------------------------------- wgrad
// Per (chunk, job): job < n2 -> a 256 x 256 tile of dW2 = dz2^T h1; job < n2
// + n1 -> a tile of dW1 = dz1^T s (+ db1 rows when it is the first column
// tile); job == n2 + n1 -> the fwd2 block sums of the chunk.
__global__ __launch_bounds__(kThreads) void big_wgrad_kernel(BigArgs a) {
    extern __shared__ __align__(16) uint16_t smem[];
    constexpr int NST = 4, STG = 2 * kBK * kTile;
    const int g = blockIdx.y;
    const int H = a.H, S = a.S, B = a.B;
    const int nth = H / kTile, nts = (S + kTile - 1) / kTile;
    const int n2 = nth * nth, n1 = nth * nts, njob = n2 + n1 + 1;
    int c, job;
    xcd_map(blockIdx.x, a.nchunk, njob, c, job);
    const int b0 = c * a.chunk;
    const int len = min(a.chunk, B - b0);
    float* part = a.part + ((int64_t)g * a.nchunk + c) * a.Pp;
    const int tid = threadIdx.x;

    if (job == n2 + n1) {
        // block sums of the chunk's 128-sample blocks, in block order
        const int k0 = b0 / kFwd2Samples, k1 = (b0 + len + kFwd2Samples - 1) / kFwd2Samples;
        const float* sp = a.spart + (int64_t)g * a.nblk * (2 * H + 1);
        for (int e = tid; e < 2 * H + 1; e += kThreads) {
            float s = 0.f;
            for (int k = k0; k < k1; ++k) s += sp[(int64_t)k * (2 * H + 1) + e];
            const int64_t off = e < H ? a.off_b2 + e : (e < 2 * H ? a.off_w3 + (e - H) : a.off_b3);
            part[off] = s;
        }
        return;
    }
    const uint16_t* A;
    const uint16_t* Bm;
    int64_t ldb;
    int fa0, fb0, fbmax, ldo;
    float* dst;
    float* rowsum = nullptr;
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
        if (nt == 0) rowsum = part + a.off_b1;
    }
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv & 1, wn = wv >> 1;
    const NatBase nb = nat_base();
    const bool sums = rowsum != nullptr && wn == 0;
    const bf16x8 one = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

    f4 acc[8][8], accb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        accb[i] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f4{0.f, 0.f, 0.f, 0.f};
    }
    const int nsl = (len + kBK - 1) / kBK;
    const int tail = len - (nsl - 1) * kBK;  // samples of the last slice, 1 .. 32

    kloop<NST, 8>(
        nsl,
        [&](int s, int buf) {
            uint16_t* st_ = smem + buf * STG;
            const int sm = len - s * kBK;
            dma_nat(A + (int64_t)s * kBK * H, H, sm, fa0, H, st_);
            dma_nat(Bm + (int64_t)s * kBK * ldb, ldb, sm, fb0, fbmax, st_ + kBK * kTile);
        },
        [&](int s, int buf) {
            uint16_t* ta = smem + buf * STG;
            uint16_t* tb = ta + kBK * kTile;
            if (s == nsl - 1 && tail < kBK) {
                // samples past the end of the chunk contribute zero
                for (int e = tid; e < 2 * (kBK - tail) * (kTile / 8); e += kThreads) {
                    const int t = e / ((kBK - tail) * (kTile / 8)), rem = e - t * ((kBK - tail) * (kTile / 8));
                    const int row = tail + rem / (kTile / 8), u = rem % (kTile / 8);
                    *(u32x4*)((t ? tb : ta) + row * kTile + 8 * u) = u32x4{0u, 0u, 0u, 0u};
                }
                __syncthreads();
            }
            bf16x8 fa[8], fb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) fb[j] = nat_frag(tb, nb, 8 * wn + j);
#pragma unroll
            for (int i = 0; i < 8; ++i) fa[i] = nat_frag(ta, nb, 8 * wm + i);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = mma(fa[i], fb[j], acc[i][j]);
                if (sums) accb[i] = mma(fa[i], one, accb[i]);
            }
        });

    const int l = tid & 63, l16 = l & 15, q = l >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int m = fa0 + 128 * wm + 16 * i + 4 * q;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int n = fb0 + 128 * wn + 16 * j + l16;
            if (n < fbmax) {
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[(int64_t)(m + r) * ldo + n] = acc[i][j][r];
            }
        }
        if (sums && l16 == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) rowsum[m + r] = accb[i][r];
        }
    }
}

constexpr size_t tile_lds_bytes() { return (size_t)4 * 2 * kTile * kBK * 2; }
template <int H>
constexpr size_t fwd2_lds_bytes() {
    return (size_t)(3 * (H + kFwd2Samples) * kBK > kFwd2Samples * H ? 3 * (H + kFwd2Samples) * kBK : kFwd2Samples * H) * 2 +
           4 * kFwd2Samples * sizeof(float);
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
int iql_big_max_chunks(int S, int H) {
    const int nth = H / kTile, nts = (S + kTile - 1) / kTile;
    const int tiles = nth * nth + nth * nts;
    return 256 / tiles > 1 ? 256 / tiles : 1;
}
// samples per weight-gradient chunk for a batch of B rows: a multiple of the
// fwd2 block, so every block's sums belong to exactly one chunk
int iql_big_chunk(int S, int H, int B) {
    const int target = iql_big_max_chunks(S, H);
    int c = (B + target - 1) / target;
    c = (c + kFwd2Samples - 1) / kFwd2Samples * kFwd2Samples;
    return c < kFwd2Samples ? kFwd2Samples : c;
}

static hipError_t big_launch(const IqlDims& d, const IqlBuffers& b, const float* tau, const void* states, int64_t ld,
                             const float* q, int B, float* out_v, const ValueOut* vo, hipStream_t stream);

hipError_t launch_iql_big_fwd_bwd(const IqlDims& d, const IqlBuffers& b, const float* tau, const void* states,
                                  int64_t ld, const float* q, int B, float* out_v, hipStream_t stream) {
    return big_launch(d, b, tau, states, ld, q, B, out_v, nullptr, stream);
}

hipError_t launch_iql_big_forward(const IqlDims& d, const IqlBuffers& b, const void* states, int64_t ld, int B,
                                  const ValueOut& vo, hipStream_t stream) {
    const float tau[2] = {0.f, 0.f};
    return big_launch(d, b, tau, states, ld, nullptr, B, nullptr, &vo, stream);
}

static hipError_t big_launch(const IqlDims& d, const IqlBuffers& b, const float* tau, const void* states, int64_t ld,
                             const float* q, int B, float* out_v, const ValueOut* vo, hipStream_t stream) {
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
    a.chunk = iql_big_chunk(S, H, B);
    a.nchunk = (B + a.chunk - 1) / a.chunk;
    a.nblk = iql_big_blocks(B);
    if (vo) {
        a.fwd_only = 1;
        a.vo = *vo;
    }

    static bool attr = false;
    if (!attr) {
        hipError_t e = allow_lds(big_tile_kernel<0>, tile_lds_bytes());
        if (e == hipSuccess) e = allow_lds(big_tile_kernel<1>, tile_lds_bytes());
        if (e == hipSuccess) e = allow_lds(big_wgrad_kernel, tile_lds_bytes());
        if (e == hipSuccess) e = allow_lds(big_fwd2_kernel<256>, fwd2_lds_bytes<256>());
        if (e == hipSuccess) e = allow_lds(big_fwd2_kernel<512>, fwd2_lds_bytes<512>());
        if (e != hipSuccess) return e;
        attr = true;
    }
    const int nst = (B + kTile - 1) / kTile;
    const dim3 gt(nst * (H / kTile), G);
    hipLaunchKernelGGL(big_tile_kernel<0>, gt, dim3(kThreads), tile_lds_bytes(), stream, a);
    const dim3 g2(a.nblk, G);
    if (H == 512) hipLaunchKernelGGL(big_fwd2_kernel<512>, g2, dim3(kThreads), fwd2_lds_bytes<512>(), stream, a);
    else hipLaunchKernelGGL(big_fwd2_kernel<256>, g2, dim3(kThreads), fwd2_lds_bytes<256>(), stream, a);
    if (vo) return hipGetLastError();
    hipLaunchKernelGGL(big_tile_kernel<1>, gt, dim3(kThreads), tile_lds_bytes(), stream, a);
    const int nth = H / kTile, nts = (S + kTile - 1) / kTile;
    const int njob = nth * nth + nth * nts + 1;
    const dim3 gw(a.nchunk * njob, G);
    hipLaunchKernelGGL(big_wgrad_kernel, gw, dim3(kThreads), tile_lds_bytes(), stream, a);
    return hipGetLastError();
}

}  // namespace iqlh
