// IQL value-network step: fused V(s) forward + expectile loss + backward,
// fixed-order gradient reduction, clipped Adam.  gfx950 MFMA.
//
// What is computed ("GPU IQL + HER Porting Plan", sections "Current State /
// IQL (CPU)" and "CUDA Kernel: iql_value_kernel.cu"):
//   z1 = W1 s + b1, h1 = relu(z1), z2 = W2 h1 + b2, h2 = relu(z2),
//   v = w3 . h2 + b3, diff = q - v, w = tau (diff >= 0) or 1 - tau,
//   loss = mean(w diff^2), dv = -2 w diff / B, and the gradients of the six
//   parameter tensors; then the global-norm clip and Adam of "DQN
//   Backward-Path NaN Audit -- SP1 Phase A" (section on iqn_adam_kernel).
// The high/low trainers of "Phase 2: Multi-Stream Graph Parallelism" (section
// "2C. Grouped GEMM for IQL") run as one grouped launch: blockIdx.y = group.
//
// MI355X design (not the pages' warp-per-sample kernel nor a chain of library
// GEMMs): one workgroup holds 128 samples of one group and runs the whole
// forward, loss and backward for them on MFMA, with the weights and the
// activations in LDS; gradients leave the workgroup as fp32 partials, a
// second kernel sums them in workgroup order (no float atomics: bitwise
// reproducible) and a third applies the clip and Adam and refreshes the
// operand-typed W1 / W2 / W2^T shadows the next step reads (no conversion or
// transpose in the hot kernel).  Three kernels:
//   * iql_fused16w_kernel (bf16 operands, hidden 128): sixteen wave64s,
//     v_mfma_f32_16x16x32_bf16, activations in natural [sample][feature]
//     tiles read back with LDS transpose loads; described at its definition.
//   * iql_fused_fs_kernel (fp32 operands, hidden 128): four wave64s share a
//     32-sample tile and split its features; described at its definition.
//   * iql_fused_kernel (hidden 32, fp32 or bf16 operands): NW wave64s of 32
//     samples each on v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2f32 in the
//     orientation D[feature][sample] = W[feature][k] act[sample][k]; the
//     accumulators of one layer are fed back, rounded to the operand type, as
//     the B operand of the next (the weight operand is read with its k
//     columns permuted to the same order), and the weight-gradient operands
//     are written to LDS transposed ([feature][sample]); bias gradients and
//     dw3 are row sums of the same tiles through an all-ones operand.
#include <hip/hip_ext.h>

#include "budget_block.hpp"
#include "common.hpp"
#include "her_block.hpp"
#include "iql_update.hpp"
#include "launch.hpp"

namespace iqlh {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- operands
template <typename T> struct Op;

template <> struct Op<uint16_t> {  // bfloat16 storage
    static constexpr int KS = 16;   // k per MFMA
    static constexpr int KPL = 8;   // k per lane (lane half h holds 8h .. 8h+7)
    static constexpr int PAD = 8;   // LDS row padding, elements (16 bytes)
    typedef bf16x8 frag;
    static IQLH_DEV f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static IQLH_DEV frag zero() { return __builtin_bit_cast(frag, u32x4{0u, 0u, 0u, 0u}); }
    static IQLH_DEV frag keep(bool c, frag x) {
        const uint32_t m = c ? 0xFFFFFFFFu : 0u;
        return __builtin_bit_cast(frag, __builtin_bit_cast(u32x4, x) & u32x4{m, m, m, m});
    }
    // KPL consecutive elements (16-byte aligned)
    static IQLH_DEV frag load(const uint16_t* p) {
        return __builtin_bit_cast(frag, *(const u32x4*)p);
    }
    // chained-k fragment of k step u for lane half h: two runs of four
    static IQLH_DEV frag load_chain(const uint16_t* row, int u, int h) {
        const int c0 = 16 * u + 4 * h;
        const u32x2 lo = *(const u32x2*)(row + c0);
        const u32x2 hi = *(const u32x2*)(row + c0 + 8);
        return __builtin_bit_cast(frag, u32x4{lo.x, lo.y, hi.x, hi.y});
    }
    // two floats -> packed bfloat16 pair, round to nearest even
    // (v_cvt_pk_bf16_f32 on gfx950)
    static IQLH_DEV uint32_t cvt2(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
    }
    // B operand of k step u from a layer's accumulators
    template <int NT>
    static IQLH_DEV frag from_acc(const f32x16 (&acc)[NT], int u) {
        const f32x16& a = acc[u >> 1];
        const int r = 8 * (u & 1);
        return __builtin_bit_cast(frag, u32x4{cvt2(a[r + 0], a[r + 1]), cvt2(a[r + 2], a[r + 3]),
                                             cvt2(a[r + 4], a[r + 5]), cvt2(a[r + 6], a[r + 7])});
    }
    static IQLH_DEV frag ones() {
        return __builtin_bit_cast(frag, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    }
    // element e (0 .. KPL-1) of a fragment, as stored
    static IQLH_DEV uint16_t half(frag f, int e) {
        const u32x4 u = __builtin_bit_cast(u32x4, f);
        return (e & 1) ? (uint16_t)(u[e >> 1] >> 16) : (uint16_t)(u[e >> 1] & 0xFFFFu);
    }
    // writes two consecutive-feature values of one sample into a [feature][sample] tile
    static IQLH_DEV void put2(uint16_t* tile, int idx, int ld, float lo, float hi) {
        const uint32_t pk = cvt2(lo, hi);
        tile[idx] = (uint16_t)(pk & 0xFFFFu);
        tile[idx + ld] = (uint16_t)(pk >> 16);
    }
    static IQLH_DEV frag make(const uint16_t* t) {
        return __builtin_bit_cast(frag, u32x4{(uint32_t)t[0] | ((uint32_t)t[1] << 16),
                                             (uint32_t)t[2] | ((uint32_t)t[3] << 16),
                                             (uint32_t)t[4] | ((uint32_t)t[5] << 16),
                                             (uint32_t)t[6] | ((uint32_t)t[7] << 16)});
    }
    static IQLH_DEV uint16_t cvt(float x) { return (uint16_t)(cvt2(x, 0.f) & 0xFFFFu); }
    static IQLH_DEV float tof(uint16_t x) { return bf2f(x); }
    static IQLH_DEV void elems(frag f, float* out) {
        const u32x4 u = __builtin_bit_cast(u32x4, f);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = bf2f((uint16_t)(u[i] & 0xFFFFu));
            out[2 * i + 1] = bf2f((uint16_t)(u[i] >> 16));
        }
    }
    static IQLH_DEV bool chain_positive(frag f, int e) {
        const u32x4 u = __builtin_bit_cast(u32x4, f);
        const uint32_t w = u[e >> 1];
        const uint16_t b = (e & 1) ? (uint16_t)(w >> 16) : (uint16_t)(w & 0xFFFFu);
        return b != 0;  // relu outputs are +0 or positive
    }
};

template <> struct Op<float> {
    static constexpr int KS = 2;
    static constexpr int KPL = 1;
    static constexpr int PAD = 4;
    typedef float frag;
    static IQLH_DEV f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static IQLH_DEV frag keep(bool c, frag x) { return keep_if(c, x); }
    static IQLH_DEV frag zero() { return 0.f; }
    static IQLH_DEV frag load(const float* p) { return *p; }
    static IQLH_DEV frag load_chain(const float* row, int u, int h) {
        return row[32 * (u >> 4) + 8 * ((u & 15) >> 2) + 4 * h + (u & 3)];
    }
    template <int NT>
    static IQLH_DEV frag from_acc(const f32x16 (&acc)[NT], int u) {
        return acc[u >> 4][u & 15];
    }
    static IQLH_DEV frag make(const float* t) { return t[0]; }
    static IQLH_DEV frag ones() { return 1.f; }
    static IQLH_DEV float half(frag f, int) { return f; }
    static IQLH_DEV void put2(float* tile, int idx, int ld, float lo, float hi) {
        tile[idx] = lo;
        tile[idx + ld] = hi;
    }
    static IQLH_DEV float cvt(float x) { return x; }
    static IQLH_DEV float tof(float x) { return x; }
    static IQLH_DEV void elems(frag f, float* out) { out[0] = f; }
    static IQLH_DEV bool chain_positive(frag f, int) { return f > 0.f; }
};

// Parameter offsets inside one group's flat vector.
struct POff {
    int64_t w1, b1, w2, b2, w3, b3;
    IQLH_DEV POff(int S, int H) {
        w1 = 0; b1 = (int64_t)H * S; w2 = b1 + H; b2 = w2 + (int64_t)H * H; w3 = b2 + H; b3 = w3 + H;
    }
};

struct FusedArgs {
    const void* states;
    int64_t ld;
    const float* q;
    const float* params;  // [G][P] fp32 master (biases, w3)
    const void* w1s;      // [G][H][SP]
    const void* w2s;      // [G][H][H]
    const void* w2ts;     // [G][H][H]
    float* part;          // [G][nwg][Pp]
    float* loss_part;     // [G][nwg]
    float* out_v;         // [G][B] or null
    const float* q_all;   // [B][A] or null: advantage-weighted policy fused in
    float* out_pi;        // [G][B][A]
    int A;                // actions, <= 16 when fused
    float beta;
    float tau0, tau1, invB;
    int B, S, nwg;
    int64_t P, Pp;
    int32_t* flags;
    int fwd_only;         // 1: V (and the bootstrap target) only, no loss or gradients
    ValueOut vo;          // outputs of the forward-only pass
    // 16-wave kernel only: HER rows relabelled in the prologue (her_on) -- the
    // batch rows from her_row0 (a multiple of 128) on are HER rows
    // 0 .. B - her_row0 - 1, built from the replay buffer rather than read from
    // `states`, and group 0 writes every HER output; the budget's pass 1
    // (nrm.nb > 0) rides on the 256-thread quarters of the other workgroups.
    int her_on, her_row0;
    HerArgs her;
    NormsArgs nrm;
    // fp32 four-wave kernel only: two workgroups per tile, workgroup 2 t
    // forming tile t's dW2 part of the partial row and 2 t + 1 its dW1 part
    int fs_split;
    // 16-wave kernel only, measurement: [G][nwg][kPhaseStamps] clock values
    // (100 MHz) at the workgroup's phase ends, or null (not recorded)
    uint64_t* stamps;
};

template <typename T, int SP, int H, int NW>
struct FusedCfg {
    static constexpr int BT = 32 * NW;
    static constexpr int NT = H / 32;
    static constexpr int PAD = Op<T>::PAD;
    static constexpr int LDA = BT + PAD;       // activation tiles [rows][LDA]
    static constexpr int LDW1 = SP + PAD;      // W1 [H][LDW1]
    static constexpr int LDW2 = H + PAD;       // W2, W2^T [H][LDW2]
    static constexpr int R0 = (H * LDW1 > H * LDA) ? H * LDW1 : H * LDA;
    static constexpr int R1 = H * LDW2;
    static constexpr int R2 = H * LDA;
    static constexpr int R3 = (SP * LDA > H * LDA) ? SP * LDA : H * LDA;
    static constexpr size_t BYTES_T = (size_t)(R0 + R1 + R2 + R3) * sizeof(T);
    static constexpr size_t BYTES = BYTES_T + (size_t)(3 * H + 2 * NW) * sizeof(float);
    static_assert(SP % 32 == 0 && H % 32 == 0, "tile shape");
    static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// out[i][j] = sum_k A[i][k] * B[j][k] over K = BT columns of two LDS tiles,
// for 32x32 output tiles [t0, t1) (row-major over NCT column tiles); stores
// fp32 results to dst[i * ldo + j] for j < ncols.  When bias_dst is given,
// the row sums sum_k A[i][k] of every row tile whose column tile 0 is in
// the range go to bias_dst[i], from an extra MFMA against an all-ones
// operand (a reduction over samples, i.e. across lanes, for free).
template <typename T, int BT, int MAXT>
IQLH_DEV void lds_gemm_store(const T* A, const T* Bm, int lda, int NCT, int t0, int t1,
                             float* dst, int ldo, int ncols, float* bias_dst) {
    typedef Op<T> O;
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
    const typename O::frag one = O::ones();
    for (int tb = t0; tb < t1; tb += MAXT) {
        const int nb = min(MAXT, t1 - tb);
        f32x16 acc[MAXT], accb[MAXT];
#pragma unroll
        for (int q = 0; q < MAXT; ++q) acc[q] = accb[q] = f32x16{};
        for (int u = 0; u < BT / O::KS; ++u) {
            const int k0 = O::KS * u + O::KPL * h;
            int last_row = -1;
            typename O::frag a = O::zero();
#pragma unroll
            for (int q = 0; q < MAXT; ++q) {
                if (q < nb) {
                    const int tau = tb + q, rt = tau / NCT, ct = tau - rt * NCT;
                    if (rt != last_row) {
                        a = O::load(A + (int64_t)(32 * rt + l32) * lda + k0);
                        last_row = rt;
                    }
                    const typename O::frag b = O::load(Bm + (int64_t)(32 * ct + l32) * lda + k0);
                    acc[q] = O::mma(a, b, acc[q]);
                    if (bias_dst && ct == 0) accb[q] = O::mma(a, one, accb[q]);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < MAXT; ++q) {
            if (q < nb) {
                const int tau = tb + q, rt = tau / NCT, ct = tau - rt * NCT;
                const int j = 32 * ct + l32;
                if (j < ncols) {
                    float* d0 = dst + (32 * rt + 4 * h) * ldo + j;  // 32-bit offsets from a uniform base
#pragma unroll
                    for (int r = 0; r < 16; ++r) d0[(8 * (r >> 2) + (r & 3)) * ldo] = acc[q][r];
                }
                if (bias_dst && ct == 0 && l32 == 0) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) bias_dst[32 * rt + 8 * (r >> 2) + 4 * h + (r & 3)] = accb[q][r];
                }
            }
        }
    }
}

// dst[i] = sum_k A[i][k] over K = BT for the 32-row tiles [rt0, rt1), by
// MFMA against an all-ones operand.
template <typename T, int BT>
IQLH_DEV void lds_rowsum(const T* A, int lda, int rt0, int rt1, float* dst) {
    typedef Op<T> O;
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
    const typename O::frag one = O::ones();
    for (int rt = rt0; rt < rt1; ++rt) {
        f32x16 acc = f32x16{};
        for (int u = 0; u < BT / O::KS; ++u)
            acc = O::mma(O::load(A + (int64_t)(32 * rt + l32) * lda + O::KS * u + O::KPL * h), one, acc);
        if (l32 == 0) {
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[32 * rt + 8 * (r >> 2) + 4 * h + (r & 3)] = acc[r];
        }
    }
}

template <typename T, int SP, int H, int NW, bool XVEC>
__global__ __launch_bounds__(64 * NW) void iql_fused_kernel(FusedArgs a) {
    typedef Op<T> O;
    typedef FusedCfg<T, SP, H, NW> C;
    constexpr int BT = C::BT, NT = C::NT, NTHR = 64 * NW;
    constexpr int KU1 = SP / O::KS;   // k steps of layer 1
    constexpr int KUH = H / O::KS;    // k steps over hidden
    extern __shared__ __align__(16) unsigned char smem[];
    T* R0 = (T*)smem;
    T* R1 = R0 + C::R0;
    T* R2 = R1 + C::R1;
    T* R3 = R2 + C::R2;
    float* sb1 = (float*)(R3 + C::R3);
    float* sb2 = sb1 + H;
    float* sw3 = sb2 + H;
    float* sred = sw3 + H;  // [2][NW]

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
    const int g = blockIdx.y, wg = blockIdx.x;
    const int S = a.S, B = a.B;
    const POff po(S, H);
    const float* prm = a.params + (int64_t)g * a.P;
    const T* w1s = (const T*)a.w1s + (int64_t)g * H * SP;
    const T* w2s = (const T*)a.w2s + (int64_t)g * H * H;
    const T* w2ts = (const T*)a.w2ts + (int64_t)g * H * H;
    float* part = a.part + ((int64_t)g * a.nwg + wg) * a.Pp;
    const float tau = g == 0 ? a.tau0 : a.tau1;

    // ---- S0: every load first (weights, biases and w3, the X fragments,
    // then Q below), the LDS stores after them: constant trip counts and
    // clamped indexes, so that no load is waited on before the next one is
    // issued (a load-store loop made each weight load a round trip of its own)
    constexpr int NL1 = H * SP / (NTHR * O::KPL), NL2 = H * H / (NTHR * O::KPL);
    static_assert(NL1 * NTHR * O::KPL == H * SP && NL2 * NTHR * O::KPL == H * H && H <= NTHR,
                  "whole staging passes");
    typename O::frag w1r[NL1], w2r[NL2];
#pragma unroll
    for (int i = 0; i < NL1; ++i) w1r[i] = O::load(w1s + (tid + i * NTHR) * O::KPL);
#pragma unroll
    for (int i = 0; i < NL2; ++i) w2r[i] = O::load(w2s + (tid + i * NTHR) * O::KPL);
    const int th = tid < H ? tid : 0;
    const float pb1 = prm[po.b1 + th], pb2 = prm[po.b2 + th], pw3 = prm[po.w3 + th];
    const int bl = 32 * wv + l32;              // sample within the tile
    const int b = wg * BT + bl;                // sample in the batch
    const bool valid = b < B;
    typename O::frag xf[KU1];
    {
        const T* xr = (const T*)a.states + (int64_t)(valid ? b : B - 1) * a.ld;
        // XVEC: S == SP and rows aligned to whole fragments (checked on the host)
#pragma unroll
        for (int u = 0; u < KU1; ++u) {
            const int k0 = O::KS * u + O::KPL * h;
            // (masked by AND rather than a select, which the compiler turns
            // into a branch around each load with a wait inside it)
            if (XVEC) {
                xf[u] = O::keep(valid, O::load(xr + k0));
            } else {
                T tmp[O::KPL];
#pragma unroll
                for (int e = 0; e < O::KPL; ++e) {
                    const int k = k0 + e;
                    tmp[e] = keep_if(valid && k < S, xr[k < S ? k : S - 1]);
                }
                xf[u] = O::make(tmp);
            }
        }
    }
    // with the policy fused in: lane (l32, h) takes actions h, h + 2, ... of
    // its sample
    float qa[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) qa[k] = 0.f;
    if (a.out_pi) {  // uniform; indexes clamped, unused values never read
        const int64_t bc = valid ? b : B - 1;
#pragma unroll
        for (int k = 0; k < 8; ++k) qa[k] = a.q_all[bc * a.A + min(h + 2 * k, a.A - 1)];
    }
#pragma unroll
    for (int i = 0; i < NL1; ++i) {
        const int idx = (tid + i * NTHR) * O::KPL, r = idx / SP, c = idx - r * SP;
        *(typename O::frag*)(R0 + r * C::LDW1 + c) = w1r[i];
    }
#pragma unroll
    for (int i = 0; i < NL2; ++i) {
        const int idx = (tid + i * NTHR) * O::KPL, r = idx / H, c = idx - r * H;
        *(typename O::frag*)(R1 + r * C::LDW2 + c) = w2r[i];
    }
    if (tid < H) {
        sb1[tid] = pb1;
        sb2[tid] = pb2;
        sw3[tid] = pw3;
    }
    lds_barrier();

    // ---- F1: z1^T = W1 * s^T
    f32x16 acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
#pragma unroll
    for (int u = 0; u < KU1; ++u) {
        const int k0 = O::KS * u + O::KPL * h;
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = O::mma(O::load(R0 + (32 * t + l32) * C::LDW1 + k0), xf[u], acc[t]);
    }
    // epilogue: h1 = relu(z1 + b1); h1^T tile to R3 (registers r, r+1 hold
    // features f, f+1 of this lane's sample)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int f = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
            const float z0 = acc[t][r] + sb1[f], z1 = acc[t][r + 1] + sb1[f + 1];
            const float y0 = z0 > 0.f ? z0 : 0.f, y1 = z1 > 0.f ? z1 : 0.f;
            acc[t][r] = y0;
            acc[t][r + 1] = y1;
            O::put2(R3, f * C::LDA + bl, C::LDA, y0, y1);
        }
    }
    typename O::frag h1f[KUH];
#pragma unroll
    for (int u = 0; u < KUH; ++u) h1f[u] = O::template from_acc<NT>(acc, u);
    // relu'(z1) of this lane's 16*NT features, one bit per accumulator register
    uint32_t mask1[(16 * NT + 31) / 32];
#pragma unroll
    for (int w = 0; w < (16 * NT + 31) / 32; ++w) mask1[w] = 0u;
    // acc holds relu outputs (+0 or positive): bits + 0x7FFFFFFF carries into
    // bit 31 exactly when the value is positive (no compare, no lane mask)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            mask1[(16 * t + r) >> 5] |= ((__float_as_uint(acc[t][r]) + 0x7FFFFFFFu) >> 31)
                                        << ((16 * t + r) & 31);
    lds_barrier();

    // ---- F2: z2^T = W2 * h1^T  (A read with the chained k order)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
#pragma unroll
    for (int u = 0; u < KUH; ++u) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = O::mma(O::load_chain(R1 + (32 * t + l32) * C::LDW2, u, h), h1f[u], acc[t]);
    }
    // epilogue: v, expectile, dv, dz2
    float vpart = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int f = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
            const float z = acc[t][r] + sb2[f];
            acc[t][r] = z;
            vpart = fmaf(sw3[f], z > 0.f ? z : 0.f, vpart);
        }
    }
    const float v = vpart + __shfl_xor(vpart, 32, 64) + prm[po.b3];
    if (a.fwd_only) {
        if (valid && h == 0) write_value(a.vo, g, B, b, v);
        return;
    }
    if (a.out_pi) {
        // pi = softmax(beta * clamp(Q - V, -10, 10)) with the row maximum
        // subtracted ("Current State / IQL (CPU)", advantage-weighted action
        // selection); the two lanes of a sample share it
        float x[8], mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            x[k] = h + 2 * k < a.A ? a.beta * fminf(fmaxf(qa[k] - v, -10.f), 10.f) : -INFINITY;
            mx = fmaxf(mx, x[k]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // the hardware exponential (about 1e-6 relative on these arguments,
        // which lie in [-20 beta, 0]), as in the bf16 hidden-128 kernel
        float se = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            x[k] = h + 2 * k < a.A ? __expf(x[k] - mx) : 0.f;
            se += x[k];
        }
        se += __shfl_xor(se, 32, 64);
        if (valid) {
            float* pr = a.out_pi + ((int64_t)g * B + b) * a.A;
            const float inv = 1.f / se;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (h + 2 * k < a.A) pr[h + 2 * k] = x[k] * inv;
        }
    }
    float dv = 0.f, lterm = 0.f;
    if (valid) {
        const float diff = a.q[b] - v;
        const float w = diff >= 0.f ? tau : 1.f - tau;
        lterm = w * diff * diff;
        dv = -2.f * w * diff * a.invB;
        if (h == 0 && a.out_v) a.out_v[(int64_t)g * B + b] = v;
    }
    {
        const float ls = wave_sum(h == 0 ? lterm : 0.f);
        const float ds = wave_sum(h == 0 ? dv : 0.f);
        if (lane == 0) { sred[wv] = ls; sred[NW + wv] = ds; }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int f = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
            const float z0 = acc[t][r], z1 = acc[t][r + 1];
            const float dz0 = z0 > 0.f ? dv * sw3[f] : 0.f;
            const float dz1 = z1 > 0.f ? dv * sw3[f + 1] : 0.f;
            const float p0 = z0 > 0.f ? z0 * dv : 0.f;   // h2 * dv: row sums give dw3
            const float p1 = z1 > 0.f ? z1 * dv : 0.f;
            acc[t][r] = dz0;
            acc[t][r + 1] = dz1;
            O::put2(R0, f * C::LDA + bl, C::LDA, dz0, dz1);  // dz2^T
            O::put2(R2, f * C::LDA + bl, C::LDA, p0, p1);
        }
    }
    typename O::frag dz2f[KUH];
#pragma unroll
    for (int u = 0; u < KUH; ++u) dz2f[u] = O::template from_acc<NT>(acc, u);
    lds_barrier();

    // ---- dw3 (row sums of h2 * dv), db3, loss, then dW2 = dz2^T h1 with db2
    lds_rowsum<T, BT>(R2, C::LDA, wv * NT / NW, (wv + 1) * NT / NW, part + po.w3);
    if (tid == 0) {
        float ls = 0.f, ds = 0.f;
        for (int i = 0; i < NW; ++i) { ls += sred[i]; ds += sred[NW + i]; }
        a.loss_part[(int64_t)g * a.nwg + wg] = ls;
        part[po.b3] = ds;
    }
    // W2^T shadow into R1 (W2 is no longer read after F2)
    for (int idx = tid * O::KPL; idx < H * H; idx += NTHR * O::KPL) {
        const int r = idx / H, c = idx - r * H;
        *(typename O::frag*)(R1 + r * C::LDW2 + c) = O::load(w2ts + idx);
    }
    {
        constexpr int T2 = NT * NT;
        const int t0 = wv * T2 / NW, t1 = (wv + 1) * T2 / NW;
        lds_gemm_store<T, BT, 4>(R0, R3, C::LDA, NT, t0, t1, part + po.w2, H, H, part + po.b2);
    }
    lds_barrier();

    // ---- s^T tile to R3 (h1^T no longer needed); B1: dh1^T = W2^T dz2^T
#pragma unroll
    for (int u = 0; u < KU1; ++u) {
#pragma unroll
        for (int i = 0; i < O::KPL; ++i) R3[(O::KS * u + O::KPL * h + i) * C::LDA + bl] = O::half(xf[u], i);
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x16{};
#pragma unroll
    for (int u = 0; u < KUH; ++u) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            acc[t] = O::mma(O::load_chain(R1 + (32 * t + l32) * C::LDW2, u, h), dz2f[u], acc[t]);
    }
    // dz1 = dh1 * relu'(z1) (mask from the rounded h1 operands), dz1^T to R2
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            const int f = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
            const int bit = 16 * t + r;
            const bool pos0 = (mask1[bit >> 5] >> (bit & 31)) & 1u;
            const bool pos1 = (mask1[(bit + 1) >> 5] >> ((bit + 1) & 31)) & 1u;
            O::put2(R2, f * C::LDA + bl, C::LDA, pos0 ? acc[t][r] : 0.f, pos1 ? acc[t][r + 1] : 0.f);
        }
    }
    lds_barrier();

    // ---- dW1 = dz1^T s with db1
    {
        constexpr int NCT = SP / 32;
        constexpr int T3 = NT * NCT;
        const int t0 = wv * T3 / NW, t1 = (wv + 1) * T3 / NW;
        lds_gemm_store<T, BT, 4>(R2, R3, C::LDA, NCT, t0, t1, part + po.w1, S, S, part + po.b1);
    }
}

// ------------------------------------------- fp32, four waves per 32 samples
// dst[32 rt + i] = the sum of the 32 columns of row 32 rt + i of an LDS tile
// (row stride LDA floats, rows 16-byte aligned): lanes 2i and 2i + 1 each add
// 16 columns from four 16-byte reads, then each other's sums.
template <int LDA>
IQLH_DEV void fs_rowsum(const float* T, int rt, float* dst) {
    static_assert(LDA % 4 == 0, "16-byte rows");
    const int lane = threadIdx.x & 63, i = lane >> 1, half = lane & 1;
    const float4* p = (const float4*)(T + (32 * rt + i) * LDA + 16 * half);
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float4 x = p[k];
        sum += (x.x + x.y) + (x.z + x.w);
    }
    sum += __shfl_xor(sum, 1, 64);
    if (half == 0) dst[32 * rt + i] = sum;
}

// Output tiles (rt, 0 .. NCT - 1) of out[i][j] = sum_k A[i][k] Bm[j][k] over
// the K = 32 columns of two LDS tiles (row stride LDA), unrolled over k;
// fp32 results to dst[i * ldo + j] for j < ncols.
template <int NCT, int LDA>
IQLH_DEV void fs_wgrad(const float* A, const float* Bm, int rt, float* dst, int ldo, int ncols) {
    typedef Op<float> O;
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
    f32x16 acc[NCT];
#pragma unroll
    for (int q = 0; q < NCT; ++q) acc[q] = f32x16{};
    const float* ar = A + (32 * rt + l32) * LDA + h;
    const float* br = Bm + l32 * LDA + h;
#pragma unroll
    for (int u = 0; u < 32 / O::KS; ++u) {
        const float av = ar[O::KS * u];
#pragma unroll
        for (int q = 0; q < NCT; ++q) acc[q] = O::mma(av, br[32 * q * LDA + O::KS * u], acc[q]);
    }
#pragma unroll
    for (int q = 0; q < NCT; ++q) {
        const int j = 32 * q + l32;
        if (j < ncols) {
            float* d0 = dst + (32 * rt + 4 * h) * ldo + j;
#pragma unroll
            for (int r = 0; r < 16; ++r) d0[(8 * (r >> 2) + (r & 3)) * ldo] = acc[q][r];
        }
    }
}

// The same step for fp32 operands at hidden 128 (e.g. batch 4096, state 42).
// The fp32 weights fill ~140 KB of LDS, so one workgroup fits a CU; with one
// wave per 32 samples (the kernel above) three of the CU's four SIMDs would
// idle.  Here four waves share one 32-sample tile and split its features:
// wave w owns row tile w (32 features) of every layer, its MFMAs read the
// other waves' activations from the tiles in LDS (natural k order), and V
// adds the four waves' partial dot products in a fixed order.  The backward
// product dh1^T = W2^T dz2^T reads W2 from LDS by columns (lane l32 takes
// column 32 w + l32 of row k: consecutive addresses), so no transposed copy
// of W2 is staged.  The weight gradients of row tile w need only wave w's
// rows of dz2 and dz1 (and every wave's h1 or s), and the bias and w3
// gradients are row sums of those rows, so after the exchange of dz2 no
// further barrier is needed.
template <int SP, int H, bool XVEC>
__global__ __launch_bounds__(256) void iql_fused_fs_kernel(FusedArgs a) {
    typedef Op<float> O;
    typedef FusedCfg<float, SP, H, 1> C;  // the 32-sample tile layout
    constexpr int NW = 4, BT = 32, NT = H / 32, KU1 = SP / O::KS, KUH = H / O::KS, NTHR = 64 * NW;
    constexpr int LDA = C::LDA;
    static_assert(NT == NW, "one row tile per wave");
    extern __shared__ __align__(16) unsigned char smem[];
    float* R0 = (float*)smem;  // W1, then dz2^T [H][LDA] and s^T [SP][LDA] behind it
    float* R1 = R0 + C::R0;    // W2
    float* R2 = R1 + C::R1;    // h2 dv, then dz1^T (each wave its own row tile)
    float* R3 = R2 + C::R2;    // h1^T
    float* Rs = R0 + H * LDA;
    static_assert(H * LDA + SP * LDA <= C::R0, "s^T behind dz2^T");
    float* sb1 = R3 + C::R3;
    float* sb2 = sb1 + H;
    float* sw3 = sb2 + H;
    float* sred = sw3 + H;     // [2]: the tile's loss and dv sums
    float* svp = sred + 2;     // [NW][BT]: each wave's part of V

    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, h = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index = row tile, uniform
    const int g = blockIdx.y;
    // with fs_split, workgroups 2 t and 2 t + 1 both run tile t's forward and
    // dz2; the first then forms dW2, db2, dw3, db3 and the loss, the second
    // dh1, dz1, dW1 and db1 (disjoint slots of the tile's partial row)
    const int wg = a.fs_split ? (int)blockIdx.x >> 1 : (int)blockIdx.x;
    const bool do_w2 = !a.fs_split || (blockIdx.x & 1) == 0;  // uniform
    const bool do_w1 = !a.fs_split || (blockIdx.x & 1) == 1;
    const int S = a.S, B = a.B;
    const POff po(S, H);
    const float* prm = a.params + (int64_t)g * a.P;
    const float* w1s = (const float*)a.w1s + (int64_t)g * H * SP;
    const float* w2s = (const float*)a.w2s + (int64_t)g * H * H;
    float* part = a.part + ((int64_t)g * a.nwg + wg) * a.Pp;
    const float tau = g == 0 ? a.tau0 : a.tau1;

    // ---- S0: loads in the order of use: W1 and the tile's s (F1; lane half
    // h holds the odd or even k of each step), q, b3, the biases and w3,
    // then W2, which goes to LDS after F1's products
    // (rows of SP and H floats and LDS strides of LDW1, LDW2: whole float4s)
    static_assert(C::LDW1 % 4 == 0 && C::LDW2 % 4 == 0 && SP % 4 == 0, "float4 rows");
    static_assert((H * SP) % (4 * NTHR) == 0 && (H * H) % (4 * NTHR) == 0 && H <= NTHR, "whole passes");
    constexpr int N1 = H * SP / (4 * NTHR), N2 = H * H / (4 * NTHR);
    typedef float f4 __attribute__((ext_vector_type(4)));  // (a union-free vector: kept in registers)
    f4 w1v[N1], w2v[N2];
#pragma unroll
    for (int i = 0; i < N1; ++i) w1v[i] = *(const f4*)(w1s + 4 * (tid + i * NTHR));
    const int bl = l32, b = wg * BT + bl;
    const bool valid = b < B;
    float xf[KU1];
    {
        const float* xr = (const float*)a.states + (int64_t)b * a.ld;
#pragma unroll
        for (int u = 0; u < KU1; ++u) {
            const int k = O::KS * u + h;
            xf[u] = (valid && (XVEC || k < S)) ? xr[k] : 0.f;
        }
    }
    const float qb = (valid && !a.fwd_only) ? a.q[b] : 0.f;  // q is null in the forward-only pass
    const float b3 = prm[po.b3];
    float pb1 = 0.f, pb2 = 0.f, pw3 = 0.f;
    if (tid < H) {
        pb1 = prm[po.b1 + tid];
        pb2 = prm[po.b2 + tid];
        pw3 = prm[po.w3 + tid];
    }
#pragma unroll
    for (int i = 0; i < N2; ++i) w2v[i] = *(const f4*)(w2s + 4 * (tid + i * NTHR));
    // with the policy fused in: wave wv takes samples 8 wv .. 8 wv + 7 of the
    // tile, eight lanes per sample, actions (lane & 7) and (lane & 7) + 8
    const int psl = 8 * wv + (lane >> 3), pb = wg * BT + psl;
    float qa[2] = {0.f, 0.f};
    if (a.out_pi && do_w2) {  // uniform; indexes clamped, unused values never read
        const int64_t pbc = min(pb, B - 1);
#pragma unroll
        for (int k = 0; k < 2; ++k) qa[k] = a.q_all[pbc * a.A + min((lane & 7) + 8 * k, a.A - 1)];
    }
#pragma unroll
    for (int i = 0; i < N1; ++i) {
        const int idx = 4 * (tid + i * NTHR), r = idx / SP, c = idx - r * SP;
        *(f4*)(R0 + r * C::LDW1 + c) = w1v[i];
    }
    if (tid < H) {
        sb1[tid] = pb1;
        sb2[tid] = pb2;
        sw3[tid] = pw3;
    }
    lds_barrier();

    // ---- F1: row tile wv of z1^T = W1 s^T; h1 = relu(z1 + b1) to h1^T (R3)
    const float* w1r = R0 + (32 * wv + l32) * C::LDW1 + h;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int u = 0; u < KU1; ++u) acc = O::mma(w1r[O::KS * u], xf[u], acc);
    // W2 to R1 (first read by F2, after the next barrier)
#pragma unroll
    for (int i = 0; i < N2; ++i) {
        const int idx = 4 * (tid + i * NTHR), r = idx / H, c = idx - r * H;
        *(f4*)(R1 + r * C::LDW2 + c) = w2v[i];
    }
    // lane (l32, h) holds features 32 wv + 8 (r >> 2) + 4 h + (r & 3) of sample l32
    uint32_t mask1 = 0u;  // relu'(z1), one bit per accumulator register
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int f = 32 * wv + 8 * (r >> 2) + 4 * h + (r & 3);
        const float z = acc[r] + sb1[f];
        const float y = z > 0.f ? z : 0.f;
        mask1 |= (z > 0.f ? 1u : 0u) << r;
        R3[f * LDA + bl] = y;
    }
    lds_barrier();

    // ---- F2: row tile wv of z2^T = W2 h1^T (h1^T from R3, every feature)
    const float* w2r = R1 + (32 * wv + l32) * C::LDW2 + h;
    acc = f32x16{};
#pragma unroll
    for (int u = 0; u < KUH; ++u) acc = O::mma(w2r[O::KS * u], R3[(O::KS * u + h) * LDA + l32], acc);
    float vpart = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int f = 32 * wv + 8 * (r >> 2) + 4 * h + (r & 3);
        const float z = acc[r] + sb2[f];
        acc[r] = z;
        vpart = fmaf(sw3[f], z > 0.f ? z : 0.f, vpart);
    }
    vpart += __shfl_xor(vpart, 32, 64);
    if (h == 0) svp[wv * BT + l32] = vpart;
    lds_barrier();
    const float v = ((svp[l32] + svp[BT + l32]) + (svp[2 * BT + l32] + svp[3 * BT + l32])) + b3;
    if (a.fwd_only) {
        if (valid && h == 0 && wv == 0) write_value(a.vo, g, B, b, v);
        return;
    }
    if (a.out_pi && do_w2) {
        // pi = softmax(beta * clamp(Q - V, -10, 10)) with the row maximum
        // subtracted ("Current State / IQL (CPU)", advantage-weighted action
        // selection), from the same V (same sum order) as the step's own
        const float vs = ((svp[psl] + svp[BT + psl]) + (svp[2 * BT + psl] + svp[3 * BT + psl])) + b3;
        float x[2], mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            x[k] = (lane & 7) + 8 * k < a.A ? a.beta * fminf(fmaxf(qa[k] - vs, -10.f), 10.f) : -INFINITY;
            mx = fmaxf(mx, x[k]);
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        // the hardware exponential (about 1e-6 relative on these arguments,
        // which lie in [-20 beta, 0]), as in the bf16 kernel
        float se = 0.f;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            x[k] = (lane & 7) + 8 * k < a.A ? __expf(x[k] - mx) : 0.f;
            se += x[k];
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) se += __shfl_xor(se, o, 64);
        if (pb < B) {
            float* pr = a.out_pi + ((int64_t)g * B + pb) * a.A;
            const float inv = 1.f / se;
#pragma unroll
            for (int k = 0; k < 2; ++k)
                if ((lane & 7) + 8 * k < a.A) pr[(lane & 7) + 8 * k] = x[k] * inv;
        }
    }
    float dv = 0.f, lterm = 0.f;
    if (valid) {
        const float diff = qb - v;
        const float w = diff >= 0.f ? tau : 1.f - tau;
        lterm = w * diff * diff;
        dv = -2.f * w * diff * a.invB;
        if (h == 0 && wv == 0 && do_w2 && a.out_v) a.out_v[(int64_t)g * B + b] = v;
    }
    if (wv == 0) {
        const float ls = wave_sum(h == 0 ? lterm : 0.f);
        const float ds = wave_sum(h == 0 ? dv : 0.f);
        if (lane == 0) { sred[0] = ls; sred[1] = ds; }
    }
    // dz2 = dv w3 relu'(z2) to dz2^T (R0: W1 is no longer read), h2 dv to
    // R2, s^T behind dz2^T (each wave a quarter of the k steps)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int f = 32 * wv + 8 * (r >> 2) + 4 * h + (r & 3);
        const float z = acc[r];
        R0[f * LDA + bl] = z > 0.f ? dv * sw3[f] : 0.f;
        R2[f * LDA + bl] = z > 0.f ? z * dv : 0.f;
    }
#pragma unroll
    for (int u = 0; u < KU1 / NW; ++u) {
        const int uu = wv * (KU1 / NW) + u;
        Rs[(O::KS * uu + h) * LDA + bl] = xf[uu];
    }
    lds_barrier();

    // ---- from here each wave reads its own rows of R0 and R2 and every row
    // of R1, R3 and s^T: dw3 and db2 (row sums), db3 and the loss
    if (do_w2) {
        fs_rowsum<LDA>(R2, wv, part + po.w3);
        fs_rowsum<LDA>(R0, wv, part + po.b2);
        if (tid == 0) {
            a.loss_part[(int64_t)g * a.nwg + wg] = sred[0];
            part[po.b3] = sred[1];
        }
    }
    if (do_w1) {
        // B1: row tile wv of dh1^T = W2^T dz2^T (A: column 32 wv + l32 of
        // W2); dz1 = dh1 relu'(z1) over this wave's rows of R2 (read above)
        acc = f32x16{};
#pragma unroll
        for (int u = 0; u < KUH; ++u)
            acc = O::mma(R1[(O::KS * u + h) * C::LDW2 + 32 * wv + l32], R0[(O::KS * u + h) * LDA + l32], acc);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int f = 32 * wv + 8 * (r >> 2) + 4 * h + (r & 3);
            R2[f * LDA + bl] = (mask1 >> r) & 1u ? acc[r] : 0.f;
        }
    }
    // dW2 = dz2^T h1, db1 (row sums of dz1), dW1 = dz1^T s
    if (do_w2) fs_wgrad<NT, LDA>(R0, R3, wv, part + po.w2, H, H);
    if (do_w1) {
        fs_rowsum<LDA>(R2, wv, part + po.b1);
        fs_wgrad<SP / 32, LDA>(R2, Rs, wv, part + po.w1, S, S);
    }
}
constexpr size_t fs_lds_bytes(size_t table_bytes, int H) { return table_bytes + (size_t)(3 * H + 2 + 4 * 32) * 4; }

// Blocks 0 .. rb - 1 of each group reduce; block rb updates its counters.
__global__ __launch_bounds__(256) void iql_reduce_kernel(const float* __restrict__ part,
                                                         const float* __restrict__ loss_part, int nwg, int nloss,
                                                         int64_t P, int64_t Pp, float invB,
                                                         float* __restrict__ grad, float* __restrict__ sq_part,
                                                         int rb, int32_t* __restrict__ tcount,
                                                         int64_t* __restrict__ step, float* __restrict__ bc,
                                                         float beta1, float beta2, float* __restrict__ out_loss,
                                                         int32_t* __restrict__ flags) {
    if ((int)blockIdx.x < rb)
        iql_reduce_block(part, loss_part, nwg, nloss, P, Pp, invB, grad, sq_part, rb, out_loss, flags, blockIdx.x,
                         blockIdx.y);
    else
        iql_count_block(tcount, step, bc, beta1, beta2, blockIdx.y);
}

template <typename T>
__global__ __launch_bounds__(256) void iql_adam_kernel(IqlDims d, IqlBuffers b, AdamHyper hp,
                                                       float* __restrict__ out_gnorm, int rb) {
    iql_adam_block<T>(d, b, hp, out_gnorm, rb, blockIdx.x, blockIdx.y, gridDim.x);
}

template <typename T>
__global__ __launch_bounds__(256) void iql_shadow_kernel(IqlDims d, IqlBuffers b) {
    const int g = blockIdx.y, H = d.H, H2 = d.H2, S = d.S, SP = d.S_pad;
    const float* prm = b.params + (int64_t)g * d.P;
    T* w1s = (T*)b.w1s + (int64_t)g * H * SP;
    T* w2s = (T*)b.w2s + (int64_t)g * H2 * H;
    T* w2ts = (T*)b.w2ts + (int64_t)g * H2 * H;
    const int64_t ow2 = (int64_t)H * S + H;
    const int64_t n1 = (int64_t)H * SP, n2 = (int64_t)H2 * H;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n1 + n2; i += (int64_t)gridDim.x * 256) {
        if (i < n1) {
            const int64_t r = i / SP, c = i - r * SP;
            w1s[i] = Op<T>::cvt(c < S ? prm[r * S + c] : 0.f);
        } else {
            // W2 [H2][H] and its transpose [H][H2]
            const int64_t q = i - n1, r = q / H, c = q - r * H;
            const float p = prm[ow2 + q];
            w2s[q] = Op<T>::cvt(p);
            w2ts[c * H2 + r] = Op<T>::cvt(p);
        }
    }
}

// ---------------------------------------------- 16x16 MFMA building blocks
// v_mfma_f32_16x16x32_bf16: D[16][16] tiles, lane l holding column l & 15 and
// rows 4 (l >> 4) + r, r = 0..3; A and B operands hold 8 consecutive k per
// lane (k = 8 (l >> 4) + 0..7 of a 32-wide step).
typedef float f32x4v __attribute__((ext_vector_type(4)));

IQLH_DEV f32x4v mma16(bf16x8 a, bf16x8 b, f32x4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
IQLH_DEV bf16x8 ld8(const uint16_t* p) { return __builtin_bit_cast(bf16x8, *(const u32x4*)p); }
// Cross-lane sums and maxima of the 16x16 kernel on VALU lane permutes
// (v_permlane16/32_swap, DPP) rather than LDS-routed shuffles.
// Over the four lane groups q (rows of 16 lanes) holding one sample, the
// same value in all four: ((x_0 + x_1) + (x_2 + x_3)).
IQLH_DEV float sum_q4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
IQLH_DEV float max_q4(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// Sum over the 16 lanes of each row (rotations by 8, 4, 2, 1 within the row),
// every lane of the row ends with it.
IQLH_DEV float row_sum16(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x128, 0xF, 0xF, false);  // row_ror:8
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x124, 0xF, 0xF, false);  // row_ror:4
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x122, 0xF, 0xF, false);  // row_ror:2
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x121, 0xF, 0xF, false);  // row_ror:1
    return x;
}

// Sums over the 16 lanes of each row for sixteen values at once by recursive
// halving: afterwards lane l16 of every row holds the sum of value l16.  The
// partners l ^ 8, l ^ 4, l ^ 2, l ^ 1 are reached with the DPP row rotation
// by 8, the half-row mirror followed by the quad reversal, and two quad
// permutations; 19 DPP operations instead of 64 for sixteen row_sum16 calls.
template <int CTRL>
IQLH_DEV float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
IQLH_DEV float row_sum16_scatter(const float (&v)[16]) {
    const int l16 = threadIdx.x & 15;
    const bool b3 = (l16 & 8) != 0, b2 = (l16 & 4) != 0, b1 = (l16 & 2) != 0, b0 = (l16 & 1) != 0;
    float a[8], c[4], d[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (b3 ? v[i + 8] : v[i]) + dpp_f<0x128>(b3 ? v[i] : v[i + 8]);  // row_ror:8
#pragma unroll
    for (int i = 0; i < 4; ++i)  // row_half_mirror, then quad_perm [3,2,1,0]
        c[i] = (b2 ? a[i + 4] : a[i]) + dpp_f<0x1B>(dpp_f<0x141>(b2 ? a[i] : a[i + 4]));
#pragma unroll
    for (int i = 0; i < 2; ++i) d[i] = (b1 ? c[i + 2] : c[i]) + dpp_f<0x4E>(b1 ? c[i] : c[i + 2]);  // quad_perm [2,3,0,1]
    return (b0 ? d[1] : d[0]) + dpp_f<0xB1>(b0 ? d[0] : d[1]);  // quad_perm [1,0,3,2]
}

// ReLU on the bit pattern, one integer max: a float with the sign bit set is
// a negative int32 and becomes +0 (a NaN keeps its payload unless its sign
// bit is set, as the reference maximum propagates NaN).  The float max would
// first canonicalise its operand, a second instruction.
IQLH_DEV float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// ---- activation tiles of the 16x16 kernel: natural [sample][feature]
// layout, rows of kNatLd elements, the 16-byte unit u of row s stored at
// unit u ^ bit2(s) ^ 8 bit3(s).  A lane writes its 4 consecutive features of
// its sample as one 8-byte store (no transposed 2-byte stores), and the
// weight-gradient products read their operands with the LDS transpose load
// ds_read_b64_tr_b16: within each group of 16 lanes, lane 4i + j receives
// element j of the 8-byte rows addressed by lanes 4e + i, e = 0..3.
// The gfx950 LDS has 64 four-byte banks and serves a 16-byte read for 16
// lanes a cycle (lane octets {0, 3}, {1, 2}, {4, 7}, {5, 6} together) and an
// 8-byte read for 32 lanes; with 288-byte rows this swizzle keeps the 16-byte
// operand reads and the transpose loads conflict-free (per-pattern
// throughput measured on the device for every access of the kernel).
constexpr int kNatLd = 144;
IQLH_DEV int nat_swz(int s) { return ((s >> 2) & 1) ^ (((s >> 3) & 1) << 3); }
IQLH_DEV int nat_off(int s, int f) { return s * kNatLd + ((((f >> 3) ^ nat_swz(s)) << 3) | (f & 7)); }

// features f .. f + 3 (f % 4 == 0) of sample s, rounded to bfloat16
IQLH_DEV void put4(uint16_t* tile, int s, int f, float x0, float x1, float x2, float x3) {
    typedef Op<uint16_t> O;
    *(u32x2*)(tile + nat_off(s, f)) = u32x2{O::cvt2(x0, x1), O::cvt2(x2, x3)};
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
IQLH_DEV u32x2 ld_tr4(const uint16_t* p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
    return __builtin_bit_cast(u32x2, r);
}
// Per-lane parts of the transpose-load addresses into a natural tile: the
// operand of column tile c (features 16c + l16) and sample block u (samples
// 32u + 8q .. 32u + 8q + 7) is read by two loads at base[h][c >> 2] +
// 32u * kNatLd + 16c, h = 0, 1 -- this lane addresses sample
// 32u + 8 (lane >> 4) + ((lane >> 2) & 3) + 4h, features 16c + 4 (lane & 3);
// the swizzle folds into the bases (bit 2 of the sample is h, bit 3 is
// lane bit 4, which moves units 2c, 2c + 1 by eight units, up for c < 4 and
// down otherwise), so every load of an operand sweep takes one base register
// and an immediate offset.
struct NatLane {
    int base[2][2];  // [h][c >> 2], elements
};
IQLH_DEV NatLane nat_lane() {
    const int lane = threadIdx.x & 63, g = lane >> 4, e = (lane >> 2) & 3, i = lane & 3;
    NatLane L;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int b = (8 * g + e + 4 * h) * kNatLd + 8 * ((i >> 1) ^ h) + 4 * (i & 1);
        L.base[h][0] = b + 64 * (g & 1);
        L.base[h][1] = b - 64 * (g & 1);
    }
    return L;
}
// The two bases of column tile c, chosen with selects: an index computed at
// run time into NatLane would put the struct in scratch memory.
struct NatBase {
    int b0, b1;
};
IQLH_DEV NatBase nat_base(const NatLane& L, int c) {
    const bool hi = c >= 4;
    return NatBase{hi ? L.base[0][1] : L.base[0][0], hi ? L.base[1][1] : L.base[1][0]};
}
IQLH_DEV bf16x8 frag_nat(const uint16_t* tile, const NatBase& nb, int c, int u) {
    const int off = 32 * u * kNatLd + 16 * c;
    const u32x2 lo = ld_tr4(tile + nb.b0 + off);
    const u32x2 hi = ld_tr4(tile + nb.b1 + off);
    return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
}

// ------------------------------------------------- 16-wave 16x16 variant
// Same computation for bf16 operands and hidden 128 with sixteen wave64s per
// 128-sample workgroup (four per SIMD, so the waits of one wave overlap the
// MFMA and LDS work of three others).  Wave w owns samples 16 (w >> 1) ..
// + 15 and the feature half 64 (w & 1) .. + 63 of every layer: a layer's
// input comes from its natural tile in LDS (the batch rows, h1, dz2), so the
// two halves of a sample group exchange activations through the tiles the
// weight-gradient products read anyway.  The products themselves are split
// over the sixteen waves as 8 row tiles x 2 column halves.

// C rows of row tile rt and column tiles c0 .. c0 + NCW - 1 of
// C[i][j] = sum_s A[s][i] B[s][j] over the 128 samples of two natural tiles;
// with bias_dst, also the column sums of A (over samples) of that row tile.
template <int NCW>
IQLH_DEV void nat_gemm16_part(const uint16_t* A, const uint16_t* Bm, int rt, int c0, float* dst, int ldo,
                              int ncols, float* bias_dst) {
    const int lane = threadIdx.x & 63, l16 = lane & 15, q = lane >> 4;
    const bf16x8 one = Op<uint16_t>::ones();
    const NatLane L = nat_lane();
    // column tiles c0 .. c0 + NCW - 1 share one half of the swizzle (c0 is a
    // multiple of NCW, NCW divides 4)
    static_assert(4 % NCW == 0, "column tiles within one swizzle half");
    const NatBase na = nat_base(L, rt), nbb = nat_base(L, c0);
    f32x4v acc[NCW], accb = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCW; ++c) acc[c] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const bf16x8 fa = frag_nat(A, na, rt, u);
#pragma unroll
        for (int c = 0; c < NCW; ++c) acc[c] = mma16(fa, frag_nat(Bm, nbb, c0 + c, u), acc[c]);
        if (bias_dst) accb = mma16(fa, one, accb);
    }
    float* d0 = dst + (16 * rt + 4 * q) * ldo;
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
        const int j = 16 * (c0 + c) + l16;
        if (j < ncols) {
#pragma unroll
            for (int r = 0; r < 4; ++r) d0[r * ldo + j] = acc[c][r];
        }
    }
    if (bias_dst && l16 == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) bias_dst[16 * rt + 4 * q + r] = accb[r];
    }
}

// LDS plan: R0 = W1 then dz2, R1 = W2 then W2^T, R2 = the batch rows s (kept
// to the end), R3 = h1 then dz1; then b1, b2, w3, the V halves, the loss
// sums and the per-sample-group dw3 sums.
template <int SP, int H>
struct Fused16wCfg {
    static constexpr int BT = 128, NW = 16;
    // weight rows of 288 bytes: the 16-byte A-operand reads of 16 rows are
    // conflict-free (272-byte rows measured two-way)
    static constexpr int LDW1 = kNatLd, LDW2 = kNatLd;
    static constexpr int NAT = BT * kNatLd;
    static constexpr int R0 = (H * LDW1 > NAT) ? H * LDW1 : NAT;
    static constexpr int R1 = H * LDW2;
    static constexpr int R2 = NAT;
    static constexpr int R3 = NAT;
    static constexpr int NF = 3 * H + 2 * BT + 2 * NW + (NW / 2) * H + 4 * kMaxSources * 4;
    static constexpr size_t BYTES = (size_t)(R0 + R1 + R2 + R3) * 2 + (size_t)NF * sizeof(float);
    static_assert(BYTES <= 160 * 1024, "LDS budget");
    static_assert(SP <= kNatLd - 16 && H <= kNatLd - 16, "natural tile width");
    static_assert(R3 * 2 >= BT * kHerGoalLds * 4 + BT * 4, "HER goals staged in R3");
};

// Thread 0's clock value at a phase end of a 16-wave workgroup (the
// instantiation that records them is used only for measurement).
template <bool ON>
IQLH_DEV void phase_stamp(uint64_t* row, int k) {
    if constexpr (ON) {
        if (threadIdx.x == 0) row[k] = __builtin_amdgcn_s_memrealtime();
    }
}

template <int SP, int H, bool XVEC, bool STAMPS = false>
__global__ __launch_bounds__(1024) void iql_fused16w_kernel(FusedArgs a) {
    typedef Fused16wCfg<SP, H> C;
    constexpr int NW = 16, BT = 128, FT = H / 32, KU1 = SP / 32, KUH = H / 32, NTHR = 1024;
    static_assert(H == 128 && SP % 32 == 0 && SP <= 128, "tile shape");
    extern __shared__ __align__(16) unsigned char smem[];
    uint16_t* R0 = (uint16_t*)smem;
    uint16_t* R1 = R0 + C::R0;
    uint16_t* R2 = R1 + C::R1;
    uint16_t* R3 = R2 + C::R2;
    float* sb1 = (float*)(R3 + C::R3);
    float* sb2 = sb1 + H;
    float* sw3 = sb2 + H;
    float* svh = sw3 + H;        // [2][BT] V halves
    float* sred = svh + 2 * BT;  // [2][NW / 2] loss and dv sums of the sample groups
    float* sdw3 = sred + NW;     // [NW / 2][H] dw3 over each sample group

    const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, q = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sg = wv >> 1, fh = wv & 1, fb = 64 * fh;
    // HER tiles first (they carry the longer prologue).  Within each range,
    // runs of 8 tiles take 8 G consecutive blocks, trainer-major, so the G
    // workgroups of a tile are 8 blocks apart: a launch sends block i to XCD
    // i mod 8, and they share that XCD's L2 for the rows they both read.  The
    // tile order of the partials is unchanged.
    int g, wg;
    {
        const int G = (int)gridDim.y, L = (int)(blockIdx.y * gridDim.x + blockIdx.x);
        const int h0 = a.her_on ? a.her_row0 / BT : a.nwg, nh = a.nwg - h0;
        const bool in_her = L < G * nh;
        const int t0 = in_her ? h0 : 0, n = in_her ? nh : h0, h = in_her ? L : L - G * nh;
        const int run = h / (8 * G), r = h % (8 * G);
        const int nr = min(8, n - 8 * run);  // tiles in this run
        g = r / nr;
        wg = t0 + 8 * run + r % nr;
        g = __builtin_amdgcn_readfirstlane(g);
        wg = __builtin_amdgcn_readfirstlane(wg);
    }
    uint64_t* const stamp_row = STAMPS ? a.stamps + ((int64_t)g * a.nwg + wg) * kPhaseStamps : nullptr;
    phase_stamp<STAMPS>(stamp_row, 0);
    const int S = a.S, B = a.B;
    const POff po(S, H);
    const float* prm = a.params + (int64_t)g * a.P;
    const uint16_t* w1s = (const uint16_t*)a.w1s + (int64_t)g * H * SP;
    const uint16_t* w2s = (const uint16_t*)a.w2s + (int64_t)g * H * H;
    const uint16_t* w2ts = (const uint16_t*)a.w2ts + (int64_t)g * H * H;
    float* part = a.part + ((int64_t)g * a.nwg + wg) * a.Pp;
    const float tau = g == 0 ? a.tau0 : a.tau1;

    // ---- S0: weights, small vectors and the batch rows to LDS (all loads
    // issued before the first wait; indexes clamped, unused values masked)
    const int bl = 16 * sg + l16;
    const int b = wg * BT + bl;
    const bool valid = b < B;
    const int bc = valid ? b : B - 1;
    constexpr int W1_PER_THREAD = H * SP / (NTHR * 8);
    constexpr int W2_PER_THREAD = H * H / (NTHR * 8);
    constexpr int X_PER_THREAD = BT * SP / (NTHR * 8);
    static_assert(W1_PER_THREAD * NTHR * 8 == H * SP && W2_PER_THREAD * NTHR * 8 == H * H &&
                  X_PER_THREAD * NTHR * 8 == BT * SP, "staging split");
    const int nrow = min(BT, B - wg * BT);  // batch rows of this tile
    // a tile of HER rows (uniform): their sources are loaded first, since the
    // relabelling below waits on them -- one lead row per thread of waves 0-1,
    // and the row of each of this thread's chunks
    const bool her_wg = a.her_on && wg * BT >= a.her_row0;
    const HerArgs& h = a.her;
    const int64_t hrow0 = (int64_t)wg * BT - a.her_row0;  // HER index of tile row 0
    u32x4 w1r[W1_PER_THREAD], w2r[W2_PER_THREAD], xr[X_PER_THREAD];
    float vb1, vb2, vw3, qb, b3, qa[4];
    // weights, biases, w3, q and Q (one copy of these loads in each branch
    // below, so that each branch issues its loads in the order it waits on them)
    auto load_weights = [&]() {
#pragma unroll
        for (int k = 0; k < W1_PER_THREAD; ++k) w1r[k] = *(const u32x4*)(w1s + (tid + k * NTHR) * 8);
#pragma unroll
        for (int k = 0; k < W2_PER_THREAD; ++k) w2r[k] = *(const u32x4*)(w2s + (tid + k * NTHR) * 8);
        const int th = tid < H ? tid : 0;
        vb1 = prm[po.b1 + th];
        vb2 = prm[po.b2 + th];
        vw3 = prm[po.w3 + th];
        qb = a.fwd_only ? 0.f : a.q[bc];  // used by valid lanes only
        b3 = prm[po.b3];
#pragma unroll
        for (int k = 0; k < 4; ++k) qa[k] = a.out_pi ? a.q_all[(int64_t)bc * a.A + min(q + 4 * k, a.A - 1)] : 0.f;
    };
    auto store_weights = [&]() {
#pragma unroll
        for (int k = 0; k < W1_PER_THREAD; ++k) {
            const int idx = (tid + k * NTHR) * 8, r = idx / SP, c = idx - r * SP;
            *(u32x4*)(R0 + r * C::LDW1 + c) = w1r[k];
        }
#pragma unroll
        for (int k = 0; k < W2_PER_THREAD; ++k) {
            const int idx = (tid + k * NTHR) * 8, r = idx / H, c = idx - r * H;
            *(u32x4*)(R1 + r * C::LDW2 + c) = w2r[k];
        }
        if (tid < H) {
            sb1[tid] = vb1;
            sb2[tid] = vb2;
            sw3[tid] = vw3;
        }
    };
    if (her_wg) {
        // a tile of HER rows: the sources first, since the relabelling waits
        // on them -- one lead row per thread of waves 0-1, and the row of each
        // of this thread's chunks -- then the weights
        const int32_t hsrc32 = h.source_idx[hrow0 + min(tid, nrow - 1)];
        int32_t hsrck[X_PER_THREAD];
#pragma unroll
        for (int k = 0; k < X_PER_THREAD; ++k) {
            const int c = tid + k * NTHR, sr = c / (SP / 8);
            hsrck[k] = h.source_idx[hrow0 + min(sr, nrow - 1)];
        }
        load_weights();
        // HER relabelling of the tile's rows, the steps and arithmetic of
        // her_block ("GPU IQL + HER Porting Plan", Phase 2): the draw while the
        // sources are in flight; the lead row's episode probe, action and
        // done with the chunks' entries of s and s'; donor, goal, distance and
        // reward; the goals exchanged through LDS (R3 is free until F1); the
        // chunks with their goal entries replaced, rounded to bfloat16 for the
        // tile.  Every group builds every row of the tile; the HER outputs of
        // tile row r are written by group r * groups / 128 alone, so that the
        // groups share the output traffic.
        const int S_ = h.S, G = h.G;
        const int ngrp = (int)gridDim.y;
        auto writes_row = [&](int r) { return r * ngrp / BT == g; };
        const bool hlead = tid < nrow;
        const bool wout = writes_row(tid);  // this lead row's outputs
        const uint64_t hr = hlead ? her_draw(h, hrow0 + tid, her_step_word(h)) : 0ull;
        // the draw runs while the sources are in flight: nothing that waits on
        // them may be scheduled above this point
        __builtin_amdgcn_sched_barrier(0);
        const int64_t hsrc = hsrc32;
        bool hok = hlead && hsrc >= 0 && hsrc < h.buffer_size;
        const EpisodeProbe probe = her_probe(h, hlead ? hsrc : 0);
        const int64_t hsc = hok ? hsrc : 0;
        // action and done through pointer selects: no branch around a load
        // (the join of one would drain every load in flight)
        const bool wact = wout && h.out_actions, wdone = wout && h.out_dones;
        const int32_t hact0 = *(wact ? h.actions + hsc : h.source_idx);
        const float hdone0 = *(wdone ? h.dones + hsc : (const float*)h.source_idx);
        // the first 16 goal entries of the source's s' and of the guessed
        // donor's, in the same round of loads as the probe (rows of at least
        // 8 whole chunks: offsets past the row end re-read its start, entries
        // past the goal are never used)
        const int64_t guess = her_guess_donor(h, hsc, hr, probe);
        auto goal16 = [&](int64_t row, float (&gv)[16]) {
            const float* rp = h.next_states + row * S_;
#pragma unroll
            for (int qd = 0; qd < 4; ++qd) {
                const float4 v = *(const float4*)(rp + (4 * qd + 4 <= S_ ? 4 * qd : 0));
                gv[4 * qd] = v.x; gv[4 * qd + 1] = v.y; gv[4 * qd + 2] = v.z; gv[4 * qd + 3] = v.w;
            }
        };
        float gs[16], gd[16];
        goal16(hsc, gs);
        goal16(guess, gd);
        // the chunks' entries of s and s' (a chunk whose row this group does
        // not output reloads s instead of s'); rows are whole 8-float chunks,
        // 16-byte aligned (iql_fused_her_ok), and a chunk past the row end
        // loads the row's last chunk and is masked
        float xs[X_PER_THREAD][8], xn[X_PER_THREAD][8];
#pragma unroll
        for (int k = 0; k < X_PER_THREAD; ++k) {
            const int c = tid + k * NTHR, sr = c / (SP / 8), k0 = 8 * (c - sr * (SP / 8));
            const bool wnext = writes_row(sr) && h.out_next_states != nullptr;
            const bool use = sr < nrow && hsrck[k] >= 0 && hsrck[k] < h.buffer_size;
            const int64_t sk = use ? hsrck[k] : 0;
            const int kc = min(k0, S_ - 8);
            const float* srow = h.states + sk * S_ + kc;
            const float* nrw = (wnext ? h.next_states : h.states) + sk * S_ + kc;
            const float4 x0 = *(const float4*)srow, x1 = *(const float4*)(srow + 4);
            const float4 y0 = *(const float4*)nrw, y1 = *(const float4*)(nrw + 4);
            const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xs[k][e] = keep_if(use && k0 + e < S_, xv[e]);
                xn[k][e] = keep_if(wnext && use && k0 + e < S_, yv[e]);
            }
        }
        store_weights();  // while the relabelling loads are in flight
        float* s_goal = (float*)R3;                              // [BT][kHerGoalLds]
        int* s_hdon = (int*)(s_goal + BT * kHerGoalLds);         // [BT], -1: a zeroed row
        if (hlead) {
            const int64_t hi = hrow0 + tid;
            int64_t donor = -1;
            if (hok) hok = her_donor(h, hsrc, hr, probe, donor);
            if (hok) {
                const float* ns = h.next_states + hsrc * S_;
                const float* nd = h.next_states + donor * S_;
                if (donor != guess) goal16(donor, gd);  // an episode end off the equal-length guess
                const float dist = her_distance_loaded(ns, nd, G, gs, gd);
#pragma unroll
                for (int d = 0; d < 16; ++d)
                    if (d < G) s_goal[tid * kHerGoalLds + d] = gd[d];
                for (int d = 16; d < G && d < kHerGoalLds; ++d) s_goal[tid * kHerGoalLds + d] = nd[d];
                if (wout) {
                    h.out_rewards[hi] = dist < h.threshold ? h.reward_hit : h.reward_miss;
                    if (h.donor_out) h.donor_out[hi] = (int32_t)donor;
                    if (h.out_actions) h.out_actions[hi] = hact0;
                    if (h.out_dones) h.out_dones[hi] = hdone0;
                    if (h.out_isw) h.out_isw[hi] = 1.f;
                }
            } else {
                donor = -1;
                if (wout) {
                    h.out_rewards[hi] = 0.f;
                    if (h.donor_out) h.donor_out[hi] = -1;
                    if (h.out_actions) h.out_actions[hi] = 0;
                    if (h.out_dones) h.out_dones[hi] = 0.f;
                    if (h.out_isw) h.out_isw[hi] = 0.f;
                    set_flag(h.flags, 0x2);
                }
            }
            s_hdon[tid] = (int)donor;
        }
        lds_barrier();
#pragma unroll
        for (int k = 0; k < X_PER_THREAD; ++k) {
            const int c = tid + k * NTHR, sr = c / (SP / 8), k0 = 8 * (c - sr * (SP / 8));
            // branch-free: the row's donor and the 8 staged goal entries at
            // k0 (clamped; G <= kHerGoalLds, iql_fused_her_ok) are read
            // whatever the chunk, then selected per entry
            const int src_r = min(sr, nrow - 1);
            const bool zero = sr >= nrow || s_hdon[src_r] < 0;
            const float* gp = s_goal + src_r * kHerGoalLds + min(k0, kHerGoalLds - 8);
            const float4 g0 = *(const float4*)gp, g1 = *(const float4*)(gp + 4);
            const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
            float x[8], y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool goal = k0 + e < G;
                x[e] = zero ? 0.f : (goal ? gv[e] : xs[k][e]);
                y[e] = zero ? 0.f : (goal ? gv[e] : xn[k][e]);
            }
            xr[k] = u32x4{pack_bf2(x[0], x[1]), pack_bf2(x[2], x[3]), pack_bf2(x[4], x[5]), pack_bf2(x[6], x[7])};
            if (writes_row(sr) && sr < nrow && k0 < S_) {  // whole chunks: S is a multiple of 8
                const int64_t hi = hrow0 + sr;
                *(u32x4*)((uint16_t*)h.out_states + hi * a.ld + k0) = xr[k];
                if (h.out_next_states) {
                    float* no = h.out_next_states + hi * S_ + k0;
                    *(float4*)no = float4{y[0], y[1], y[2], y[3]};
                    *(float4*)(no + 4) = float4{y[4], y[5], y[6], y[7]};
                }
            }
        }
    } else {
        load_weights();
#pragma unroll
        for (int k = 0; k < X_PER_THREAD; ++k) {
            const int c = tid + k * NTHR, sr = c / (SP / 8), k0 = 8 * (c - sr * (SP / 8));
            const int row = wg * BT + sr;
            const bool ok = row < B;
            const uint16_t* src = (const uint16_t*)a.states + (int64_t)(ok ? row : B - 1) * a.ld;
            u32x4 x;
            if (XVEC) {
                x = *(const u32x4*)(src + k0);
            } else {
                uint16_t t8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint16_t v = src[min(k0 + e, S - 1)];
                    t8[e] = (uint16_t)keep_if(k0 + e < S, (uint32_t)v);
                }
                x = u32x4{(uint32_t)t8[0] | ((uint32_t)t8[1] << 16), (uint32_t)t8[2] | ((uint32_t)t8[3] << 16),
                          (uint32_t)t8[4] | ((uint32_t)t8[5] << 16), (uint32_t)t8[6] | ((uint32_t)t8[7] << 16)};
            }
            xr[k] = u32x4{keep_if(ok, x.x), keep_if(ok, x.y), keep_if(ok, x.z), keep_if(ok, x.w)};
        }
    }
    // the budget's pass 1 on the workgroups that hold no HER rows: quarter
    // wv / 4 (256 threads) of host workgroup hidx runs block
    // quarter * hosts + hidx with the arithmetic of norms_block
    const int nhost_wg = a.her_on ? a.her_row0 / BT : a.nwg;
    const int hosts = (int)gridDim.y * nhost_wg;
    const int nblk = (!her_wg && a.nrm.nb > 0) ? (wv >> 2) * hosts + g * nhost_wg + wg : a.nrm.nb;
    float* snrm = sdw3 + (NW / 2) * H;  // [4 quarters][kMaxSources][4 waves]
    if (nblk < a.nrm.nb) {  // uniform per wave
        float acc[kMaxSources];
        norms_thread(a.nrm.s, a.nrm.n, a.nrm.vec, nblk, a.nrm.nb, tid & 255, acc);
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j) {
            if (j < a.nrm.s.k) {
                const float w = wave_sum(acc[j]);
                if (lane == 0) snrm[((wv >> 2) * kMaxSources + j) * 4 + (wv & 3)] = w;
            }
        }
    }
    if (!her_wg) store_weights();
#pragma unroll
    for (int k = 0; k < X_PER_THREAD; ++k) {
        const int c = tid + k * NTHR, sr = c / (SP / 8), k0 = 8 * (c - sr * (SP / 8));
        *(u32x4*)(R2 + nat_off(sr, k0)) = xr[k];
    }
    lds_barrier();
    phase_stamp<STAMPS>(stamp_row, 1);
    // the quarter's budget partials: its four wave sums added in block_sum_k's order
    if (nblk < a.nrm.nb && (tid & 255) == 0) {
#pragma unroll
        for (int j = 0; j < kMaxSources; ++j) {
            if (j < a.nrm.s.k) {
                float t = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) t += snrm[((wv >> 2) * kMaxSources + j) * 4 + i];
                a.nrm.partials[(int64_t)j * a.nrm.nb + nblk] = t;
            }
        }
    }

    // ---- F1: z1^T = W1 s^T + b1 for this wave's 64 features
    f32x4v acc[FT];
#pragma unroll
    for (int t = 0; t < FT; ++t) acc[t] = *(const f32x4v*)(sb1 + fb + 16 * t + 4 * q);
#pragma unroll
    for (int u = 0; u < KU1; ++u) {
        const bf16x8 xb = ld8(R2 + nat_off(bl, 32 * u + 8 * q));
#pragma unroll
        for (int t = 0; t < FT; ++t)
            acc[t] = mma16(ld8(R0 + (fb + 16 * t + l16) * C::LDW1 + 32 * u + 8 * q), xb, acc[t]);
    }
    uint32_t mask1 = 0u;  // relu'(z1), bit 4t + r
#pragma unroll
    for (int t = 0; t < FT; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float y = relu_bits(acc[t][r]);
            acc[t][r] = y;
            mask1 |= min(__float_as_uint(y), 1u) << (4 * t + r);  // y >= +0: bit set iff y != 0
        }
        put4(R3, bl, fb + 16 * t + 4 * q, acc[t][0], acc[t][1], acc[t][2], acc[t][3]);  // h1
    }
    lds_barrier();
    phase_stamp<STAMPS>(stamp_row, 2);

    // ---- F2: z2^T = W2 h1^T + b2, V = w3 . relu(z2) + b3 over both halves
#pragma unroll
    for (int t = 0; t < FT; ++t) acc[t] = *(const f32x4v*)(sb2 + fb + 16 * t + 4 * q);
#pragma unroll
    for (int u = 0; u < KUH; ++u) {
        const bf16x8 hb = ld8(R3 + nat_off(bl, 32 * u + 8 * q));
#pragma unroll
        for (int t = 0; t < FT; ++t)
            acc[t] = mma16(ld8(R1 + (fb + 16 * t + l16) * C::LDW2 + 32 * u + 8 * q), hb, acc[t]);
    }
    f32x4v w3v[FT];
#pragma unroll
    for (int t = 0; t < FT; ++t) w3v[t] = *(const f32x4v*)(sw3 + fb + 16 * t + 4 * q);
    float vpart = 0.f;
#pragma unroll
    for (int t = 0; t < FT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) vpart = fmaf(w3v[t][r], relu_bits(acc[t][r]), vpart);
    vpart = sum_q4(vpart);
    if (q == 0) svh[fh * BT + bl] = vpart;
    lds_barrier();
    phase_stamp<STAMPS>(stamp_row, 3);
    const float v = (svh[bl] + svh[BT + bl]) + b3;
    if (a.fwd_only) {
        if (valid && fh == 0 && q == 0) write_value(a.vo, g, B, b, v);
        return;
    }
    float dv = 0.f, lterm = 0.f;
    if (valid) {
        const float diff = qb - v;
        const float w = diff >= 0.f ? tau : 1.f - tau;
        lterm = w * diff * diff;
        dv = -2.f * w * diff * a.invB;
        if (fh == 0 && q == 0 && a.out_v) a.out_v[(int64_t)g * B + b] = v;
    }
    // the two waves of a sample group split the per-sample work: one the loss
    // sums (here), the other the (heavier) policy (in the dW2 phase, whose
    // waves mostly wait on LDS and MFMA), alternating with the sample group so
    // that every SIMD runs two of each (waves go to SIMDs round-robin)
    const bool policy_wave = fh == ((sg >> 1) & 1);
    if (!policy_wave) {
        const float ls = row_sum16(lterm);
        const float ds = row_sum16(dv);
        if (lane == 0) { sred[sg] = ls; sred[NW / 2 + sg] = ds; }
    }
    // dz2 = dv w3 relu'(z2) -> R0 (W1 is dead); dw3 over this sample group
    static_assert(FT == 4, "sixteen values per lane for the dw3 sums");
    float hv[16];  // h2 dv of this lane's sample, features fb + 16 t + 4 q + r at 4 t + r
#pragma unroll
    for (int t = 0; t < FT; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float z = acc[t][r];
            hv[4 * t + r] = relu_bits(z) * dv;
            acc[t][r] = z > 0.f ? dv * w3v[t][r] : 0.f;
        }
        put4(R0, bl, fb + 16 * t + 4 * q, acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
    }
    // lane l16 ends with the sample-group sum of value l16
    sdw3[sg * H + fb + 16 * (l16 >> 2) + 4 * q + (l16 & 3)] = row_sum16_scatter(hv);
    lds_barrier();
    phase_stamp<STAMPS>(stamp_row, 4);

    // ---- W2^T to R1 (W2 is dead); loss, db3, dw3; dW2 = dz2^T h1 with db2
    {
        u32x4 w2t[W2_PER_THREAD];
#pragma unroll
        for (int k = 0; k < W2_PER_THREAD; ++k) w2t[k] = *(const u32x4*)(w2ts + (tid + k * NTHR) * 8);
        if (tid < H) {
            float s3 = 0.f;
#pragma unroll
            for (int i = 0; i < NW / 2; ++i) s3 += sdw3[i * H + tid];
            part[po.w3 + tid] = s3;
        }
        if (tid == 0) {
            float ls = 0.f, ds = 0.f;
            for (int i = 0; i < NW / 2; ++i) { ls += sred[i]; ds += sred[NW / 2 + i]; }
            a.loss_part[(int64_t)g * a.nwg + wg] = ls;
            part[po.b3] = ds;
        }
        if (policy_wave && a.out_pi) {
            // pi = softmax(beta * clamp(Q - V, -10, 10)) with the row maximum
            // subtracted ("Current State / IQL (CPU)", advantage-weighted
            // action selection); the four lanes of a sample share it
            float x[4], mx = -INFINITY;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const bool on = q + 4 * k < a.A;
                x[k] = on ? a.beta * fminf(fmaxf(qa[k] - v, -10.f), 10.f) : -INFINITY;
                mx = fmaxf(mx, x[k]);
            }
            mx = max_q4(mx);
            // the hardware exponential (about 1e-6 relative on these
            // arguments, which lie in [-20 beta, 0]) instead of the
            // full-precision expf
            float se = 0.f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[k] = q + 4 * k < a.A ? __expf(x[k] - mx) : 0.f;
                se += x[k];
            }
            se = sum_q4(se);
            if (valid) {
                float* pr = a.out_pi + ((int64_t)g * B + b) * a.A;
                const float inv = 1.f / se;  // one division, then products
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (q + 4 * k < a.A) pr[q + 4 * k] = x[k] * inv;
            }
        }
        nat_gemm16_part<H / 32>(R0, R3, sg, (H / 32) * fh, part + po.w2, H, H, fh == 0 ? part + po.b2 : nullptr);
#pragma unroll
        for (int k = 0; k < W2_PER_THREAD; ++k) {
            const int idx = (tid + k * NTHR) * 8, r = idx / H, c = idx - r * H;
            *(u32x4*)(R1 + r * C::LDW2 + c) = w2t[k];
        }
    }
    lds_barrier();
    phase_stamp<STAMPS>(stamp_row, 5);

    // ---- B1: dh1^T = W2^T dz2^T for this wave's features; dz1 -> R3 (h1 is dead)
#pragma unroll
    for (int t = 0; t < FT; ++t) acc[t] = f32x4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < KUH; ++u) {
        const bf16x8 db = ld8(R0 + nat_off(bl, 32 * u + 8 * q));
#pragma unroll
        for (int t = 0; t < FT; ++t)
            acc[t] = mma16(ld8(R1 + (fb + 16 * t + l16) * C::LDW2 + 32 * u + 8 * q), db, acc[t]);
    }
#pragma unroll
    for (int t = 0; t < FT; ++t) {
        float d[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)  // keep dh1 where relu'(z1) = 1: AND with the sign-extended mask bit
            d[r] = __int_as_float(__float_as_int(acc[t][r]) & __builtin_amdgcn_sbfe((int)mask1, 4 * t + r, 1));
        put4(R3, bl, fb + 16 * t + 4 * q, d[0], d[1], d[2], d[3]);
    }
    lds_barrier();
    phase_stamp<STAMPS>(stamp_row, 6);

    // ---- dW1 = dz1^T s with db1
    nat_gemm16_part<SP / 32>(R3, R2, sg, (SP / 32) * fh, part + po.w1, S, S, fh == 0 ? part + po.b1 : nullptr);
    phase_stamp<STAMPS>(stamp_row, 7);
}

template <int SP, int H, bool XVEC>
static hipError_t run_fused16w_x(const FusedArgs& fa, int G, hipStream_t stream, hipEvent_t ev0,
                                 hipEvent_t ev1) {
    typedef Fused16wCfg<SP, H> C;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)iql_fused16w_kernel<SP, H, XVEC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::BYTES);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void*)iql_fused16w_kernel<SP, H, XVEC, true>,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if (fa.stamps) {  // measurement: the instantiation that records phase ends
        hipLaunchKernelGGL((iql_fused16w_kernel<SP, H, XVEC, true>), dim3(fa.nwg, G), dim3(1024), C::BYTES, stream,
                           fa);
        return hipGetLastError();
    }
    if (ev0)
        hipExtLaunchKernelGGL((iql_fused16w_kernel<SP, H, XVEC>), dim3(fa.nwg, G), dim3(1024), C::BYTES, stream,
                              ev0, ev1, 0, fa);
    else
        hipLaunchKernelGGL((iql_fused16w_kernel<SP, H, XVEC>), dim3(fa.nwg, G), dim3(1024), C::BYTES, stream, fa);
    return hipGetLastError();
}

template <int SP, int H>
static hipError_t run_fused16w(const FusedArgs& fa, int G, hipStream_t stream, hipEvent_t ev0,
                               hipEvent_t ev1) {
    const bool xvec = fa.S == SP && fa.ld % 8 == 0 && ((uintptr_t)fa.states % 16) == 0;
    return xvec ? run_fused16w_x<SP, H, true>(fa, G, stream, ev0, ev1)
                : run_fused16w_x<SP, H, false>(fa, G, stream, ev0, ev1);
}

// ------------------------------------------------------------- dispatch
template <typename T, int SP, int H, int NW, bool XVEC>
static hipError_t run_fused_x(const FusedArgs& fa, int G, hipStream_t stream, hipEvent_t ev0,
                              hipEvent_t ev1) {
    typedef FusedCfg<T, SP, H, NW> C;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)iql_fused_kernel<T, SP, H, NW, XVEC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::BYTES);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if (ev0)  // events recorded by the dispatch itself: kernel time only
        hipExtLaunchKernelGGL((iql_fused_kernel<T, SP, H, NW, XVEC>), dim3(fa.nwg, G), dim3(64 * NW),
                              C::BYTES, stream, ev0, ev1, 0, fa);
    else
        hipLaunchKernelGGL((iql_fused_kernel<T, SP, H, NW, XVEC>), dim3(fa.nwg, G), dim3(64 * NW),
                           C::BYTES, stream, fa);
    return hipGetLastError();
}

template <typename T, int SP, int H, int NW>
static hipError_t run_fused(const FusedArgs& fa, int G, hipStream_t stream, hipEvent_t ev0,
                            hipEvent_t ev1) {
    const bool xvec = fa.S == SP && fa.ld % Op<T>::KPL == 0 &&
                      ((uintptr_t)fa.states % (sizeof(T) * Op<T>::KPL)) == 0;
    return xvec ? run_fused_x<T, SP, H, NW, true>(fa, G, stream, ev0, ev1)
                : run_fused_x<T, SP, H, NW, false>(fa, G, stream, ev0, ev1);
}

template <int SP, int H, bool XVEC>
static hipError_t run_fused_fs_x(const FusedArgs& fa, int G, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    typedef FusedCfg<float, SP, H, 1> C;
    const size_t bytes = fs_lds_bytes(C::BYTES_T, H);
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)iql_fused_fs_kernel<SP, H, XVEC>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    // while the tiles leave compute units idle (one workgroup each on the
    // MI355X's 256), two workgroups share each tile's backward pass
    FusedArgs f = fa;
    f.fs_split = !fa.fwd_only && 2 * fa.nwg * G <= 256;
    const int gx = f.fs_split ? 2 * fa.nwg : fa.nwg;
    if (ev0)
        hipExtLaunchKernelGGL((iql_fused_fs_kernel<SP, H, XVEC>), dim3(gx, G), dim3(256), bytes, stream, ev0, ev1, 0,
                              f);
    else
        hipLaunchKernelGGL((iql_fused_fs_kernel<SP, H, XVEC>), dim3(gx, G), dim3(256), bytes, stream, f);
    return hipGetLastError();
}

template <int SP, int H>
static hipError_t run_fused_fs(const FusedArgs& fa, int G, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
    const bool xvec = fa.S == SP;
    return xvec ? run_fused_fs_x<SP, H, true>(fa, G, stream, ev0, ev1)
                : run_fused_fs_x<SP, H, false>(fa, G, stream, ev0, ev1);
}

struct Variant {
    int dtype, SP, H, NW;
    hipError_t (*fn)(const FusedArgs&, int, hipStream_t, hipEvent_t, hipEvent_t);
};
static const Variant kVariants[] = {
    // bf16, hidden 128: eight 16-sample waves per 128-sample workgroup
    {1, 128, 128, 4, &run_fused16w<128, 128>},
    {1, 64, 128, 4, &run_fused16w<64, 128>},
    // hidden 32: one wave per 32-sample workgroup (a single 32x32 output tile
    // per weight-gradient product, so more waves would leave it to one wave
    // over four times the samples)
    {1, 32, 32, 1, &run_fused<uint16_t, 32, 32, 1>},
    {0, 32, 32, 1, &run_fused<float, 32, 32, 1>},
    // fp32, hidden 128: four waves share each 32-sample workgroup
    {0, 64, 128, 1, &run_fused_fs<64, 128>},
};

static const Variant* pick(int dtype, int S, int H) {
    const Variant* best = nullptr;
    for (const Variant& v : kVariants)
        if (v.dtype == dtype && v.H == H && S <= v.SP && (!best || v.SP < best->SP)) best = &v;
    return best;
}

bool iql_supported(int dtype, int S, int H) { return pick(dtype, S, H) != nullptr; }
int iql_tile_samples(int dtype, int S, int H) {
    const Variant* v = pick(dtype, S, H);
    return v ? 32 * v->NW : 0;
}
int iql_s_pad(int dtype, int S, int H) {
    const Variant* v = pick(dtype, S, H);
    return v ? v->SP : 0;
}
int iql_reduce_blocks(int64_t P) { return (int)((P + kRedParams - 1) / kRedParams); }

// Every fused tile kernel computes the policy from its own V for up to 16
// actions.
bool iql_fused_policy(const IqlDims& d, int A) {
    return !d.layered && A >= 1 && A <= 16 && iql_supported(d.dtype, d.S, d.H);
}

// The policy runs inside the forward/backward launch: in every fused tile
// kernel (A <= 16), or in the wide-hidden weight-gradient launch's spare
// workgroups (A = 4, 8, 16, 32 or 64, 16-byte aligned rows, at least 8 idle
// compute units).
bool iql_policy_in_launch(const IqlDims& d, int B, int A, const void* q_all, const void* out_pi) {
    return iql_fused_policy(d, A) || (d.layered && d.big && iql_big_policy_ok(d, B, A, q_all, out_pi));
}

// The shapes that run iql_fused16w_kernel (bf16, hidden 128, state <= 128).
static bool is_fused16w(const IqlDims& d) { return !d.layered && d.dtype == 1 && d.H == 128 && d.S <= 128; }
bool iql_runs_fused16w(const IqlDims& d) { return is_fused16w(d); }

// HER rows the forward/backward launch can relabel itself: the batch tail
// from a 128-row boundary, bf16, rows of whole 16-byte-aligned 8-float chunks,
// goals of at most kHerGoalLds entries.
bool iql_fused_her_ok(const IqlDims& d, const HerArgs& her, const void* states, int64_t ld, int B) {
    if (!is_fused16w(d) || her.n <= 0 || her.n > B || her.S != d.S || !her.out_bf16 || her.out_ld != ld) return false;
    if (her.S % 8 != 0 || ld % 8 != 0 || her.G > kHerGoalLds) return false;
    const uintptr_t al = (uintptr_t)her.states | (uintptr_t)her.next_states | (uintptr_t)her.out_states |
                         (uintptr_t)her.out_next_states;
    if (al & 15u) return false;
    const int row0 = B - her.n;
    return row0 % 128 == 0 && (const char*)her.out_states == (const char*)states + (int64_t)row0 * ld * 2;
}

bool iql_fused_norms_ok(const IqlDims& d, int B, int her_rows, int nb) {
    if (!is_fused16w(d) || nb <= 0) return false;
    const int hosts = d.G * (her_rows > 0 ? (B - her_rows) / 128 : (B + 127) / 128);
    return nb <= 4 * hosts;
}

hipError_t launch_iql_fwd_bwd(const IqlDims& d, const IqlBuffers& b, const float* tau,
                              const void* states, int64_t ld, const float* q, int B, float* out_v,
                              hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1,
                              const float* q_all, int A, float beta, float* out_pi, const HerArgs* her,
                              const NormsArgs* nrm, uint64_t* stamps) {
    if (d.layered) {
        if (ev0) (void)hipEventRecord(ev0, stream);
        if (out_pi && !d.big) return hipErrorInvalidValue;
        hipError_t e = d.big ? launch_iql_big_fwd_bwd(d, b, tau, states, ld, q, B, out_v, stream, q_all, A, beta,
                                                      out_pi)
                             : launch_iql_layered_fwd_bwd(d, b, tau, states, ld, q, B, out_v, stream);
        if (ev1 && e == hipSuccess) e = hipEventRecord(ev1, stream);
        return e;
    }
    const Variant* var = pick(d.dtype, d.S, d.H);
    if (!var) return hipErrorInvalidValue;
    const int BT = 32 * var->NW;
    FusedArgs fa{};  // zero: fwd_only = 0, vo unused
    fa.states = states; fa.ld = ld; fa.q = q; fa.params = b.params;
    fa.w1s = b.w1s; fa.w2s = b.w2s; fa.w2ts = b.w2ts;
    fa.part = b.part; fa.loss_part = b.loss_part; fa.out_v = out_v;
    fa.q_all = q_all; fa.out_pi = out_pi; fa.A = A; fa.beta = beta;
    fa.tau0 = tau[0]; fa.tau1 = tau[d.G > 1 ? 1 : 0]; fa.invB = 1.f / (float)B;
    fa.B = B; fa.S = d.S; fa.nwg = (B + BT - 1) / BT; fa.P = d.P; fa.Pp = d.Pp; fa.flags = b.flags;
    if (her) {
        if (!iql_fused_her_ok(d, *her, states, ld, B)) return hipErrorInvalidValue;
        fa.her_on = 1;
        fa.her_row0 = B - her->n;
        fa.her = *her;
    }
    if (nrm) {
        if (!iql_fused_norms_ok(d, B, her ? her->n : 0, nrm->nb)) return hipErrorInvalidValue;
        fa.nrm = *nrm;
    }
    if (stamps) {
        if (!is_fused16w(d)) return hipErrorInvalidValue;
        fa.stamps = stamps;
    }
    return var->fn(fa, d.G, stream, ev0, ev1);
}

hipError_t launch_iql_forward_values(const IqlDims& d, const IqlBuffers& b, const void* states, int64_t ld, int B,
                                     const ValueOut& vo, hipStream_t stream) {
    if (d.layered)
        return d.big ? launch_iql_big_forward(d, b, states, ld, B, vo, stream)
                     : launch_iql_layered_forward(d, b, states, ld, B, vo, stream);
    const Variant* var = pick(d.dtype, d.S, d.H);
    if (!var) return hipErrorInvalidValue;
    const int BT = 32 * var->NW;
    FusedArgs fa{};
    fa.states = states; fa.ld = ld; fa.params = b.params;
    fa.w1s = b.w1s; fa.w2s = b.w2s; fa.w2ts = b.w2ts;
    fa.part = b.part; fa.loss_part = b.loss_part;
    fa.invB = 1.f / (float)B;
    fa.B = B; fa.S = d.S; fa.nwg = (B + BT - 1) / BT; fa.P = d.P; fa.Pp = d.Pp; fa.flags = b.flags;
    fa.fwd_only = 1;
    fa.vo = vo;
    return var->fn(fa, d.G, stream, nullptr, nullptr);
}

// ---------------------------------------------------------- row conversion
// f32 <-> bf16 (round to nearest even) of a [rows][cols] block; one thread per
// element pair along a row.
__global__ __launch_bounds__(256) void convert_rows_kernel(const void* __restrict__ src, int src_dtype, int64_t src_ld,
                                                           void* __restrict__ dst, int dst_dtype, int64_t dst_ld,
                                                           int rows, int cols) {
    const int64_t n = (int64_t)rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t r = i / cols, c = i - r * cols;
        const float x = src_dtype == 1 ? bf2f(((const uint16_t*)src)[r * src_ld + c]) : ((const float*)src)[r * src_ld + c];
        if (dst_dtype == 1) ((uint16_t*)dst)[r * dst_ld + c] = f2bf(x);
        else ((float*)dst)[r * dst_ld + c] = x;
    }
}

hipError_t launch_convert_rows(const void* src, int src_dtype, int64_t src_ld, void* dst, int dst_dtype,
                               int64_t dst_ld, int rows, int cols, hipStream_t stream) {
    const int64_t n = (int64_t)rows * cols;
    const int64_t bn = (n + 255) / 256;
    const int blocks = (int)(bn < 2048 ? bn : 2048);
    hipLaunchKernelGGL(convert_rows_kernel, dim3(blocks), dim3(256), 0, stream, src, src_dtype, src_ld, dst, dst_dtype,
                       dst_ld, rows, cols);
    return hipGetLastError();
}

bool iql_partial_counts(const IqlDims& d, int B, int* nwg, int* nloss) {
    if (d.big) {
        const int c = iql_big_chunk(d.S, d.H, d.G, B);
        *nwg = (B + c - 1) / c;
        *nloss = iql_big_blocks(B);
        return true;
    }
    if (d.layered) {
        *nwg = (B + iql_layered_chunk() - 1) / iql_layered_chunk();
        *nloss = (B + 63) / 64;
        return true;
    }
    const Variant* var = pick(d.dtype, d.S, d.H);
    if (!var) return false;
    const int BT = 32 * var->NW;
    *nwg = *nloss = (B + BT - 1) / BT;
    return true;
}

int iql_adam_blocks(int64_t P) {
    const int64_t abn = (P + 255) / 256;
    return (int)(abn < 512 ? abn : 512);
}

hipError_t launch_iql_update(const IqlDims& d, const IqlBuffers& b, const AdamHyper& hp, int B,
                             float* out_loss, float* out_gnorm, hipStream_t stream) {
    int nwg, nloss;
    if (!iql_partial_counts(d, B, &nwg, &nloss)) return hipErrorInvalidValue;
    const int rb = iql_reduce_blocks(d.P);
    hipLaunchKernelGGL(iql_reduce_kernel, dim3(rb + 1, d.G), dim3(256), 0, stream, b.part, b.loss_part,
                       nwg, nloss, d.P, d.Pp, 1.f / (float)B, b.grad, b.sq_part, rb, b.t, b.step, b.bc,
                       hp.beta1, hp.beta2, out_loss, b.flags);
    const int ab = iql_adam_blocks(d.P);
    if (d.dtype == 1)
        hipLaunchKernelGGL(iql_adam_kernel<uint16_t>, dim3(ab, d.G), dim3(256), 0, stream, d, b, hp,
                           out_gnorm, rb);
    else
        hipLaunchKernelGGL(iql_adam_kernel<float>, dim3(ab, d.G), dim3(256), 0, stream, d, b, hp,
                           out_gnorm, rb);
    return hipGetLastError();
}

// Polyak averaging of the target copy ("GPU IQL + HER Porting Plan", section
// "Rust Integration: gpu_iql_trainer.rs", target_ema_update): target +=
// tau (params - target), every element of every group.
__global__ __launch_bounds__(256) void iql_target_ema_kernel(float* __restrict__ target,
                                                             const float* __restrict__ params, int64_t n, float tau) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        target[i] = fmaf(tau, params[i] - target[i], target[i]);
}

hipError_t launch_iql_target_ema(const IqlDims& d, const IqlBuffers& b, float tau, hipStream_t stream) {
    const int64_t n = (int64_t)d.G * d.P;
    const int64_t bn = (n + 255) / 256;
    const int blocks = (int)(bn < 1024 ? bn : 1024);
    hipLaunchKernelGGL(iql_target_ema_kernel, dim3(blocks), dim3(256), 0, stream, b.target, b.params, n, tau);
    return hipGetLastError();
}

hipError_t launch_iql_refresh_shadows(const IqlDims& d, const IqlBuffers& b, hipStream_t stream) {
    const int64_t n = (int64_t)d.H * d.S_pad + (int64_t)d.H2 * d.H;
    const int64_t bn = (n + 255) / 256;
    const int blocks = (int)(bn < 1024 ? bn : 1024);
    if (d.dtype == 1)
        hipLaunchKernelGGL(iql_shadow_kernel<uint16_t>, dim3(blocks, d.G), dim3(256), 0, stream, d, b);
    else
        hipLaunchKernelGGL(iql_shadow_kernel<float>, dim3(blocks, d.G), dim3(256), 0, stream, d, b);
    return hipGetLastError();
}

}  // namespace iqlh
