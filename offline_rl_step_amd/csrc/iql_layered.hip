// IQL value-network step, layered form for shapes the fused tile kernel
// cannot hold on chip (hidden widths beyond 128, e.g. 512; state dims
// beyond 64 in fp32).  Same arithmetic as the fused kernel ("GPU IQL + HER
// Porting Plan", section "Current State / IQL (CPU)"), with activations
// staged in HBM:
//
//   L1  h1 = relu(s W1^T + b1)                    GEMM, epilogue -> H1 [B][H]
//   L2  z2 = h1 W2^T + b2                         GEMM, epilogue -> Z2 [B][H] f32
//   R   v = relu(z2) . w3 + b3, expectile, dv,    one wave per row
//       dz2 = dv w3 relu'(z2), p2 = relu(z2) dv   -> DZ2, P2 [B][H], loss terms
//   L3  dz1 = (dz2 W2) * relu'(z1)                GEMM, epilogue -> DZ1 [B][H]
//   W   dW2 = dz2^T h1, dW1 = dz1^T s over one    split-K GEMM, one chunk of
//       chunk of rows, db1, db2, dw3, db3          samples per partial row
//
// then the fixed-order partial reduction and Adam shared with the fused path.
//
// The GEMM is one MFMA tile routine: C[m][n] = sum_k A[m][k] B[n][k], 128x128
// output tiles, four waves of 64x64 (2x2 MFMA 32x32 tiles), K staged through
// LDS 32 at a time.  Each operand is read either K-contiguous (16-byte loads)
// or from [k][row] storage with the transpose done while staging to LDS, so
// the weight-gradient products read dz2, h1, dz1 and s in place: no
// transposed copy ever goes to HBM.  Row sums (bias gradients, dw3) come from
// an extra MFMA against an all-ones operand.
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float lf32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 lbf16x2 __attribute__((ext_vector_type(2)));

template <typename T> struct LOp;
template <> struct LOp<uint16_t> {
    static constexpr int KS = 16, KPL = 8, EPV = 8;  // elements per 16-byte vector
    typedef bf16x8 frag;
    static IQLH_DEV f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static IQLH_DEV frag load(const uint16_t* p) { return __builtin_bit_cast(frag, *(const u32x4*)p); }
    static IQLH_DEV frag ones() {
        return __builtin_bit_cast(frag, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    }
    static IQLH_DEV uint16_t cvt(float x) {
        return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(lf32x2{x, 0.f}, lbf16x2)) &
                          0xFFFFu);
    }
    static IQLH_DEV float tof(uint16_t x) { return __uint_as_float(((uint32_t)x) << 16); }
};
template <> struct LOp<float> {
    static constexpr int KS = 2, KPL = 1, EPV = 4;
    typedef float frag;
    static IQLH_DEV f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static IQLH_DEV frag load(const float* p) { return *p; }
    static IQLH_DEV frag ones() { return 1.f; }
    static IQLH_DEV float cvt(float x) { return x; }
    static IQLH_DEV float tof(float x) { return x; }
};

constexpr int kTM = 128, kTN = 128, kTK = 32, kTPAD = 8;  // tile, K stage, LDS row padding
constexpr int kLdsRow = kTK + kTPAD;

// One operand of a tile GEMM: element (row, k) of a logical [rows][K] matrix.
struct Operand {
    const void* p;
    int64_t ld;     // storage row stride (elements)
    int rows, K;    // logical extent; reads outside are zero
    int trans;      // 0: storage [row][k]; 1: storage [k][row]
    int64_t roff;   // row offset added to the logical row (chunk origin)
    int64_t koff;   // k offset added to the logical k
};

// Stages rows [r0, r0+128) x k [k0, k0+32) of an operand into LDS [128][kLdsRow].
template <typename T>
IQLH_DEV void stage(const Operand& o, int r0, int k0, T* lds) {
    typedef LOp<T> O;
    const T* base = (const T*)o.p;
    const int tid = threadIdx.x;
    if (!o.trans) {
        // 128 rows x 32 k = 128 * (32 / EPV) vectors
        constexpr int VPR = kTK / O::EPV;
        for (int v = tid; v < kTM * VPR; v += 256) {
            const int r = v / VPR, kk = (v - r * VPR) * O::EPV;
            const int gr = r0 + r, gk = k0 + kk;
            T tmp[O::EPV];
            if (gr < o.rows && gk + O::EPV <= o.K) {
                const T* src = base + (o.roff + gr) * o.ld + o.koff + gk;
                if ((((uintptr_t)src) & 15u) == 0) {
                    *(u32x4*)tmp = *(const u32x4*)src;
                } else {
#pragma unroll
                    for (int e = 0; e < O::EPV; ++e) tmp[e] = src[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < O::EPV; ++e)
                    tmp[e] = (gr < o.rows && gk + e < o.K) ? base[(o.roff + gr) * o.ld + o.koff + gk + e] : (T)0;
            }
            *(u32x4*)(lds + r * kLdsRow + kk) = *(const u32x4*)tmp;
        }
    } else {
        // storage [k][row]: 32 k-rows x 128 contiguous rows; transpose into LDS
        constexpr int VPR = kTM / O::EPV;
        for (int v = tid; v < kTK * VPR; v += 256) {
            const int kk = v / VPR, r = (v - kk * VPR) * O::EPV;
            const int gk = k0 + kk, gr = r0 + r;
            T tmp[O::EPV];
#pragma unroll
            for (int e = 0; e < O::EPV; ++e)
                tmp[e] = (gk < o.K && gr + e < o.rows) ? base[(o.koff + gk) * o.ld + o.roff + gr + e] : (T)0;
#pragma unroll
            for (int e = 0; e < O::EPV; ++e) lds[(r + e) * kLdsRow + kk] = tmp[e];
        }
    }
}

// acc[2][2] += A_tile(rows 64*wm..) x B_tile(rows 64*wn..)^T over K; optional
// ones-products for the row sums of A (accb[2]).
template <typename T, bool ROWSUM>
IQLH_DEV void tile_gemm(const Operand& A, const Operand& Bo, int m0, int n0, int K, T* lA, T* lB,
                        f32x16 (&acc)[2][2], f32x16 (&accb)[2]) {
    typedef LOp<T> O;
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wv >> 1, wn = wv & 1;
    const typename O::frag one = O::ones();
    for (int k0 = 0; k0 < K; k0 += kTK) {
        __syncthreads();
        stage<T>(A, m0, k0, lA);
        stage<T>(Bo, n0, k0, lB);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kTK / O::KS; ++u) {
            const int kk = O::KS * u + O::KPL * h;
            typename O::frag a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = O::load(lA + (64 * wm + 32 * i + l32) * kLdsRow + kk);
#pragma unroll
            for (int j = 0; j < 2; ++j) b[j] = O::load(lB + (64 * wn + 32 * j + l32) * kLdsRow + kk);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) acc[i][j] = O::mma(a[i], b[j], acc[i][j]);
            if (ROWSUM && wn == 0) {
#pragma unroll
                for (int i = 0; i < 2; ++i) accb[i] = O::mma(a[i], one, accb[i]);
            }
        }
    }
}

// ------------------------------------------------------------ forward GEMMs
struct FwdArgs {
    Operand A, B;          // A = activations [Bsz][K], B = weight shadow [N][K]
    int M, N, K;
    const float* bias;     // [N] (group slice)
    void* out;             // [M][N] operand-typed (L1) or f32 (L2)
    const void* mask;      // L3: H1 [M][N] operand-typed, relu'(z1) = (h1 > 0)
    int mode;              // 0: L1 relu -> T ; 1: L2 bias -> f32 ; 2: L3 mask -> T
    int64_t gstride_w;     // per-group strides (elements) for weights / activation inputs / outputs
    int64_t gstride_in;
    int64_t gstride_out;
    int64_t gstride_bias;
};

template <typename T>
__global__ __launch_bounds__(256) void layer_gemm_kernel(FwdArgs a) {
    __shared__ __align__(16) T lA[kTM * kLdsRow];
    __shared__ __align__(16) T lB[kTN * kLdsRow];
    const int g = blockIdx.z;
    Operand A = a.A, Bo = a.B;
    Bo.p = (const T*)Bo.p + g * a.gstride_w;
    if (a.mode != 0) A.p = (const T*)A.p + g * a.gstride_in;  // per-group activations
    const int m0 = blockIdx.x * kTM, n0 = blockIdx.y * kTN;
    f32x16 acc[2][2], accb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) { accb[i] = f32x16{}; for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{}; }
    tile_gemm<T, false>(A, Bo, m0, n0, a.K, lA, lB, acc, accb);
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
    const int wv = threadIdx.x >> 6, wm = wv >> 1, wn = wv & 1;
    const float* bias = a.bias ? a.bias + g * a.gstride_bias : nullptr;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 64 * wn + 32 * j + l32;
            if (n >= a.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m >= a.M) continue;
                const int64_t o = g * a.gstride_out + (int64_t)m * a.N + n;
                float z = acc[i][j][r];
                if (a.mode == 0) {
                    z += bias[n];
                    ((T*)a.out)[o] = LOp<T>::cvt(z > 0.f ? z : 0.f);
                } else if (a.mode == 1) {
                    ((float*)a.out)[o] = z + bias[n];
                } else {
                    const float h1 = LOp<T>::tof(((const T*)a.mask)[o]);
                    ((T*)a.out)[o] = LOp<T>::cvt(h1 > 0.f ? z : 0.f);
                }
            }
        }
}

// ------------------------------------------------------------ per-row pass
// v, expectile loss term, dv; dz2 = dv w3 relu'(z2) and p2 = relu(z2) dv.
struct RowArgs {
    const float* z2;      // [G][B][H]
    const float* q;       // [B]
    const float* params;  // [G][P]
    void* dz2;            // [G][B][H]
    void* p2;             // [G][B][H]
    float* dv_out;        // [G][B]
    float* out_v;         // [G][B] or null
    float* loss_part;     // [G][nblk]
    float tau0, tau1, invB;
    int B, H, nblk;
    int64_t P, w3off;
    int fwd_only;  // 1: V (and the bootstrap target) only
    ValueOut vo;
};

constexpr int kRowsPerBlock = 64;  // 4 waves x 16 rows

template <typename T>
__global__ __launch_bounds__(256) void iql_rows_kernel(RowArgs a) {
    __shared__ float wl[4];
    const int g = blockIdx.y, lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const float* w3 = a.params + g * a.P + a.w3off;
    const float b3 = w3[a.H];
    const float tau = g == 0 ? a.tau0 : a.tau1;
    float lsum = 0.f;
    for (int rr = 0; rr < kRowsPerBlock / 4; ++rr) {
        const int b = blockIdx.x * kRowsPerBlock + wv * (kRowsPerBlock / 4) + rr;
        if (b >= a.B) break;  // wave-uniform
        const float* z = a.z2 + ((int64_t)g * a.B + b) * a.H;
        float s = 0.f;
        for (int hh = lane; hh < a.H; hh += 64) {
            const float zz = z[hh];
            s = fmaf(w3[hh], zz > 0.f ? zz : 0.f, s);
        }
        const float v = wave_sum(s) + b3;
        if (a.fwd_only) {
            if (lane == 0) write_value(a.vo, g, a.B, b, v);
            continue;
        }
        const float diff = a.q[b] - v;
        const float w = diff >= 0.f ? tau : 1.f - tau;
        const float dv = -2.f * w * diff * a.invB;
        if (lane == 0) {
            lsum += w * diff * diff;
            a.dv_out[(int64_t)g * a.B + b] = dv;
            if (a.out_v) a.out_v[(int64_t)g * a.B + b] = v;
        }
        T* dz = (T*)a.dz2 + ((int64_t)g * a.B + b) * a.H;
        T* pp = (T*)a.p2 + ((int64_t)g * a.B + b) * a.H;
        for (int hh = lane; hh < a.H; hh += 64) {
            const float zz = z[hh];
            dz[hh] = LOp<T>::cvt(zz > 0.f ? dv * w3[hh] : 0.f);
            pp[hh] = LOp<T>::cvt(zz > 0.f ? zz * dv : 0.f);
        }
    }
    if (lane == 0) wl[wv] = lsum;
    __syncthreads();
    if (threadIdx.x == 0 && !a.fwd_only) a.loss_part[(int64_t)g * a.nblk + blockIdx.x] = wl[0] + wl[1] + wl[2] + wl[3];
}

// ---------------------------------------------- split-K weight gradients
// Job kinds per (chunk, tile): 0 = dW2 (+db2), 1 = dW1 (+db1), 2 = dw3, 3 = db3.
struct WgradArgs {
    const void* dz2;   // [G][B][H]
    const void* h1;    // [G][B][H]
    const void* dz1;   // [G][B][H]
    const void* p2;    // [G][B][H]
    const void* x;     // [B][ld]
    const float* dv;   // [G][B]
    int64_t ld;
    int B, S, H, H2, chunk, nchunk;  // H, H2: first and second hidden widths
    int nt_h, nt_h2, nt_s;  // 128-tiles along H, H2 and S
    float* part;       // [G][nchunk][Pp]
    int64_t Pp;
    int64_t off_w1, off_b1, off_w2, off_b2, off_w3, off_b3;
};

template <typename T>
__global__ __launch_bounds__(256) void iql_wgrad_kernel(WgradArgs a) {
    __shared__ __align__(16) T lA[kTM * kLdsRow];
    __shared__ __align__(16) T lB[kTN * kLdsRow];
    __shared__ float red[4];
    const int g = blockIdx.z / a.nchunk, c = blockIdx.z - g * a.nchunk;
    const int b0 = c * a.chunk;
    const int K = min(a.chunk, a.B - b0);
    const int64_t gs = (int64_t)g * a.B * a.H, gs2 = (int64_t)g * a.B * a.H2;
    float* part = a.part + ((int64_t)g * a.nchunk + c) * a.Pp;
    const int n_w2 = a.nt_h2 * a.nt_h, n_w1 = a.nt_h * a.nt_s;
    int job = blockIdx.x;
    const int lane = threadIdx.x & 63, l32 = lane & 31, h = lane >> 5;
    const int wv = threadIdx.x >> 6, wm = wv >> 1, wn = wv & 1;
    if (job == n_w2 + n_w1 + a.nt_h2) {
        // db3 = sum of dv over the chunk
        float s = 0.f;
        for (int i = threadIdx.x; i < K; i += 256) s += a.dv[(int64_t)g * a.B + b0 + i];
        s = block_sum<256>(s, red);
        if (threadIdx.x == 0) part[a.off_b3] = s;
        return;
    }
    // operands: logical [rows = feature][K = sample] read from [sample][feature]
    Operand A, Bo;
    int M, N;
    float *dst, *bias_dst;
    int ldo;
    if (job < n_w2) {  // dW2 [H2][H] = dz2^T h1
        A = Operand{(const T*)a.dz2 + gs2, a.H2, a.H2, K, 1, 0, b0};
        Bo = Operand{(const T*)a.h1 + gs, a.H, a.H, K, 1, 0, b0};
        M = a.H2; N = a.H; dst = part + a.off_w2; bias_dst = part + a.off_b2; ldo = a.H;
    } else if (job < n_w2 + n_w1) {
        job -= n_w2;
        A = Operand{(const T*)a.dz1 + gs, a.H, a.H, K, 1, 0, b0};
        Bo = Operand{a.x, a.ld, a.S, K, 1, 0, b0};
        M = a.H; N = a.S; dst = part + a.off_w1; bias_dst = part + a.off_b1; ldo = a.S;
    } else {
        job -= n_w2 + n_w1;  // dw3: row sums of p2^T, one 128-row tile
        A = Operand{(const T*)a.p2 + gs2, a.H2, a.H2, K, 1, 0, b0};
        Bo = A;
        M = a.H2; N = 0; dst = nullptr; bias_dst = part + a.off_w3; ldo = 0;
    }
    const int ntn = N > 0 ? (N + kTN - 1) / kTN : 1;
    const int m0 = (job / ntn) * kTM, n0 = (job % ntn) * kTN;
    f32x16 acc[2][2], accb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) { accb[i] = f32x16{}; for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{}; }
    tile_gemm<T, true>(A, Bo, m0, n0, K, lA, lB, acc, accb);
    if (dst) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int n = n0 + 64 * wn + 32 * j + l32;
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                    if (m < M) dst[(int64_t)m * ldo + n] = acc[i][j][r];
                }
            }
    }
    // row sums over the chunk: only the first column tile writes them
    if (n0 == 0 && wn == 0 && l32 == 0) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + 64 * wm + 32 * i + 8 * (r >> 2) + 4 * h + (r & 3);
                if (m < M) bias_dst[m] = accb[i][r];
            }
    }
}

// ------------------------------------------------------------ dispatch
constexpr int kChunk = 2048;

bool iql_layered_supported(int dtype, int S, int H) {
    (void)dtype;
    return S >= 1 && H >= 1 && S <= 4096 && H <= 4096;
}
int iql_layered_chunk() { return kChunk; }

static hipError_t layered_launch(const IqlDims& d, const IqlBuffers& b, const float* tau, const void* states,
                                 int64_t ld, const float* q, int B, float* out_v, const ValueOut* vo,
                                 hipStream_t stream);

hipError_t launch_iql_layered_fwd_bwd(const IqlDims& d, const IqlBuffers& b, const float* tau,
                                      const void* states, int64_t ld, const float* q, int B,
                                      float* out_v, hipStream_t stream) {
    return layered_launch(d, b, tau, states, ld, q, B, out_v, nullptr, stream);
}

hipError_t launch_iql_layered_forward(const IqlDims& d, const IqlBuffers& b, const void* states, int64_t ld,
                                      int B, const ValueOut& vo, hipStream_t stream) {
    const float tau[2] = {0.f, 0.f};
    return layered_launch(d, b, tau, states, ld, nullptr, B, nullptr, &vo, stream);
}

static hipError_t layered_launch(const IqlDims& d, const IqlBuffers& b, const float* tau, const void* states,
                                 int64_t ld, const float* q, int B, float* out_v, const ValueOut* vo,
                                 hipStream_t stream) {
    // H: first hidden width (h1, dz1), H2: second (z2, dz2, p2)
    const int G = d.G, S = d.S, H = d.H, H2 = d.H2;
    const int nchunk = (B + kChunk - 1) / kChunk;
    const int nblk = (B + kRowsPerBlock - 1) / kRowsPerBlock;
    const int64_t gH = (int64_t)B * H, gH2 = (int64_t)B * H2;  // per-group activation strides of this call
    const int64_t ob2 = (int64_t)H * S + H + (int64_t)H2 * H;   // flat offset of b2
    // L1: h1 = relu(s W1^T + b1)
    FwdArgs f1{};
    f1.A = Operand{states, ld, B, S, 0, 0, 0};
    f1.B = Operand{b.w1s, d.S_pad, H, S, 0, 0, 0};
    f1.M = B; f1.N = H; f1.K = S;
    f1.bias = b.params + (int64_t)H * S; f1.gstride_bias = d.P;
    f1.out = b.act_h1; f1.mode = 0;
    f1.gstride_w = (int64_t)H * d.S_pad; f1.gstride_out = gH;
    const dim3 gridf((B + kTM - 1) / kTM, (H + kTN - 1) / kTN, G);
    if (d.dtype == 1) hipLaunchKernelGGL(layer_gemm_kernel<uint16_t>, gridf, dim3(256), 0, stream, f1);
    else hipLaunchKernelGGL(layer_gemm_kernel<float>, gridf, dim3(256), 0, stream, f1);
    // L2: z2 = h1 W2^T + b2 (f32), W2 [H2][H]
    FwdArgs f2{};
    f2.A = Operand{b.act_h1, H, B, H, 0, 0, 0};
    f2.B = Operand{b.w2s, H, H2, H, 0, 0, 0};
    f2.M = B; f2.N = H2; f2.K = H;
    f2.bias = b.params + ob2; f2.gstride_bias = d.P;
    f2.out = b.act_z2; f2.mode = 1;
    f2.gstride_w = (int64_t)H2 * H; f2.gstride_in = gH; f2.gstride_out = gH2;
    const dim3 grid2((B + kTM - 1) / kTM, (H2 + kTN - 1) / kTN, G);
    if (d.dtype == 1) hipLaunchKernelGGL(layer_gemm_kernel<uint16_t>, grid2, dim3(256), 0, stream, f2);
    else hipLaunchKernelGGL(layer_gemm_kernel<float>, grid2, dim3(256), 0, stream, f2);
    // R: v, expectile, dv, dz2, p2
    RowArgs ra{};
    ra.z2 = b.act_z2; ra.q = q; ra.params = b.params; ra.dz2 = b.act_dz2; ra.p2 = b.act_p2;
    ra.dv_out = b.act_dv; ra.out_v = out_v; ra.loss_part = b.loss_part;
    ra.tau0 = tau[0]; ra.tau1 = tau[G > 1 ? 1 : 0]; ra.invB = 1.f / (float)B;
    ra.B = B; ra.H = H2; ra.nblk = nblk; ra.P = d.P;
    ra.w3off = ob2 + H2;
    if (vo) {
        ra.fwd_only = 1;
        ra.vo = *vo;
    }
    if (d.dtype == 1) hipLaunchKernelGGL(iql_rows_kernel<uint16_t>, dim3(nblk, G), dim3(256), 0, stream, ra);
    else hipLaunchKernelGGL(iql_rows_kernel<float>, dim3(nblk, G), dim3(256), 0, stream, ra);
    if (vo) return hipGetLastError();
    // L3: dz1 = (dz2 W2) * relu'(z1)   (B operand: W2^T shadow [H][H2], rows h1, k = h2)
    FwdArgs f3{};
    f3.A = Operand{b.act_dz2, H2, B, H2, 0, 0, 0};
    f3.B = Operand{b.w2ts, H2, H, H2, 0, 0, 0};
    f3.M = B; f3.N = H; f3.K = H2;
    f3.bias = nullptr; f3.out = b.act_dz1; f3.mask = b.act_h1; f3.mode = 2;
    f3.gstride_w = (int64_t)H2 * H; f3.gstride_in = gH2; f3.gstride_out = gH;
    if (d.dtype == 1) hipLaunchKernelGGL(layer_gemm_kernel<uint16_t>, gridf, dim3(256), 0, stream, f3);
    else hipLaunchKernelGGL(layer_gemm_kernel<float>, gridf, dim3(256), 0, stream, f3);
    // W: split-K weight gradients into the partial rows of each chunk
    WgradArgs wa{};
    wa.dz2 = b.act_dz2; wa.h1 = b.act_h1; wa.dz1 = b.act_dz1; wa.p2 = b.act_p2; wa.x = states;
    wa.dv = b.act_dv; wa.ld = ld; wa.B = B; wa.S = S; wa.H = H; wa.H2 = H2; wa.chunk = kChunk; wa.nchunk = nchunk;
    wa.nt_h = (H + kTM - 1) / kTM; wa.nt_h2 = (H2 + kTM - 1) / kTM; wa.nt_s = (S + kTN - 1) / kTN;
    wa.part = b.part; wa.Pp = d.Pp;
    wa.off_w1 = 0; wa.off_b1 = (int64_t)H * S; wa.off_w2 = wa.off_b1 + H;
    wa.off_b2 = ob2; wa.off_w3 = ob2 + H2; wa.off_b3 = wa.off_w3 + H2;
    const int jobs = wa.nt_h2 * wa.nt_h + wa.nt_h * wa.nt_s + wa.nt_h2 + 1;
    const dim3 gridw(jobs, 1, nchunk * G);
    if (d.dtype == 1) hipLaunchKernelGGL(iql_wgrad_kernel<uint16_t>, gridw, dim3(256), 0, stream, wa);
    else hipLaunchKernelGGL(iql_wgrad_kernel<float>, gridw, dim3(256), 0, stream, wa);
    return hipGetLastError();
}

}  // namespace iqlh
