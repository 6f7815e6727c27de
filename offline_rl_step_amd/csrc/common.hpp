// Device helpers shared by the IQL + HER kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define IQLH_DEV __device__ __forceinline__

namespace iqlh {

constexpr int kWave = 64;

// ---------------------------------------------------------------- bfloat16
// Round-to-nearest-even float -> bfloat16 bits, NaN becoming 0x7FC0: the
// hardware conversion (v_cvt_pk_bf16_f32, two values per instruction) with
// NaN set explicitly.
typedef float f32x2_cv __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cv __attribute__((ext_vector_type(2)));
IQLH_DEV uint32_t pack_bf2(float lo, float hi) {
    uint32_t p = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_cv{lo, hi}, bf16x2_cv));
    if (lo != lo) p = (p & 0xFFFF0000u) | 0x7FC0u;
    if (hi != hi) p = (p & 0x0000FFFFu) | 0x7FC00000u;
    return p;
}
IQLH_DEV uint16_t f2bf(float x) { return (uint16_t)(pack_bf2(x, 0.f) & 0xFFFFu); }
IQLH_DEV float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// ---------------------------------------------------------------- Philox
// Philox4x64-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds of two 64x64->128 multiplies with the
// key bumped by two Weyl constants between rounds.
struct u64x4 { uint64_t x, y, z, w; };

// Full 64 x 64 -> 128-bit product, schoolbook on 32-bit halves: four
// 32 x 32 -> 64 multiply-adds (v_mad_u64_u32) with the partial products
// shared between the high and the low word.
IQLH_DEV void mulhilo64(uint64_t a, uint64_t b, uint64_t& hi, uint64_t& lo) {
    const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
    const uint32_t b0 = (uint32_t)b, b1 = (uint32_t)(b >> 32);
    const uint64_t p00 = (uint64_t)a0 * b0;
    const uint64_t t1 = (uint64_t)a0 * b1 + (p00 >> 32);    // < 2^64
    const uint64_t t2 = (uint64_t)a1 * b0 + (uint32_t)t1;   // < 2^64
    hi = (uint64_t)a1 * b1 + (t1 >> 32) + (t2 >> 32);
    lo = (t2 << 32) | (uint32_t)p00;
}

IQLH_DEV u64x4 philox4x64_10(u64x4 c, uint64_t k0, uint64_t k1) {
    const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += W0; k1 += W1; }
        uint64_t hi0, lo0, hi1, lo1;
        mulhilo64(M0, c.x, hi0, lo0);
        mulhilo64(M1, c.z, hi1, lo1);
        c = u64x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
    }
    return c;
}

// lo + floor(r * span / 2^64); exact, span >= 1.
IQLH_DEV int64_t uniform_index(uint64_t r, int64_t lo, uint64_t span) {
    return lo + (int64_t)__umul64hi(r, span);
}

// ---------------------------------------------------------------- reductions
IQLH_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}
IQLH_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

// Block sum in a fixed order (deterministic).  `red` holds >= NT/64 floats.
template <int NT>
IQLH_DEV float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NT / kWave; ++i) s += red[i];
    return s;
}

// Workgroup barrier for data exchanged through LDS only: waits for this
// wave's LDS operations (lgkmcnt 0), not for its global stores, which
// __syncthreads' release fence would drain first (about a microsecond after
// a burst of stores).  For kernels whose waves never read each other's global
// writes.  The empty asm statements keep the compiler from moving memory
// accesses across it.
IQLH_DEV void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// c ? x : 0 by bit masking.  The loaded x is consumed on every path, which
// keeps the compiler from sinking its load into a lane-dependent branch (a
// branch whose end then waits for every load the wave has in flight).
IQLH_DEV float keep_if(bool c, float x) { return __uint_as_float(__float_as_uint(x) & (c ? 0xFFFFFFFFu : 0u)); }
IQLH_DEV uint32_t keep_if(bool c, uint32_t x) { return x & (c ? 0xFFFFFFFFu : 0u); }
IQLH_DEV uint16_t keep_if(bool c, uint16_t x) { return (uint16_t)(x & (c ? 0xFFFFu : 0u)); }

IQLH_DEV void set_flag(int32_t* flags, int32_t bit) {
    if (flags) atomicOr(flags, bit);
}

}  // namespace iqlh
