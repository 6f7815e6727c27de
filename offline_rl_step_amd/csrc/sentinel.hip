// Fused non-finite sentinel: one launch checks a list of fp32 buffers and
// raises a sticky per-slot flag for each buffer that holds a NaN or an
// infinity ("DQN Backward-Path NaN Audit -- SP1 Phase A", section "Phase E
// -- SP2 fused NaN check kernel": several per-buffer checks replaced by one
// launch over a table of buffers; a slot flag is written 1 and never
// cleared; null entries are skipped).
//
// MI355X layout: each slot is cut into 4096-element pieces, one 256-thread
// block per piece (16 elements a thread, as four 16-byte loads when the
// buffer is 16-byte aligned), so a long buffer streams at HBM rate and many
// short ones share one launch.  A value is non-finite when its exponent
// bits are all ones.
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

// All eight exponent bits set: an infinity or a NaN.
IQLH_DEV bool nonfinite_bits(float x) { return (__float_as_uint(x) | 0x807FFFFFu) == 0xFFFFFFFFu; }

__global__ __launch_bounds__(256) void nonfinite_sentinel_kernel(SentinelArgs a) {
    const int bx = blockIdx.x;
    int s = 0;
    while (s + 1 < a.nslots && a.block0[s + 1] <= bx) ++s;  // block-uniform
    const float* p = a.ptr[s];
    const int64_t n = a.n[s];
    const int64_t base = (int64_t)(bx - a.block0[s]) * kSentinelPiece;
    bool bad = false;
    if ((a.vec >> s) & 1u) {
        const float4* p4 = (const float4*)(p + base);
#pragma unroll
        for (int k = 0; k < kSentinelPiece / 1024; ++k) {
            const int64_t e = base + 4 * (threadIdx.x + 256 * k);
            if (e + 4 <= n) {
                const float4 x = p4[threadIdx.x + 256 * k];
                bad |= nonfinite_bits(x.x) || nonfinite_bits(x.y) || nonfinite_bits(x.z) || nonfinite_bits(x.w);
            } else {
                for (int64_t j = e; j < n && j < e + 4; ++j) bad |= nonfinite_bits(p[j]);
            }
        }
    } else {
#pragma unroll 4
        for (int k = 0; k < kSentinelPiece / 256; ++k) {
            const int64_t e = base + threadIdx.x + 256 * k;
            if (e < n) bad |= nonfinite_bits(p[e]);
        }
    }
    if (__syncthreads_or(bad) && threadIdx.x == 0) a.flags[s] = 1;
}

hipError_t launch_nonfinite_sentinel(const SentinelArgs& a, int blocks, hipStream_t stream) {
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(nonfinite_sentinel_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace iqlh
