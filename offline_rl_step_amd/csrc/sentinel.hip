// Fused non-finite sentinel: one launch checks a list of fp32 buffers and
// raises a sticky per-slot flag for each buffer that holds a NaN or an
// infinity ("DQN Backward-Path NaN Audit -- SP1 Phase A", section "Phase E
// -- SP2 fused NaN check kernel": several per-buffer checks replaced by one
// launch over a table of buffers; a slot flag is written 1 and never
// cleared; null entries are skipped).
//
// MI355X layout: each slot is cut into 8192-element pieces, one 256-thread
// block per piece (32 elements a thread, as eight 16-byte loads in flight
// together when the buffer is 16-byte aligned), so a long buffer streams at
// HBM rate and many short ones share one launch.  A value is non-finite when its exponent
// bits are all ones.
#include "common.hpp"
#include "launch.hpp"

namespace iqlh {

// All eight exponent bits set: an infinity or a NaN (1u, else 0u).
IQLH_DEV uint32_t nonfinite_word(float x) { return (__float_as_uint(x) | 0x807FFFFFu) == 0xFFFFFFFFu ? 1u : 0u; }

__global__ __launch_bounds__(256) void nonfinite_sentinel_kernel(SentinelArgs a) {
    const int bx = blockIdx.x;
    int s = 0;
    while (s + 1 < a.nslots && a.block0[s + 1] <= bx) ++s;  // block-uniform
    const float* p = a.ptr[s];
    const int64_t n = a.n[s];
    const int64_t base = (int64_t)(bx - a.block0[s]) * kSentinelPiece;
    uint32_t bad = 0u;
    if (((a.vec >> s) & 1u) && base + kSentinelPiece <= n) {
        // a whole piece of an aligned slot (block-uniform): every quad's load
        // issued before any is tested, no lane-dependent branch among them
        constexpr int Q = kSentinelPiece / 1024;
        const float4* p4 = (const float4*)(p + base);
        float4 x[Q];
#pragma unroll
        for (int k = 0; k < Q; ++k) x[k] = p4[threadIdx.x + 256 * k];
#pragma unroll
        for (int k = 0; k < Q; ++k)
            bad |= nonfinite_word(x[k].x) | nonfinite_word(x[k].y) | nonfinite_word(x[k].z) | nonfinite_word(x[k].w);
    } else {
        // the last piece of a slot, or an unaligned slot: element by element,
        // loads at clamped indices (n >= 1) and the results masked, so that
        // no branch separates one load from the next
#pragma unroll 8
        for (int k = 0; k < kSentinelPiece / 256; ++k) {
            const int64_t e = base + threadIdx.x + 256 * k;
            bad |= keep_if(e < n, nonfinite_word(p[e < n ? e : n - 1]));
        }
    }
    if (__syncthreads_or((int)bad) && threadIdx.x == 0) a.flags[s] = 1;
}

hipError_t launch_nonfinite_sentinel(const SentinelArgs& a, int blocks, hipStream_t stream) {
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(nonfinite_sentinel_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace iqlh
