// HER goal relabelling with sparse-reward recomputation, gfx950.
//
// Follows "GPU IQL + HER Porting Plan": section "CUDA Kernel:
// her_relabel_kernel.cu" (copy s and s' of the source, overwrite the goal
// entries of both with the donor's next-state goal, copy action and done,
// reward from the Euclidean goal distance against the threshold) and section
// "Donor Index Generation" (final / future / random donors).
//
// MI355X layout: a 256-thread workgroup owns 32 relabelled rows, arranged so
// the chain of dependent memory round trips is three (source index -> episode
// end / source row -> donor goal) instead of one per step of the pages' kernel:
//   Phase A, every thread: reads its rows' source indices and issues the
//     16-byte loads of its quads of s and s' (these do not depend on the
//     donor).
//   Phase 1, one thread per row, concurrently: Philox draw, episode lookup,
//     donor, both goals loaded together, the binary32 reward, action and
//     done.  The lookup probes the episode at the interpolation guess
//     src * E / size (two independent loads: one round trip, always, for
//     equal-length episodes) and falls back to a bounded binary search; one
//     lane per row keeps the 64-bit Philox rounds off the other lanes.
//   Phase B, after one barrier: goal entries patched from LDS and the rows
//     written straight into the caller's merged batch (bf16 or f32) -- no
//     staging buffers and no device-to-device concatenation.
#include "her_block.hpp"

namespace iqlh {

__global__ __launch_bounds__(256) void her_relabel_kernel(HerArgs a) { her_block(a, blockIdx.x); }

hipError_t launch_her_relabel(const HerArgs& a, hipStream_t stream) {
    if (a.n <= 0) return hipSuccess;
    const unsigned blocks = (unsigned)((a.n + kHerRows - 1) / kHerRows);
    hipLaunchKernelGGL(her_relabel_kernel, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace iqlh
