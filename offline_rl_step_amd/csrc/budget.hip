// Budgeted clipped-SAXPY gradient accumulation and flat clipped Adam, gfx950.
//
// Follows "Gradient Stability -- Proper Multi-Task Gradient Isolation + Full
// Spectral Norm", section "Design -- Why the current per-component clipping is
// wrong" / "Proper design" (source k owns the fraction f_k of max_grad_norm;
// each source is clipped to its own budget in isolation and added with its
// scale; Adam keeps its safety clip at max_grad_norm) and "Task 1" (clipped
// SAXPY grad += alpha * clip(scratch, budget) with the scratch buffer's own
// norm).  The Adam step follows "DQN Backward-Path NaN Audit -- SP1 Phase A",
// section on iqn_adam_kernel.
//
// HBM-bound, three launches, all reductions in a fixed order (no float
// atomics, bitwise reproducible):
//   1. norms : one pass reads all k sources, per-block partial sums of squares;
//   2. saxpy : every block folds the partials into the k clip scales (same
//              order in every block), writes grad = sum_k alpha_k c_k s_k and a
//              per-block partial of ||grad||^2;
//   3. adam  : every block folds the grad partials into the combined norm and
//              applies the clipped Adam update, zeroing grad.
#include <mutex>

#include "budget_block.hpp"

namespace iqlh {

int budget_num_blocks(int64_t n) {
    const int64_t quads = (n + 3) / 4;
    int64_t nb = (quads + kBT - 1) / kBT;
    if (nb < 1) nb = 1;
    if (nb > kMaxBlocks) nb = kMaxBlocks;
    return (int)nb;
}

__global__ __launch_bounds__(kBT) void budget_norms_kernel(SourceSet s, int64_t n, int vec,
                                                             float* __restrict__ partials) {
    norms_block(s, n, vec, partials, blockIdx.x, gridDim.x);
}

// Blocks 0 .. nb - 1 run pass 2; with an Adam update, block nb counts its step.
__global__ __launch_bounds__(kBT) void budget_saxpy_kernel(SourceSet s, int64_t n, int vec, float mgn,
                                                            const float* __restrict__ partials,
                                                            float* __restrict__ grad,
                                                            float* __restrict__ gpart,
                                                            float* __restrict__ out_norms, int nb,
                                                            int32_t* __restrict__ adam_t, float* __restrict__ bc,
                                                            float beta1, float beta2) {
    if ((int)blockIdx.x < nb)
        saxpy_block<true>(s, n, vec, mgn, partials, grad, gpart, out_norms, blockIdx.x, nb);
    else
        adam_count_block(adam_t, bc, beta1, beta2);
}

__global__ __launch_bounds__(kBT) void norm_finalize_kernel(const float* __restrict__ p, int nb,
                                                             float* __restrict__ out) {
    norm_finalize_block(p, nb, out);
}

__global__ __launch_bounds__(kBT) void adam_flat_kernel(float* __restrict__ params, float* __restrict__ grad,
                                                         float* __restrict__ m, float* __restrict__ v,
                                                         const float* __restrict__ bc,
                                                         const float* __restrict__ sq_part, int nb, int64_t n,
                                                         int vec, AdamHyper hp, float* __restrict__ out_norm,
                                                         int32_t* __restrict__ flags) {
    adam_flat_block(params, grad, m, v, bc, sq_part, nb, n, vec, hp, out_norm, flags, blockIdx.x, gridDim.x);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

hipError_t launch_adam_flat(float* params, float* grad, float* m, float* v, const float* bc,
                            const float* sq_partials, int nb, int64_t n, const AdamHyper& hp,
                            float* out_norm, int32_t* flags, hipStream_t stream) {
    const int blocks = budget_num_blocks(n);
    const int vec = aligned16(params) && aligned16(grad) && aligned16(m) && aligned16(v);
    hipLaunchKernelGGL(adam_flat_kernel, dim3(blocks), dim3(kBT), 0, stream, params, grad, m, v, bc,
                       sq_partials, nb, n, vec, hp, out_norm, flags);
    return hipGetLastError();
}

hipError_t launch_budget(float* grad, const SourceSet& s, int64_t n, float mgn, float* out_norms,
                         float* params, float* m, float* v, int32_t* t, int32_t* flags,
                         const AdamHyper* hp, float* work, hipStream_t stream) {
    const int nb = budget_num_blocks(n);
    float* partials = work;
    float* gpart = work + (int64_t)s.k * nb;
    float* bc = gpart + nb;
    int vec = aligned16(grad);
    for (int j = 0; j < s.k; ++j) vec = vec && aligned16(s.ptr[j]);
    hipLaunchKernelGGL(budget_norms_kernel, dim3(nb), dim3(kBT), 0, stream, s, n, vec, partials);
    hipLaunchKernelGGL(budget_saxpy_kernel, dim3(nb + (hp ? 1 : 0)), dim3(kBT), 0, stream, s, n, vec, mgn,
                       partials, grad, gpart, out_norms, nb, t, bc, hp ? hp->beta1 : 0.f, hp ? hp->beta2 : 0.f);
    if (hp) {
        float* comb = out_norms ? out_norms + s.k : nullptr;
        return launch_adam_flat(params, grad, m, v, bc, gpart, nb, n, *hp, comb, flags, stream);
    }
    if (out_norms)
        hipLaunchKernelGGL(norm_finalize_kernel, dim3(1), dim3(kBT), 0, stream, gpart, nb,
                           out_norms + s.k);
    return hipGetLastError();
}

// ------------------------------------------------- allocation-free variant
// The largest workspace the three passes use (kMaxSources + 1 sets of
// kMaxBlocks partial sums and the two Adam bias corrections) as a file-scope
// device array, for callers that cannot allocate.  Every device the library
// runs on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device copy: kernels receive the
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchFloats = (size_t)(kMaxSources + 1) * kMaxBlocks + 2;
static __device__ __align__(256) float scratch[kScratchFloats];

size_t budget_scratch_bytes() { return sizeof(float) * kScratchFloats; }

// Device address of the current device's scratch, looked up once per device
// (with that device current) and kept; the passes need no initial contents.
hipError_t budget_scratch_ptr(float** out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static float* ptrs[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptrs[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        ptrs[dev] = (float*)p;
    }
    *out = ptrs[dev];
    return hipSuccess;
}

}  // namespace iqlh
