// The GPU side of the hybrid decode step's final add (FreeToken PR #491,
// "refactor(moe): extract hybrid decode orchestration", section 4: the CPU
// and GPU partial results are added).  The CPU partial sits in pinned,
// device-mapped host memory; it is folded into the fp32 term the routed
// combine adds (the shared term, or nothing), so the combine itself is
// unchanged.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void hybrid_add_kernel(float *__restrict__ addend,
                                                          const float *__restrict__ partial, int n,
                                                          int accumulate) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float p = partial[i];
    addend[i] = accumulate ? addend[i] + p : p;
}

}  // namespace

hipError_t launch_hybrid_add(float *addend, const float *partial, int n, int accumulate,
                             hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(hybrid_add_kernel, dim3((n + 255) / 256), dim3(256), 0, s, addend, partial, n,
                       accumulate);
    return hipGetLastError();
}

}  // namespace moe
