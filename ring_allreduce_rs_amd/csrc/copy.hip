// copy.hip -- plain 16-byte device copy: the reference stream for bandwidth
// ceilings and for scaling the hardware byte counters.
#include "common.h"

namespace arlib {

__global__ __launch_bounds__(kThreads) void k_copy(u32x4* __restrict__ dst,
                                                   const u32x4* __restrict__ src, size_t nvec) {
    const size_t base = (size_t)blockIdx.x * (kThreads * kCopyUnroll) + threadIdx.x;
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const size_t i = base + (size_t)u * kThreads;
        v[u] = i < nvec ? ld16<true>(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
        const size_t i = base + (size_t)u * kThreads;
        if (i < nvec) st16<true>(dst + i, v[u]);
    }
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
    const size_t nvec = bytes / 16;
    if (nvec == 0) return hipSuccess;
    const size_t blocks = ceil_div(nvec, (size_t)kThreads * kCopyUnroll);
    if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_copy, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<u32x4*>(dst), reinterpret_cast<const u32x4*>(src), nvec);
    return hipGetLastError();
}

}  // namespace arlib
