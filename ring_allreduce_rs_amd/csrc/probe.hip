// probe.hip -- how many one-wave blocks a compute unit holds at once under a
// given dynamic LDS reservation: the mechanism behind the fused kernels'
// residency caps, measured rather than assumed.
#include <hip/hip_runtime.h>

#include "probe.h"

namespace arlib {
namespace {

// hardware register reads (s_getreg): HW_ID bits 15:8 hold the CU, shader
// array and shader engine of the wave; XCC_ID bits 3:0 its accelerator die
constexpr unsigned kHwIdAll = 4u | (0u << 6) | (31u << 11);
constexpr unsigned kXccIdLow4 = 20u | (0u << 6) | (3u << 11);

__global__ __launch_bounds__(64) void k_residency_probe(unsigned* __restrict__ cur,
                                                        unsigned* __restrict__ mx, int spin) {
    if (threadIdx.x != 0) return;
    const unsigned hw = __builtin_amdgcn_s_getreg(kHwIdAll);
    const unsigned xcc = __builtin_amdgcn_s_getreg(kXccIdLow4);
    const unsigned key = ((xcc & 0xfu) << 8) | ((hw >> 8) & 0xffu);   // < kProbeSlots
    const unsigned c = atomicAdd(&cur[key], 1u) + 1u;
    atomicMax(&mx[key], c);
    for (int i = 0; i < spin; ++i) __builtin_amdgcn_s_sleep(127);   // bounded: spin rounds
    atomicSub(&cur[key], 1u);
}

}  // namespace

hipError_t launch_residency_probe(unsigned* cur, unsigned* mx, unsigned lds_bytes,
                                  unsigned blocks, int spin, hipStream_t s) {
    hipLaunchKernelGGL(k_residency_probe, dim3(blocks), dim3(64), lds_bytes, s, cur, mx, spin);
    return hipGetLastError();
}

}  // namespace arlib
