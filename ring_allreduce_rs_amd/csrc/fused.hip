// fused.hip -- dispatch of the one-pass kernels (fused_impl.h) by element
// type, and the one-pass AllGather (a copy of each owner's chunk).
#include "fused_impl.h"

namespace arlib {

template <int EB>
static hipError_t launch_fused_ag(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const dim3 block(kFusedThreads);
    if (p.vec && p.lead)
        hipLaunchKernelGGL((k_fused<OpCopy<EB>, KIND_FUSED_AG, true, 0, FusedWide, ORDER_RING, true>),
                           grid, block, 0, s, a);
    else if (p.vec)
        hipLaunchKernelGGL((k_fused<OpCopy<EB>, KIND_FUSED_AG, true, 0, FusedWide>), grid, block, 0,
                           s, a);
    else
        hipLaunchKernelGGL((k_fused<OpCopy<EB>, KIND_FUSED_AG, false, 0, FusedWide>), grid, block,
                           0, s, a);
    return hipGetLastError();
}

hipError_t launch_fused_kind(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    if (p.kind == KIND_FUSED_AG)
        return elem_bytes(p.dtype) == 2 ? launch_fused_ag<2>(p, a, grid, s)
                                        : launch_fused_ag<4>(p, a, grid, s);
    switch (p.dtype) {
        case AR_INT32: return launch_fused_i32(p, a, grid, s);
        case AR_FLOAT32: return launch_fused_f32(p, a, grid, s);
        case AR_BFLOAT16: return launch_fused_bf16(p, a, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace arlib
