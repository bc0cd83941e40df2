// fused.hip -- dispatch of the one-pass kernels (fused_impl.h) by element
// type, and the one-pass AllGather (a copy of each owner's chunk).
#include "fused_impl.h"

namespace arlib {

template <int EB>
static hipError_t launch_fused_ag(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const dim3 block(kFusedThreads);
    // large calls: one unit per lane under a residency cap (fused_variant,
    // fused_waves_per_cu), the reservation being dynamic LDS no kernel reads
    const bool paced = fused_variant(p) == CFG_PACED;
    const unsigned lds = fused_lds_reserve(p);
    // 8 ranks: the rank loop unrolled, in the line-aligned form whatever the
    // layout (lead 0 when the layout is aligned).  Measured on MI355X against
    // the run-time-N kernel: 8 x 25 MiB fp32 37.2 vs 38.9 us, bf16 -2 %,
    // ragged counts -1.6 %; the plain 8-rank form was slower (40.1 us).
    if (p.vec && p.nranks == 8) {
        if (paced)
            hipLaunchKernelGGL(
                (k_fused<OpCopy<EB>, KIND_FUSED_AG, true, 8, FusedPaced, ORDER_RING, true>), grid,
                block, lds, s, a);
        else
            hipLaunchKernelGGL(
                (k_fused<OpCopy<EB>, KIND_FUSED_AG, true, 8, FusedWide, ORDER_RING, true>), grid,
                block, 0, s, a);
        return hipGetLastError();
    }
    if (paced) {
        if (p.lead)
            hipLaunchKernelGGL(
                (k_fused<OpCopy<EB>, KIND_FUSED_AG, true, 0, FusedPaced, ORDER_RING, true>), grid,
                block, lds, s, a);
        else
            hipLaunchKernelGGL((k_fused<OpCopy<EB>, KIND_FUSED_AG, true, 0, FusedPaced>), grid,
                               block, lds, s, a);
        return hipGetLastError();
    }
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
