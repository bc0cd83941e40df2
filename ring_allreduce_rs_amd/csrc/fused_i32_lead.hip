// fused_i32_lead.hip -- the line-aligned (LEAD) one-pass kernels for one
// element type, in a translation unit of their own so they compile in
// parallel with the plain ones.
#include "fused_impl.h"

namespace arlib {

hipError_t launch_fused_i32_lead(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    return p.op == AR_MAX ? launch_fused_op<OpI32Max, true>(p, a, grid, s)
                          : launch_fused_op<OpI32Sum, true>(p, a, grid, s);
}

}  // namespace arlib
