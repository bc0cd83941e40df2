// fused_i32.hip -- one-pass kernels instantiated for one element type (kept in
// a translation unit of its own so the types compile in parallel).
#include "fused_impl.h"

namespace arlib {

hipError_t launch_fused_i32(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    if (use_lead(p)) return launch_fused_i32_lead(p, a, grid, s);
    return p.op == AR_MAX ? launch_fused_op<OpI32Max>(p, a, grid, s)
                          : launch_fused_op<OpI32Sum>(p, a, grid, s);
}

}  // namespace arlib
