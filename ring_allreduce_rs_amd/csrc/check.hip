// check.hip -- on-device checker of an AllReduce result: whether every rank
// holds the same bits, and how far rank 0 is from a binary64 reference.
//
// An AllReduce leaves every participant with the same reduced data ("AllReduce",
// compassingai.com, section 3 技术原理); for a floating-point SUM the result is
// also compared with the exact sum through an error bound.  The checker does
// both over the whole array without copying it to the host:
//   pass 1 (k_check_partial): a grid of at most kCheckMaxBlocks blocks walks
//     the positions; each lane compares every rank with rank 0 and, given a
//     reference, forms |x - ref| in binary64; the lane results are combined
//     across the wavefront with shuffles (sum of counts, minimum position,
//     maximum error), across the block's waves through LDS, and each block
//     writes one partial record to a scratch array;
//   pass 2 (k_check_final): one block folds the partial records the same way
//     and writes the result.
// Two passes and a fixed combination tree make the result deterministic and
// need no atomics.
#include <mutex>

#include "common.h"

namespace arlib {

// The scratch of ar_check_noalloc: kCheckMaxBlocks partial records resident
// on every GPU the library runs on, for the life of the process.  Host code
// uses the per-device address from check_static_scratch(), never this name
// (on the host it only stands in for the symbol).
static __device__ __align__(256) CheckPartial scratch[kCheckMaxBlocks];

namespace {

__device__ __forceinline__ double elem_to_f64(uint32_t u, int dtype) {
    if (dtype == AR_INT32) return (double)(int32_t)u;
    if (dtype == AR_FLOAT32) return (double)__uint_as_float(u);
    return (double)__uint_as_float(u << 16);   // bf16 widens exactly
}

struct Acc {
    unsigned long long mismatched;
    unsigned long long first;      // smallest mismatching position, ~0 if none
    unsigned long long over;
    double max_err;                // largest finite-or-inf error seen
    unsigned nan;                  // 1 if some error was NaN
};

__device__ __forceinline__ void combine(Acc& a, const Acc& b) {
    a.mismatched += b.mismatched;
    a.first = b.first < a.first ? b.first : a.first;
    a.over += b.over;
    a.max_err = b.max_err > a.max_err ? b.max_err : a.max_err;
    a.nan |= b.nan;
}

// Butterfly over the 64 lanes of a wavefront: after it every lane holds the
// combination of all 64 lanes' values.
__device__ __forceinline__ Acc wave_combine(Acc a) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        Acc o;
        o.mismatched = __shfl_xor(a.mismatched, d, 64);
        o.first = __shfl_xor(a.first, d, 64);
        o.over = __shfl_xor(a.over, d, 64);
        o.max_err = __shfl_xor(a.max_err, d, 64);
        o.nan = __shfl_xor(a.nan, d, 64);
        combine(a, o);
    }
    return a;
}

// The block's waves: each wave's lane 0 leaves its combination in LDS and
// thread 0 folds them in wave order.
__device__ __forceinline__ bool block_combine(Acc& a) {
    __shared__ Acc lds[kCheckThreads / 64];
    a = wave_combine(a);
    const unsigned wave = threadIdx.x / 64;
    if ((threadIdx.x & 63) == 0) lds[wave] = a;
    __syncthreads();
    if (threadIdx.x != 0) return false;
    a = lds[0];
    for (unsigned w = 1; w < kCheckThreads / 64; ++w) combine(a, lds[w]);
    return true;
}

__device__ __forceinline__ Acc acc_zero() {
    Acc a;
    a.mismatched = 0;
    a.first = ~0ull;
    a.over = 0;
    a.max_err = 0.0;
    a.nan = 0;
    return a;
}

template <int EB>
__global__ __launch_bounds__(kCheckThreads) void k_check_partial(const CheckArgs a,
                                                                 CheckPartial* __restrict__ part) {
    Acc acc = acc_zero();
    const size_t stride = (size_t)gridDim.x * kCheckThreads;
    for (size_t i = (size_t)blockIdx.x * kCheckThreads + threadIdx.x; i < a.count; i += stride) {
        const uint32_t v0 = ld_elem<EB>(reinterpret_cast<const char*>(a.t.p[0]) + i * EB);
        bool diff = false;
        for (int r = 1; r < a.n; ++r)
            diff |= ld_elem<EB>(reinterpret_cast<const char*>(a.t.p[r]) + i * EB) != v0;
        if (diff) {
            ++acc.mismatched;
            if (i < acc.first) acc.first = i;
        }
        if (a.ref) {
            const double e = fabs(elem_to_f64(v0, a.dtype) - a.ref[i]);
            if (e != e) {
                acc.nan = 1;
                ++acc.over;
            } else {
                if (e > acc.max_err) acc.max_err = e;
                if (a.bound && !(e <= a.bound[i])) ++acc.over;
            }
        }
    }
    if (block_combine(acc)) {
        CheckPartial& p = part[blockIdx.x];
        p.mismatched = acc.mismatched;
        p.first = acc.first;
        p.over = acc.over;
        p.max_err = acc.max_err;
        p.nan = acc.nan;
    }
}

__global__ __launch_bounds__(kCheckThreads) void k_check_final(const CheckPartial* __restrict__ part,
                                                               unsigned nparts, size_t count,
                                                               ar_check_result* __restrict__ out) {
    Acc acc = acc_zero();
    for (unsigned j = threadIdx.x; j < nparts; j += kCheckThreads) {
        Acc b;
        b.mismatched = part[j].mismatched;
        b.first = part[j].first;
        b.over = part[j].over;
        b.max_err = part[j].max_err;
        b.nan = part[j].nan;
        combine(acc, b);
    }
    if (block_combine(acc)) {
        out->mismatched = acc.mismatched;
        out->first_mismatch = acc.mismatched ? acc.first : (unsigned long long)count;
        out->over_bound = acc.over;
        out->max_abs_err = acc.nan ? __longlong_as_double(0x7ff8000000000000ll) : acc.max_err;
    }
}

}  // namespace

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
CheckPartial* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t check_static_scratch(int device, CheckPartial** out) {
    *out = nullptr;
    if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[device] = static_cast<CheckPartial*>(p);
    }
    *out = g_scratch_ptr[device];
    return hipSuccess;
}

unsigned check_blocks(size_t count) {
    const size_t want = ceil_div(count, (size_t)kCheckThreads);
    return (unsigned)(want == 0 ? 1 : want < kCheckMaxBlocks ? want : kCheckMaxBlocks);
}

hipError_t launch_check(const CheckArgs& a, CheckPartial* part, ar_check_result* out,
                        hipStream_t s) {
    const unsigned blocks = check_blocks(a.count);
    if (a.count > 0) {
        if (a.eb == 2)
            hipLaunchKernelGGL(k_check_partial<2>, dim3(blocks), dim3(kCheckThreads), 0, s, a, part);
        else
            hipLaunchKernelGGL(k_check_partial<4>, dim3(blocks), dim3(kCheckThreads), 0, s, a, part);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_check_final, dim3(1), dim3(kCheckThreads), 0, s, part,
                       a.count > 0 ? blocks : 0u, a.count, out);
    return hipGetLastError();
}

}  // namespace arlib
