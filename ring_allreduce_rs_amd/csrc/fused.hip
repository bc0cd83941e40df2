// fused.hip -- the one-pass ring AllReduce / ReduceScatter / AllGather kernel.
//
// Ring schedule (pwwt.cn page "Allreduce：大模型分布式训练的核心通信算法与优化实践",
// section 2.2, read as: ReduceScatter step k sends chunk (r-k-1) mod N from
// rank r to rank r+1; AllGather step k forwards chunk (r-k) mod N).  Chunk c
// is therefore folded over ranks c+1, c+2, ..., c-1, c, left to right, and
// ends on rank c.  k_fused reads each 16-byte unit of chunk c from every rank
// (in that order, kBatch ranks of loads in flight before the adds), folds in
// registers with the same per-hop rounding as the per-step ring, and stores
// the result to all N ranks (AllReduce), to the owner only (ReduceScatter), or
// copies the owner's unit to the others (AllGather): 2*N*K bytes for an
// AllReduce, the minimum.
//
// Block -> work mapping: block b handles tile (b mod tiles) of chunk
// (b / tiles), so the chunk -- and with it the first rank of the fold and
// every rank pointer -- is uniform across the block and lives in scalar
// registers.  A chunk whose start is not 16-byte aligned (counts not divisible
// by N, e.g. 268,435,459 over 16 ranks) has a head of up to 15 bytes and a
// tail, handled element by element by lanes of the chunk's first tile.
#include "common.h"

namespace arlib {

// Units ubase, ubase+kFusedThreads, ... (CFG::U of them, bounded by `units`)
// of the range starting at byte offset byte0 in every rank buffer; CFG::B
// ranks of loads are issued before they are folded.  NR > 0 fixes the rank
// count at compile time (loops fully unrolled); NR == 0 reads it from the
// arguments.
template <class Op, int MODE, bool VEC, int NR, class CFG>
__device__ __forceinline__ void fused_units(const Args& a, int c, int start, size_t byte0,
                                            size_t ubase, size_t units) {
    using X = Unit<Op, VEC, kFusedNT>;
    using T = typename X::T;
    constexpr int U = CFG::U;
    constexpr int kB = CFG::B;
    const int n = NR > 0 ? NR : a.n;
    bool ok[U];
    size_t off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t idx = ubase + (size_t)u * kFusedThreads;
        ok[u] = idx < units;
        off[u] = byte0 + idx * X::kBytes;
    }
    T acc[U];
    if constexpr (MODE == KIND_FUSED_AG) {
        const char* src = rank_ptr(a, c);
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = ok[u] ? X::ld(src + off[u]) : X::zero();
        for (int r = 0; r < n; ++r) {
            if (r == c) continue;
            char* dst = rank_ptr(a, r);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) X::st(dst + off[u], acc[u]);
        }
        return;
    } else {
        // ring order: start = c+1, then c+2, ..., ending with c itself
        int r = start;
#pragma unroll
        for (int j0 = 0; j0 < (NR > 0 ? NR : AR_MAX_RANKS); j0 += kB) {
            if (NR == 0 && j0 >= n) break;
            T v[kB][U];
            int rr = r;
#pragma unroll
            for (int j = 0; j < kB; ++j) {
                // kWrapLoads: issue every slot's load (ranks wrap mod n, so the
                // addresses stay valid) and keep only the first n in the fold;
                // a uniform guard here lets the compiler serialise the loads
                if (CFG::kWrapLoads || j0 + j < n) {
                    const char* src = rank_ptr(a, rr);
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[j][u] = ok[u] ? X::ld(src + off[u]) : X::zero();
                    rr = (rr + 1 == n) ? 0 : rr + 1;
                }
            }
            // keep the adds behind the whole batch: one memory round trip
            if constexpr (CFG::kWrapLoads) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kB; ++j) {
                if (j0 + j < n) {
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        acc[u] = (j0 + j == 0) ? v[j][u] : X::comb(acc[u], v[j][u]);
                }
            }
            r = rr;
        }
        if (a.avg) {
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] = X::fin(acc[u], a.nf, a.inv);
        }
        if constexpr (MODE == KIND_FUSED_RS) {
            char* dst = rank_ptr(a, c);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) X::st(dst + off[u], acc[u]);
        } else {
#pragma unroll
            for (int r2 = 0; r2 < (NR > 0 ? NR : AR_MAX_RANKS); ++r2) {
                if (NR == 0 && r2 >= n) break;
                char* dst = rank_ptr(a, r2);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (ok[u]) X::st(dst + off[u], acc[u]);
            }
        }
    }
}

template <class Op, int MODE, bool VEC, int NR, class CFG>
__global__ __launch_bounds__(kFusedThreads) void k_fused(const Args a) {
    constexpr int EB = Op::kElemBytes;
    const int n = NR > 0 ? NR : a.n;
    const int c = (int)(blockIdx.x / a.tiles);
    const unsigned tile = blockIdx.x - (unsigned)c * a.tiles;
    size_t lo, len;
    chunk_bounds(a, c, lo, len);
    if (len == 0) return;
    const Span sp = make_span<EB, VEC>(lo, len, a.mis);
    const int start = (c + 1 == n) ? 0 : c + 1;
    const size_t ubase = (size_t)tile * (kFusedThreads * CFG::U) + threadIdx.x;
    if (ubase < sp.units)
        fused_units<Op, MODE, VEC, NR, CFG>(a, c, start, sp.body * EB, ubase, sp.units);
    if constexpr (VEC) {
        // heads have at most 15 bytes (< 8 elements), as do tails
        if (tile == 0) {
            const unsigned t = threadIdx.x;
            if (t < sp.nhead)
                fused_units<Op, MODE, false, NR, FusedDeep>(a, c, start, (lo + t) * EB, 0, 1);
            else if (t >= kTailLane && t - kTailLane < sp.ntail)
                fused_units<Op, MODE, false, NR, FusedDeep>(a, c, start,
                                                            (sp.tail + (t - kTailLane)) * EB, 0, 1);
        }
    }
}

template <class Op, int MODE, bool VEC>
static void launch_fused_n(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const dim3 block(kFusedThreads);
    const int cfg = fused_variant(p);
    const bool n8 = AR_SPECIALIZE_N && VEC && p.nranks == 8;
    if (cfg == CFG_TINY) {
        // element-wise units whatever the alignment (the grid was sized so)
        hipLaunchKernelGGL((k_fused<Op, MODE, false, 0, FusedTiny>), grid, block, 0, s, a);
    } else if (cfg == CFG_DEEP) {
        // the runtime-N loop measured faster than the 8-rank unrolled one here
        hipLaunchKernelGGL((k_fused<Op, MODE, VEC, 0, FusedDeep>), grid, block, 0, s, a);
    } else if (cfg == CFG_MID) {
        hipLaunchKernelGGL((k_fused<Op, MODE, VEC, 0, FusedMid>), grid, block, 0, s, a);
    } else {
        if (n8) hipLaunchKernelGGL((k_fused<Op, MODE, VEC, 8, FusedWide>), grid, block, 0, s, a);
        else hipLaunchKernelGGL((k_fused<Op, MODE, VEC, 0, FusedWide>), grid, block, 0, s, a);
    }
}

template <class Op>
static hipError_t launch_fused_op(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    if (p.kind == KIND_FUSED_AR) {
        if (p.vec) launch_fused_n<Op, KIND_FUSED_AR, true>(p, a, grid, s);
        else launch_fused_n<Op, KIND_FUSED_AR, false>(p, a, grid, s);
    } else if (p.kind == KIND_FUSED_RS) {
        if (p.vec) launch_fused_n<Op, KIND_FUSED_RS, true>(p, a, grid, s);
        else launch_fused_n<Op, KIND_FUSED_RS, false>(p, a, grid, s);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int EB>
static hipError_t launch_fused_ag(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const dim3 block(kFusedThreads);
    if (p.vec)
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
    const bool mx = p.op == AR_MAX;
    switch (p.dtype) {
        case AR_INT32:
            return mx ? launch_fused_op<OpI32Max>(p, a, grid, s) : launch_fused_op<OpI32Sum>(p, a, grid, s);
        case AR_FLOAT32:
            return mx ? launch_fused_op<OpF32Max>(p, a, grid, s) : launch_fused_op<OpF32Sum>(p, a, grid, s);
        case AR_BFLOAT16:
            return mx ? launch_fused_op<OpBF16Max>(p, a, grid, s)
                      : launch_fused_op<OpBF16Sum>(p, a, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace arlib
