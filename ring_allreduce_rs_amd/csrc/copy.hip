// copy.hip -- calibration streams: a plain 16-byte device copy (the reference
// stream for bandwidth ceilings and for scaling the hardware byte counters),
// and an R-read / W-write stream laid out like the fused AllReduce kernel
// (the ceiling of its access pattern without the reduction).
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

// R-read / W-write stream.  The tiling is the fused kernel's: one 64-lane
// wave per block, CFG::U units of 16 bytes per lane (WIDE: 4, so block b
// reads the same 4 KiB of every source and writes the same 4 KiB of every
// destination; PACED: 1, with the same cap on waves per CU as the fused
// kernel); sources are loaded 8 at a time before they are combined,
// destinations are written one after another.  The sources are combined with XOR (one bitwise
// instruction per word and source, no rounding), which keeps every load
// needed and makes the output checkable.  With no source the destinations
// get zeros; with no destination the combination is kept alive in a
// register so the loads still happen.  NR > 0 fixes both counts at compile
// time (the 8-rank fused kernel's fully unrolled form); NR == 0 reads them.
// TL adds a timeline: block b writes the device's constant-rate real-time
// counter at its start to ts[2b], and after all of its stores have completed
// to ts[2b + 1] (launched with at least one destination).
struct StreamArgs {
    RankTable src;
    RankTable dst;
    size_t units;   // 16-byte units per buffer
    int nsrc;
    int ndst;
    unsigned long long* ts;   // TL only
};

template <int NR, class CFG, bool TL = false>
__global__ __launch_bounds__(kFusedThreads) void k_stream(const StreamArgs a) {
    unsigned long long t0 = 0;
    if constexpr (TL) t0 = __builtin_amdgcn_s_memrealtime();
    constexpr int U = CFG::U;
    constexpr int kB = CFG::B;
    constexpr int kMax = NR > 0 ? NR : AR_MAX_RANKS;
    const int ns = NR > 0 ? NR : a.nsrc;
    const int nd = NR > 0 ? NR : a.ndst;
    const size_t ubase = (size_t)blockIdx.x * (kFusedThreads * U) + threadIdx.x;
    bool ok[U];
    size_t off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const size_t idx = ubase + (size_t)u * kFusedThreads;
        ok[u] = idx < a.units;
        off[u] = idx * 16;
    }
    u32x4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = u32x4{0u, 0u, 0u, 0u};
    // (rolled for a run-time source count at one unit per lane, as in the
    // fused kernel: unrolled, the loads of later batches were hoisted and
    // the kernel took 226 VGPRs)
    constexpr int kOuter = NR > 0 || U > 1 ? (kMax + kB - 1) / kB : 1;
#pragma unroll kOuter
    for (int j0 = 0; j0 < kMax; j0 += kB) {
        if (NR == 0 && j0 >= ns) break;
        u32x4 v[kB][U];
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            if (j0 + j < ns) {
                const char* s = reinterpret_cast<const char*>(a.src.p[j0 + j]);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    v[j][u] = ok[u] ? ld16<kFusedNT>(s + off[u]) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int j = 0; j < kB; ++j) {
            if (j0 + j < ns) {
#pragma unroll
                for (int u = 0; u < U; ++u) acc[u] ^= v[j][u];
            }
        }
    }
    if (nd == 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) asm volatile("" ::"v"(acc[u]));
        return;
    }
#pragma unroll
    for (int w = 0; w < kMax; ++w) {
        if (NR == 0 && w >= nd) break;
        char* d = reinterpret_cast<char*>(a.dst.p[w]);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (ok[u]) st16<kFusedNT>(d + off[u], acc[u]);
    }
    if constexpr (TL) {
        __builtin_amdgcn_s_waitcnt(0);   // every load and store of the wave done
        const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
        if (threadIdx.x == 0) {
            a.ts[2 * (size_t)blockIdx.x] = t0;
            a.ts[2 * (size_t)blockIdx.x + 1] = t1;
        }
    }
}

hipError_t launch_stream(const void* const* src, int nsrc, void* const* dst, int ndst,
                         size_t bytes, bool caps, hipStream_t stream) {
    if (nsrc < 0 || ndst < 0 || nsrc > AR_MAX_RANKS || ndst > AR_MAX_RANKS)
        return hipErrorInvalidValue;
    StreamArgs a;
    for (int r = 0; r < AR_MAX_RANKS; ++r) {
        a.src.p[r] = r < nsrc ? const_cast<void*>(src[r]) : nullptr;
        a.dst.p[r] = r < ndst ? dst[r] : nullptr;
    }
    a.units = bytes / 16;
    a.nsrc = nsrc;
    a.ndst = ndst;
    a.ts = nullptr;
    if (a.units == 0 || nsrc + ndst == 0) return hipSuccess;
    // the fused kernel's choice for an AllReduce of nsrc ranks of `bytes`
    // each: PACED (one unit per lane, capped) from 8 sources up when the
    // sources hold more than kPacedMinBytes in all, else WIDE
    const bool paced = caps && nsrc >= kBatch && (size_t)nsrc * bytes > kPacedMinBytes;
    const size_t per_block = (size_t)kFusedThreads * (paced ? FusedPaced::U : FusedWide::U);
    const size_t blocks = ceil_div(a.units, per_block);
    if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks), block(kFusedThreads);
    const unsigned lds = paced ? lds_for_waves(kPacedRingWaves) : 0u;
    const bool n8 = nsrc == 8 && ndst == 8;
    if (paced && n8)
        hipLaunchKernelGGL((k_stream<8, FusedPaced>), grid, block, lds, stream, a);
    else if (paced)
        hipLaunchKernelGGL((k_stream<0, FusedPaced>), grid, block, lds, stream, a);
    else if (n8)
        hipLaunchKernelGGL((k_stream<8, FusedWide>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((k_stream<0, FusedWide>), grid, block, 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_stream_timeline(void* const* bufs, int n, size_t bytes, unsigned lds,
                                  unsigned long long* ts, hipStream_t stream) {
    if (n < 1 || n > AR_MAX_RANKS || !ts) return hipErrorInvalidValue;
    StreamArgs a;
    for (int r = 0; r < AR_MAX_RANKS; ++r) a.src.p[r] = a.dst.p[r] = r < n ? bufs[r] : nullptr;
    a.units = bytes / 16;
    a.nsrc = a.ndst = n;
    a.ts = ts;
    if (a.units == 0) return hipSuccess;
    const size_t blocks = ceil_div(a.units, (size_t)kFusedThreads * FusedPaced::U);
    if (blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)blocks), block(kFusedThreads);
    if (n == 8)
        hipLaunchKernelGGL((k_stream<8, FusedPaced, true>), grid, block, lds, stream, a);
    else
        hipLaunchKernelGGL((k_stream<0, FusedPaced, true>), grid, block, lds, stream, a);
    return hipGetLastError();
}

}  // namespace arlib
