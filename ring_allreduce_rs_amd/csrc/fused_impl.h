// fused_impl.h -- the one-pass ring AllReduce / ReduceScatter / AllGather kernel
// (templates; instantiated per element type by fused_<type>.hip).
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
#pragma once

#include "common.h"

namespace arlib {

// Units ubase, ubase+kFusedThreads, ... (CFG::U of them, bounded by `units`)
// of the range starting at byte offset byte0 in every rank buffer; CFG::B
// ranks of loads are issued before they are folded.  NR > 0 fixes the rank
// count at compile time (loops fully unrolled); NR == 0 reads it from the
// arguments.
constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// A pause (s_sleep, in units of 64 cycles) between the fold and the stores
// of the 8-rank PACED ring and double-tree AllReduce over fp32.  Measured on
// MI355X in one process, pause 16 against none: 8 x 25 MiB AVG 69.9 -> 68.6
// us and 72.7 -> 71.8 us (two machines), SUM 72.7 -> 71.8, MAX 70.0 -> 69.1,
// double tree 69.9 -> 68.8; 8 x 100-200 MiB 2.4-2.9 % faster.  The int32
// kernels re-read their rank pointers from the argument block between the
// fold and the stores, which already delays their stores by a scalar
// round trip: a pause slowed them (8 x 25 MiB SUM 68.9 -> 71.7 us), as it
// did bf16 (71.5 -> 74.6), the pairwise orders (72.8 -> 73.9) and left the
// run-time rank count and the ReduceScatter level.
template <class Op, int MODE, int NR, class CFG, int ORDER>
constexpr int kStorePause =
    (std::is_same_v<CFG, FusedPaced> && NR == 8 && MODE == KIND_FUSED_AR &&
     (ORDER == ORDER_RING || ORDER == ORDER_DTREE) &&
     (std::is_same_v<Op, OpF32Sum> || std::is_same_v<Op, OpF32Max>))
        ? 16
        : 0;

template <class Op, int MODE, bool VEC, int NR, class CFG, int ORDER = ORDER_RING,
          bool LEAD = false>
__device__ __forceinline__ void fused_units(const Args& a, int c, int start, size_t byte0,
                                            size_t ubase, size_t units, unsigned lead = 0) {
    using X = Unit<Op, VEC, kFusedNT>;
    using T = typename X::T;
    constexpr int U = CFG::U;
    constexpr int kB = CFG::B;
    const int n = NR > 0 ? NR : a.n;
    bool ok[U];
    size_t off[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        // slot ubase + u*threads of the tile grid is unit (slot - lead) of the
        // body; a slot before the body wraps to a huge idx and fails the test
        const size_t idx = ubase + (size_t)u * kFusedThreads - (LEAD ? lead : 0u);
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
    } else if constexpr (ORDER == ORDER_PAIR || ORDER == ORDER_PAIR_BITREV) {
        // Pairwise tree over positions 0..n-1 (n a power of two); position q
        // holds rank q (PAIR) or rank bitrev(q) (PAIR_BITREV).  Each batch of
        // bn positions is folded as a subtree; batch results are merged as
        // they arrive, batch k taking its left partners from the levels whose
        // bit is set in k (a binary counter), which is the same balanced tree.
        // Every operator here is commutative, so a node's operand order does
        // not change its bits.
        (void)start;
        const int lg = 31 - __builtin_clz((unsigned)n);
        const int bn = n < kB ? n : kB;
        constexpr int kLevels = ilog2((NR > 0 ? NR : AR_MAX_RANKS) / kB);
        T st[kLevels > 0 ? kLevels : 1][U];
#pragma unroll
        for (int j0 = 0; j0 < (NR > 0 ? NR : AR_MAX_RANKS); j0 += kB) {
            if (NR == 0 && j0 >= n) break;
            const int k = j0 / kB;
            T v[kB][U];
#pragma unroll
            for (int j = 0; j < kB; ++j) {
                if (CFG::kWrapLoads || j < bn) {
                    const int q = j0 + (j & (bn - 1));
                    const int rank = ORDER == ORDER_PAIR || lg == 0
                                         ? q
                                         : (int)(__builtin_bitreverse32((unsigned)q) >> (32 - lg));
                    const char* src = rank_ptr(a, rank);
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[j][u] = ok[u] ? X::ld(src + off[u]) : X::zero();
                }
            }
            if constexpr (CFG::kWrapLoads) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int w = 1; w < kB; w *= 2) {
#pragma unroll
                for (int j = 0; j + w < kB; j += 2 * w) {
                    if (j + w < bn) {
#pragma unroll
                        for (int u = 0; u < U; ++u) v[j][u] = X::fold(v[j][u], v[j + w][u]);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] = v[0][u];
#pragma unroll
            for (int l = 0; l < kLevels; ++l) {
                if ((k >> l) & 1) {
#pragma unroll
                    for (int u = 0; u < U; ++u) acc[u] = X::fold(st[l][u], acc[u]);
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) st[l][u] = acc[u];
                    break;
                }
            }
        }
    } else if constexpr (ORDER == ORDER_DTREE) {
        // Double binary tree c (0 or 1) over positions 0..n-1 (n a power of
        // two); position p holds rank (p - c) mod n.  Position 0 is the root,
        // whose one child is n/2; a position whose lowest set bit is b > 1 has
        // children p - b/2 and p + b/2, so every subtree spans consecutive
        // positions.  A node folds (left (+) own) (+) right, the root own (+)
        // child.  The positions are scanned in order: an odd p is a finished
        // one-node subtree; as long as the finished subtree is a right child
        // (bit i of p set at level i) it closes its parent with the pending
        // (left (+) own) kept in pend[i]; an even p > 0 leaves its own pending
        // value in pend[ctz p].  With the loops unrolled every position and
        // level is a compile-time constant; only the rank count bounds them.
        (void)start;
        constexpr int kMaxN = NR > 0 ? NR : AR_MAX_RANKS;
        constexpr int kMaxL = ilog2(kMaxN);
        const int bn = n < kB ? n : kB;
        T root[U], cur[U];
        T pend[kMaxL > 0 ? kMaxL : 1][U];
#pragma unroll
        for (int u = 0; u < U; ++u) root[u] = cur[u] = X::zero();
#pragma unroll
        for (int j0 = 0; j0 < kMaxN; j0 += kB) {
            if (NR == 0 && j0 >= n) break;
            T v[kB][U];
#pragma unroll
            for (int j = 0; j < kB; ++j) {
                if (CFG::kWrapLoads || j < bn) {
                    const int q = j0 + (j & (bn - 1));
                    const int rank = q >= c ? q - c : q - c + n;
                    const char* src = rank_ptr(a, rank);
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[j][u] = ok[u] ? X::ld(src + off[u]) : X::zero();
                }
            }
            if constexpr (CFG::kWrapLoads) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < kB; ++j) {
                // (no early exits: they keep the compiler from unrolling these
                // loops, and the pending values would go to scratch memory)
                if (j >= bn) continue;
                const int p = j0 + j;
                if (p == 0) {
#pragma unroll
                    for (int u = 0; u < U; ++u) root[u] = v[j][u];
                } else if (p & 1) {
#pragma unroll
                    for (int u = 0; u < U; ++u) cur[u] = v[j][u];
                    // climb while the finished subtree is a right child: level
                    // i is reached when bits 1..i of p are all set
#pragma unroll
                    for (int i = 1; i < kMaxL; ++i) {
                        const int m = (2 << i) - 2;
                        if ((p & m) == m) {
#pragma unroll
                            for (int u = 0; u < U; ++u) cur[u] = X::fold(pend[i][u], cur[u]);
                        }
                    }
                } else {
                    const int lvl = __builtin_ctz((unsigned)p);
#pragma unroll
                    for (int u = 0; u < U; ++u) pend[lvl][u] = X::fold(cur[u], v[j][u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = n > 1 ? X::fold(root[u], cur[u]) : root[u];
    }
    if constexpr (MODE != KIND_FUSED_AG) {
        if constexpr (ORDER == ORDER_RING) {
        // ring order: start = c+1, then c+2, ..., ending with c itself
        int r = start;
        // With a run-time rank count and one unit per lane the batch loop
        // stays rolled: unrolled, the compiler hoisted later batches' loads
        // over the adds of the fp32 SUM kernel (228 VGPRs, one wave per SIMD,
        // 16 x 64 MiB 637 us against 342 us rolled).
        constexpr int kOuter =
            NR > 0 ? (NR + kB - 1) / kB : U > 1 ? (AR_MAX_RANKS + kB - 1) / kB : 1;
#pragma unroll kOuter
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
                        acc[u] = (j0 + j == 0) ? v[j][u] : X::fold(acc[u], v[j][u]);
                }
            }
            r = rr;
        }
        }  // ORDER_RING
        // every order folds with X::fold; a NaN becomes canonical here
#pragma unroll
        for (int u = 0; u < U; ++u) acc[u] = X::canon(acc[u]);
        if (a.avg) {
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] = X::fin(acc[u], a.nf, a.inv);
        }
        if constexpr (kStorePause<Op, MODE, NR, CFG, ORDER> > 0) {
            // the empty asm needs the folded values, so the fold (and any
            // AVG division) finishes before the pause begins
#pragma unroll
            for (int u = 0; u < U; ++u) asm volatile("" ::"v"(acc[u]));
            __builtin_amdgcn_s_sleep(kStorePause<Op, MODE, NR, CFG, ORDER>);
        }
        if constexpr (MODE == KIND_FUSED_RS) {
            char* dst = rank_ptr(a, c);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (ok[u]) X::st(dst + off[u], acc[u]);
        } else {
            if constexpr (ORDER != ORDER_RING || NR == 0) {
                // Hiding the offsets stops the compiler from keeping the load
                // addresses alive across the fold for reuse by these stores
                // (the pairwise orders load ranks in the stores' order: 56
                // more VGPRs; the run-time-N fp32 MAX loop: 17 more), which
                // costs a wave per SIMD.  Recomputing them is cheap.  The
                // 8-rank ring kernel does not reuse them and is left as is.
#pragma unroll
                for (int u = 0; u < U; ++u) asm volatile("" : "+v"(off[u]));
            }
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

// LEAD: tiles start on 128-byte lines (see below); launched only for plans
// whose chunk bodies can start off a line, so the aligned case keeps the
// plain indexing.
template <class Op, int MODE, bool VEC, int NR, class CFG, int ORDER = ORDER_RING,
          bool LEAD = false>
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
    // Tiles start on a 128-byte line of rank 0's buffer: a body starting
    // `lead` units past a line leaves the first `lead` slots of tile 0 idle,
    // so no wave access straddles a line that the next tile touches again.
    // The host sizes the grid for that slack whenever a lead can occur.
    const unsigned lead =
        VEC && LEAD
            ? (unsigned)(((reinterpret_cast<uintptr_t>(a.t.p[0]) + sp.body * EB) & 127u) >> 4)
            : 0u;
    const size_t ubase = (size_t)tile * (kFusedThreads * CFG::U) + threadIdx.x;
    if (ubase < sp.units + lead)
        fused_units<Op, MODE, VEC, NR, CFG, ORDER, LEAD>(a, c, start, sp.body * EB, ubase,
                                                         sp.units, lead);
    if constexpr (VEC) {
        // heads have at most 15 bytes (< 8 elements), as do tails
        if (tile == 0) {
            const unsigned t = threadIdx.x;
            if (t < sp.nhead)
                fused_units<Op, MODE, false, NR, FusedDeep, ORDER>(a, c, start, (lo + t) * EB, 0,
                                                                   1);
            else if (t >= kTailLane && t - kTailLane < sp.ntail)
                fused_units<Op, MODE, false, NR, FusedDeep, ORDER>(a, c, start,
                                                            (sp.tail + (t - kTailLane)) * EB, 0, 1);
        }
    }
}

// Which indexing a 16-byte-path plan runs with.  The line-aligned (LEAD)
// kernels are needed whenever a chunk body can start off a 128-byte line
// (p.lead).  On line-aligned layouts both forms are correct; measured on
// MI355X the LEAD forms ran 0.5-2.8 % faster there on the DEEP and run-time-N
// WIDE shapes, and 3.7 % slower on the 8-rank WIDE kernel, which therefore
// keeps the plain indexing when the layout allows it.  The 8-rank PACED
// kernels measured within 0.5 % either way, except ReduceScatter (LEAD 3.7 %
// slower) and 8 x 200 MiB (LEAD 1.2 % faster): they keep the plain form too.
inline bool use_lead(const Plan& p) {
    const int cfg = fused_variant(p);
    const bool n8_wide = p.nranks == 8 && (cfg == CFG_WIDE || cfg == CFG_PACED);
    return p.vec && (p.lead || !n8_wide);
}

template <class Op, int MODE, bool VEC, int ORDER, bool LEAD = false>
inline hipError_t launch_fused_n(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const dim3 block(kFusedThreads);
    const int cfg = fused_variant(p);
    const bool n8 = VEC && p.nranks == 8;
    // dynamic LDS that no kernel touches: it only caps the waves per CU
    const unsigned lds = fused_lds_reserve(p);
    // PACED runs the 16-byte path only, and bf16 only in the 8-rank form
    constexpr bool kPaced8 = VEC;
    constexpr bool kPacedN = VEC && Op::kElemBytes == 4;
    if constexpr (VEC && !LEAD) {
        // plain 16-byte indexing: the aligned 8-rank WIDE / PACED kernels
        // only (use_lead)
        if (!n8) return hipErrorInvalidConfiguration;
        if (cfg == CFG_WIDE)
            hipLaunchKernelGGL((k_fused<Op, MODE, true, 8, FusedWide, ORDER>), grid, block, lds, s, a);
        else if constexpr (kPaced8) {
            if (cfg != CFG_PACED) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL((k_fused<Op, MODE, true, 8, FusedPaced, ORDER>), grid, block, lds, s, a);
        } else {
            return hipErrorInvalidConfiguration;
        }
    } else if (cfg == CFG_TINY) {
        // element-wise units whatever the alignment (the grid was sized so);
        // never planned for the double tree (fused_variant)
        if constexpr (ORDER == ORDER_DTREE) return hipErrorInvalidConfiguration;
        else
            hipLaunchKernelGGL((k_fused<Op, MODE, false, 0, FusedTiny, ORDER>), grid, block, lds, s,
                               a);
    } else if (cfg == CFG_DEEP) {
        // the runtime-N loop measured faster than the 8-rank unrolled one here
        hipLaunchKernelGGL((k_fused<Op, MODE, VEC, 0, FusedDeep, ORDER, LEAD>), grid, block, lds, s, a);
    } else if (cfg == CFG_PACED) {
        if (n8) {
            if constexpr (kPaced8)
                hipLaunchKernelGGL((k_fused<Op, MODE, true, 8, FusedPaced, ORDER, LEAD>), grid, block,
                                   lds, s, a);
            else
                return hipErrorInvalidConfiguration;
        } else if constexpr (kPacedN && ORDER == ORDER_RING) {
            hipLaunchKernelGGL((k_fused<Op, MODE, true, 0, FusedPaced, ORDER_RING, LEAD>), grid, block,
                               lds, s, a);
        } else {
            return hipErrorInvalidConfiguration;   // fused_variant never asks
        }
    } else if (n8) {
        hipLaunchKernelGGL((k_fused<Op, MODE, VEC, 8, FusedWide, ORDER, LEAD>), grid, block, lds, s, a);
    } else if constexpr (ORDER == ORDER_RING) {
        hipLaunchKernelGGL((k_fused<Op, MODE, VEC, 0, FusedWide, ORDER_RING, LEAD>), grid, block, lds,
                           s, a);
    } else {
        return hipErrorInvalidConfiguration;   // no such kernel (fused_variant never asks)
    }
    return hipSuccess;
}

// LEAD selects the line-aligned instantiations (16-byte path only); the
// per-type files compile them in translation units of their own.
template <class Op, int MODE, int ORDER, bool LEAD>
inline hipError_t launch_fused_v(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    if constexpr (LEAD) return launch_fused_n<Op, MODE, true, ORDER, true>(p, a, grid, s);
    else
        return p.vec ? launch_fused_n<Op, MODE, true, ORDER>(p, a, grid, s)
                     : launch_fused_n<Op, MODE, false, ORDER>(p, a, grid, s);
}

template <class Op, bool LEAD = false>
inline hipError_t launch_fused_op(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const bool rs = p.kind == KIND_FUSED_RS;
    if (p.kind != KIND_FUSED_AR && !rs) return hipErrorInvalidValue;
    hipError_t e = hipErrorInvalidValue;
    switch (p.order) {
        case ORDER_RING:
            e = rs ? launch_fused_v<Op, KIND_FUSED_RS, ORDER_RING, LEAD>(p, a, grid, s)
                   : launch_fused_v<Op, KIND_FUSED_AR, ORDER_RING, LEAD>(p, a, grid, s);
            break;
        case ORDER_PAIR:   // recursive doubling: AllReduce only
            if (!rs) e = launch_fused_v<Op, KIND_FUSED_AR, ORDER_PAIR, LEAD>(p, a, grid, s);
            break;
        case ORDER_PAIR_BITREV:
            e = rs ? launch_fused_v<Op, KIND_FUSED_RS, ORDER_PAIR_BITREV, LEAD>(p, a, grid, s)
                   : launch_fused_v<Op, KIND_FUSED_AR, ORDER_PAIR_BITREV, LEAD>(p, a, grid, s);
            break;
        case ORDER_DTREE:   // double binary tree: AllReduce only
            if (!rs) e = launch_fused_v<Op, KIND_FUSED_AR, ORDER_DTREE, LEAD>(p, a, grid, s);
            break;
        default:
            break;
    }
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace arlib
