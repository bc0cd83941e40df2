// steps.hip -- one kernel launch per step of the ring, recursive-doubling,
// recursive halving-doubling and double-binary-tree AllReduce.
//
//   k_rs_step      one ring ReduceScatter step: every rank's chunk folded into
//                  its successor's copy (AVG divide fused into the last step).
//   k_ag_step      one ring AllGather step: chunk copied to the successor.
//   k_tree_step    one recursive-doubling step ("集合通信基础AllReduce、Ring算法
//                  与NCCL全解析", section 4.1): both partners of a pair get the
//                  combination of their vectors.
//   k_hd_rs_step / k_hd_ag_step
//                  recursive-halving ReduceScatter and recursive-doubling
//                  AllGather steps (the same page's "Recursive Doubling /
//                  Halving", read as the bandwidth-optimal variant).
//   k_dtree_step   one level of the double binary tree (two complementary
//                  trees, each reducing half the vector up and broadcasting
//                  it down).
//
// These kernels keep ordinary (cached) stores: each step re-reads what the
// previous one wrote, and with working sets up to the Infinity Cache size
// those reads hit it.
#include "common.h"

namespace arlib {

// dst[i] <- comb(src[i], dst[i]) (REDUCE) or dst[i] <- src[i] (copy); with
// `both`, src[i] also receives the combination (tree).
template <class Op, bool VEC, bool REDUCE, bool BOTH>
__device__ __forceinline__ void pair_units(char* src, char* dst, size_t byte0, size_t ubase,
                                           size_t units, bool fin, float nf, float inv) {
    using X = Unit<Op, VEC, kStepNT>;
    using T = typename X::T;
    bool ok[kUnroll];
    size_t off[kUnroll];
    T x[kUnroll], y[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const size_t idx = ubase + (size_t)u * kThreads;
        ok[u] = idx < units;
        off[u] = byte0 + idx * X::kBytes;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        x[u] = ok[u] ? X::ld(src + off[u]) : X::zero();
        if constexpr (REDUCE) y[u] = ok[u] ? X::ld(dst + off[u]) : X::zero();
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        T z = x[u];
        if constexpr (REDUCE) {
            z = X::comb(x[u], y[u]);
            if (fin) z = X::fin(z, nf, inv);
        }
        if (ok[u]) {
            X::st(dst + off[u], z);
            if constexpr (BOTH) X::st(src + off[u], z);
        }
    }
}

template <class Op, bool VEC, bool REDUCE, bool BOTH>
__device__ __forceinline__ void pair_range(char* src, char* dst, size_t lo, size_t len,
                                           unsigned mis, unsigned tile, bool fin, float nf,
                                           float inv) {
    constexpr int EB = Op::kElemBytes;
    const Span sp = make_span<EB, VEC>(lo, len, mis);
    const size_t ubase = (size_t)tile * (kThreads * kUnroll) + threadIdx.x;
    if (ubase < sp.units)
        pair_units<Op, VEC, REDUCE, BOTH>(src, dst, sp.body * EB, ubase, sp.units, fin, nf, inv);
    if constexpr (VEC) {
        if (tile == 0) {
            const unsigned t = threadIdx.x;
            if (t < sp.nhead)
                pair_units<Op, false, REDUCE, BOTH>(src, dst, (lo + t) * EB, 0, 1, fin, nf, inv);
            else if (t >= kTailLane && t - kTailLane < sp.ntail)
                pair_units<Op, false, REDUCE, BOTH>(src, dst, (sp.tail + (t - kTailLane)) * EB, 0,
                                                    1, fin, nf, inv);
        }
    }
}

// ReduceScatter step k: rank r folds its chunk (r-k-1) mod N into rank r+1.
template <class Op, bool VEC>
__global__ __launch_bounds__(kThreads) void k_rs_step(const Args a) {
    const int n = a.n;
    const int r = (int)(blockIdx.x / a.tiles);
    const unsigned tile = blockIdx.x - (unsigned)r * a.tiles;
    const int c = (r + 2 * n - a.step - 1) % n;
    const int d = (r + 1 == n) ? 0 : r + 1;
    size_t lo, len;
    chunk_bounds(a, c, lo, len);
    if (len == 0) return;
    const bool fin = a.avg && a.step == n - 2;   // the receiver now owns chunk c
    pair_range<Op, VEC, true, false>(rank_ptr(a, r), rank_ptr(a, d), lo, len, a.mis, tile,
                                     fin, a.nf, a.inv);
}

// AllGather step k: rank r forwards chunk (r-k) mod N to rank r+1 unchanged.
template <class Op, bool VEC>
__global__ __launch_bounds__(kThreads) void k_ag_step(const Args a) {
    const int n = a.n;
    const int r = (int)(blockIdx.x / a.tiles);
    const unsigned tile = blockIdx.x - (unsigned)r * a.tiles;
    const int c = (r + n - a.step) % n;
    const int d = (r + 1 == n) ? 0 : r + 1;
    size_t lo, len;
    chunk_bounds(a, c, lo, len);
    if (len == 0) return;
    pair_range<Op, VEC, false, false>(rank_ptr(a, r), rank_ptr(a, d), lo, len, a.mis, tile,
                                      false, a.nf, a.inv);
}

// Recursive-doubling step s: pair q is (r, r | 2^s) with bit s of r clear.
template <class Op, bool VEC>
__global__ __launch_bounds__(kThreads) void k_tree_step(const Args a) {
    const unsigned q = blockIdx.x / a.tiles;
    const unsigned tile = blockIdx.x - q * a.tiles;
    const int s = a.step;
    const unsigned low = q & ((1u << s) - 1u);
    const int r = (int)(((q >> s) << (s + 1)) | low);
    const int p = r | (1 << s);
    const bool fin = a.avg && (2 << s) == a.n;   // last step
    pair_range<Op, VEC, true, true>(rank_ptr(a, p), rank_ptr(a, r), 0, a.count, a.mis, tile,
                                    fin, a.nf, a.inv);
}

// Recursive-halving ReduceScatter step s: distance d = N / 2^(s+1); rank r
// keeps the d chunks starting at r with its low log2(d) bits cleared and folds
// partner r^d's copy of them into its own.  The partner keeps the other half
// of the same 2d-chunk segment, so nothing read in a step is written in it.
// After the last step (d = 1) rank r holds the finished chunk r.
template <class Op, bool VEC>
__global__ __launch_bounds__(kThreads) void k_hd_rs_step(const Args a) {
    const int n = a.n;
    const int r = (int)(blockIdx.x / a.tiles);
    const unsigned tile = blockIdx.x - (unsigned)r * a.tiles;
    const int d = n >> (a.step + 1);
    const int keep = r & ~(d - 1);
    const int p = r ^ d;
    size_t lo, len0, lo1, len1;
    chunk_bounds(a, keep, lo, len0);
    chunk_bounds(a, keep + d - 1, lo1, len1);
    const size_t len = lo1 + len1 - lo;
    if (len == 0) return;
    const bool fin = a.avg && d == 1;
    pair_range<Op, VEC, true, false>(rank_ptr(a, p), rank_ptr(a, r), lo, len, a.mis, tile, fin,
                                     a.nf, a.inv);
}

// Recursive-doubling AllGather step t: distance d = 2^t; rank r copies the d
// finished chunks held by partner r^d.
template <class Op, bool VEC>
__global__ __launch_bounds__(kThreads) void k_hd_ag_step(const Args a) {
    const int r = (int)(blockIdx.x / a.tiles);
    const unsigned tile = blockIdx.x - (unsigned)r * a.tiles;
    const int d = 1 << a.step;
    const int p = r ^ d;
    const int first = p & ~(d - 1);
    size_t lo, len0, lo1, len1;
    chunk_bounds(a, first, lo, len0);
    chunk_bounds(a, first + d - 1, lo1, len1);
    const size_t len = lo1 + len1 - lo;
    if (len == 0) return;
    pair_range<Op, VEC, false, false>(rank_ptr(a, p), rank_ptr(a, r), lo, len, a.mis, tile,
                                      false, a.nf, a.inv);
}

// ---------------------------------------------------------------- double binary tree
//
// Two complementary in-order binary trees ("AllReduce", compassingai.com,
// section 3: reduce leaves-to-root, broadcast root-to-leaves; the double tree
// runs two disjoint trees at once, each with part of the data).  Shape on
// positions 0..N-1 (N a power of two): position 0 is the root with the single
// child N/2; position v with lowest set bit b > 1 has children v - b/2 and
// v + b/2.  Tree 0 places rank v at position v and carries elements
// [0, ceil(count/2)); tree 1 places rank (v-1) mod N at position v and
// carries the rest.  Steps (L = log2 N):
//   s <  L-1  reduce level l = s+1: node v <- (left (+) own) (+) right
//   s == L-1  root: node 0 <- own (+) node N/2, AVG divides here
//   s == L    node N/2 <- node 0
//   s >  L    broadcast level l = 2L-s: both children <- node v

enum DtMode { DT_REDUCE3 = 0, DT_REDUCE2 = 1, DT_COPY1 = 2, DT_COPY2 = 3 };

// a, b, c are left child / own (parent) / right child (REDUCE3, COPY2) or
// unused / own / child (REDUCE2, COPY1).
template <class Op, bool VEC, int MODE>
__device__ __forceinline__ void dt_units(char* a, char* b, char* c, size_t byte0, size_t ubase,
                                         size_t units, bool fin, float nf, float inv) {
    using X = Unit<Op, VEC, kStepNT>;
    using T = typename X::T;
    bool ok[kUnroll];
    size_t off[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const size_t idx = ubase + (size_t)u * kThreads;
        ok[u] = idx < units;
        off[u] = byte0 + idx * X::kBytes;
    }
    T x[kUnroll], y[kUnroll], z[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        y[u] = ok[u] ? X::ld(b + off[u]) : X::zero();
        if constexpr (MODE == DT_REDUCE3) x[u] = ok[u] ? X::ld(a + off[u]) : X::zero();
        if constexpr (MODE == DT_REDUCE3 || MODE == DT_REDUCE2)
            z[u] = ok[u] ? X::ld(c + off[u]) : X::zero();
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        if (!ok[u]) continue;
        if constexpr (MODE == DT_REDUCE3) {
            X::st(b + off[u], X::comb(X::comb(x[u], y[u]), z[u]));
        } else if constexpr (MODE == DT_REDUCE2) {
            T r = X::comb(y[u], z[u]);
            if (fin) r = X::fin(r, nf, inv);
            X::st(b + off[u], r);
        } else if constexpr (MODE == DT_COPY1) {
            X::st(c + off[u], y[u]);
        } else {
            X::st(a + off[u], y[u]);
            X::st(c + off[u], y[u]);
        }
    }
}

template <class Op, bool VEC, int MODE>
__device__ __forceinline__ void dt_range(char* a, char* b, char* c, size_t lo, size_t len,
                                         unsigned mis, unsigned tile, bool fin, float nf,
                                         float inv) {
    constexpr int EB = Op::kElemBytes;
    const Span sp = make_span<EB, VEC>(lo, len, mis);
    const size_t ubase = (size_t)tile * (kThreads * kUnroll) + threadIdx.x;
    if (ubase < sp.units)
        dt_units<Op, VEC, MODE>(a, b, c, sp.body * EB, ubase, sp.units, fin, nf, inv);
    if constexpr (VEC) {
        if (tile == 0) {
            const unsigned t = threadIdx.x;
            if (t < sp.nhead)
                dt_units<Op, false, MODE>(a, b, c, (lo + t) * EB, 0, 1, fin, nf, inv);
            else if (t >= kTailLane && t - kTailLane < sp.ntail)
                dt_units<Op, false, MODE>(a, b, c, (sp.tail + (t - kTailLane)) * EB, 0, 1, fin,
                                          nf, inv);
        }
    }
}

__device__ __forceinline__ int dt_rank(int tree, int v, int n) {
    return tree == 0 ? v : ((v - 1) & (n - 1));
}

// One double-tree step; block b = (tree, node j, tile) with `tiles` tiles per node.
template <class Op, bool VEC>
__global__ __launch_bounds__(kThreads) void k_dtree_step(const Args a) {
    const int n = a.n;
    const int L = 31 - __builtin_clz((unsigned)n);
    const int s = a.step;
    const unsigned g = blockIdx.x / a.tiles;
    const unsigned tile = blockIdx.x - g * a.tiles;
    int lvl, mode;
    if (s < L - 1) { lvl = s + 1; mode = DT_REDUCE3; }
    else if (s == L - 1) { lvl = L; mode = DT_REDUCE2; }
    else if (s == L) { lvl = L; mode = DT_COPY1; }
    else { lvl = 2 * L - s; mode = DT_COPY2; }
    const unsigned nodes = (mode == DT_REDUCE3 || mode == DT_COPY2) ? (unsigned)(n >> (lvl + 1)) : 1u;
    const int tree = (int)(g / nodes);
    const int j = (int)(g - (unsigned)tree * nodes);
    const size_t half = (a.count + 1) / 2;
    const size_t lo = tree == 0 ? 0 : half;
    const size_t len = tree == 0 ? half : a.count - half;
    if (len == 0) return;
    if (mode == DT_REDUCE3 || mode == DT_COPY2) {
        const int v = (2 * j + 1) << lvl;
        const int hb = 1 << (lvl - 1);
        char* left = rank_ptr(a, dt_rank(tree, v - hb, n));
        char* own = rank_ptr(a, dt_rank(tree, v, n));
        char* right = rank_ptr(a, dt_rank(tree, v + hb, n));
        if (mode == DT_REDUCE3)
            dt_range<Op, VEC, DT_REDUCE3>(left, own, right, lo, len, a.mis, tile, false, a.nf,
                                          a.inv);
        else
            dt_range<Op, VEC, DT_COPY2>(left, own, right, lo, len, a.mis, tile, false, a.nf,
                                        a.inv);
    } else {
        char* root = rank_ptr(a, dt_rank(tree, 0, n));
        char* child = rank_ptr(a, dt_rank(tree, n / 2, n));
        if (mode == DT_REDUCE2)
            dt_range<Op, VEC, DT_REDUCE2>(nullptr, root, child, lo, len, a.mis, tile,
                                          a.avg != 0, a.nf, a.inv);
        else
            dt_range<Op, VEC, DT_COPY1>(nullptr, root, child, lo, len, a.mis, tile, false, a.nf,
                                        a.inv);
    }
}

template <class Op, bool VEC>
static hipError_t launch_step_op(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const dim3 block(kThreads);
    switch (p.kind) {
        case KIND_RS_STEP:
            hipLaunchKernelGGL((k_rs_step<Op, VEC>), grid, block, 0, s, a);
            break;
        case KIND_TREE_STEP:
            hipLaunchKernelGGL((k_tree_step<Op, VEC>), grid, block, 0, s, a);
            break;
        case KIND_HD_RS_STEP:
            hipLaunchKernelGGL((k_hd_rs_step<Op, VEC>), grid, block, 0, s, a);
            break;
        case KIND_DT_STEP:
            hipLaunchKernelGGL((k_dtree_step<Op, VEC>), grid, block, 0, s, a);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int EB, bool VEC>
static hipError_t launch_step_copy(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const dim3 block(kThreads);
    using Op = OpCopy<EB>;
    switch (p.kind) {
        case KIND_AG_STEP:
            hipLaunchKernelGGL((k_ag_step<Op, VEC>), grid, block, 0, s, a);
            break;
        case KIND_HD_AG_STEP:
            hipLaunchKernelGGL((k_hd_ag_step<Op, VEC>), grid, block, 0, s, a);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class Op>
static hipError_t launch_step_vec(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    return p.vec ? launch_step_op<Op, true>(p, a, grid, s) : launch_step_op<Op, false>(p, a, grid, s);
}

hipError_t launch_step_kind(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    if (p.kind == KIND_AG_STEP || p.kind == KIND_HD_AG_STEP) {
        if (elem_bytes(p.dtype) == 2)
            return p.vec ? launch_step_copy<2, true>(p, a, grid, s)
                         : launch_step_copy<2, false>(p, a, grid, s);
        return p.vec ? launch_step_copy<4, true>(p, a, grid, s)
                     : launch_step_copy<4, false>(p, a, grid, s);
    }
    const bool mx = p.op == AR_MAX;
    switch (p.dtype) {
        case AR_INT32:
            return mx ? launch_step_vec<OpI32Max>(p, a, grid, s) : launch_step_vec<OpI32Sum>(p, a, grid, s);
        case AR_FLOAT32:
            return mx ? launch_step_vec<OpF32Max>(p, a, grid, s) : launch_step_vec<OpF32Sum>(p, a, grid, s);
        case AR_BFLOAT16:
            return mx ? launch_step_vec<OpBF16Max>(p, a, grid, s)
                      : launch_step_vec<OpBF16Sum>(p, a, grid, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace arlib
