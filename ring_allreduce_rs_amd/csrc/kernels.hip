// kernels.hip -- HIP kernels of the ring / tree AllReduce for CDNA4 (gfx950).
//
// All N logical ranks are buffers in one GPU's HBM.  The path is pure
// streaming (about (N-1)/(8N) flop per byte for fp32), so every kernel is
// built around 16-byte coalesced loads and stores: consecutive lanes of a
// 64-wide wavefront touch consecutive 16 bytes of the same rank buffer.  No
// LDS, no MFMA -- nothing here is a contraction.
//
// Ring schedule (pwwt.cn page "Allreduce：大模型分布式训练的核心通信算法与优化实践",
// section 2.2, read as: ReduceScatter step k sends chunk (r-k-1) mod N from
// rank r to rank r+1; AllGather step k forwards chunk (r-k) mod N).  Chunk c
// is therefore folded over ranks c+1, c+2, ..., c-1, c, left to right, and
// ends on rank c.
//
// Kernels:
//   k_fused<MODE>  one pass; each lane loads one 16-byte unit from every rank
//                  (in ring order, kBatch ranks of loads in flight before the
//                  adds), folds them in order in registers, and stores the
//                  result to all N ranks (AllReduce), to the owner only
//                  (ReduceScatter) or copies the owner's unit to the others
//                  (AllGather).  Bitwise equal to the per-step ring because the
//                  fold order and per-hop rounding are the same.
//   k_rs_step      one ReduceScatter step: every rank's chunk folded into its
//                  successor's copy (AVG divide fused into the last step).
//   k_ag_step      one AllGather step: chunk copied to the successor.
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
//   k_copy         plain 16-byte copy, the bandwidth / counter calibration.
//
// Block -> work mapping: block b handles tile (b mod tiles) of chunk
// (b / tiles), so the chunk -- and with it the first rank of the fold and
// every rank pointer -- is uniform across the block and lives in scalar
// registers.  A chunk whose start is not 16-byte aligned (counts not divisible
// by N, e.g. 268,435,459 over 16 ranks) has a head of up to 15 bytes and a
// tail, handled element by element by lanes of the chunk's first tile.
#include "elem.h"
#include "launch.h"

namespace arlib {

#ifndef AR_FUSED_NT
#define AR_FUSED_NT 1
#endif
#ifndef AR_STEP_NT
#define AR_STEP_NT 0
#endif

#ifndef AR_FUSED_THREADS
#define AR_FUSED_THREADS 64
#endif
#ifndef AR_FUSED_UNROLL
#define AR_FUSED_UNROLL 4
#endif
#ifndef AR_SPECIALIZE_N
#define AR_SPECIALIZE_N 1
#endif

constexpr int kThreads = 256;       // per-step kernels: 4 wavefronts of 64
constexpr int kUnroll = 2;          // per-step kernels: 16-byte units per lane per tile
constexpr int kFusedThreads = AR_FUSED_THREADS;
constexpr int kFusedUnroll = AR_FUSED_UNROLL;
constexpr int kBatch = 8;           // ranks of loads issued before they are folded
constexpr int kTailLane = 32;       // first lane that handles a chunk's tail elements
// Streaming (non-temporal) loads and stores.  The fused kernel touches every
// byte once, so caching it only evicts useful lines: on MI355X 8 x 25 MiB went
// from 86 us to 77 us with both loads and stores streaming.  The per-step
// kernels are the opposite case: each step re-reads what the previous step
// wrote, and a 200 MiB working set stays in the 256 MB Infinity Cache when
// the stores are ordinary (ring 8 x 25 MiB: 169 us with, 189 us without).
constexpr bool kFusedNT = AR_FUSED_NT != 0;
constexpr bool kStepNT = AR_STEP_NT != 0;
constexpr int kCopyUnroll = 1;  // the plain copy streams best with one unit per lane

struct Args {
    RankTable t;
    size_t count;     // elements per rank
    size_t per;       // chunk length L = ceil(count / N)
    int n;            // ranks
    int step;         // step index (per-step kernels)
    unsigned tiles;   // tiles per chunk (per pair for the tree)
    unsigned mis;     // every buffer's address mod 16, in bytes
    int avg;          // 1: divide the finished sum by n
    float nf;         // (float)n
    float inv;        // 1/n when n is a power of two (exact), else 0
};

template <class Op, bool VEC, bool NT = false>
struct Unit;

template <class Op, bool NT>
struct Unit<Op, true, NT> {
    using T = u32x4;
    static constexpr int kBytes = 16;
    __device__ static T ld(const char* p) { return ld16<NT>(p); }
    __device__ static void st(char* p, T v) { st16<NT>(p, v); }
    __device__ static T comb(T a, T b) { return comb4<Op>(a, b); }
    __device__ static T fin(T a, float nf, float inv) { return finish4<Op>(a, nf, inv); }
    __device__ static T zero() { return u32x4{0u, 0u, 0u, 0u}; }
};

template <class Op, bool NT>
struct Unit<Op, false, NT> {
    using T = uint32_t;
    static constexpr int kBytes = Op::kElemBytes;
    __device__ static T ld(const char* p) { return ld_elem<Op::kElemBytes>(p); }
    __device__ static void st(char* p, T v) { st_elem<Op::kElemBytes>(p, v); }
    __device__ static T comb(T a, T b) { return Op::comb_elem(a, b); }
    __device__ static T fin(T a, float nf, float inv) { return Op::finish_elem(a, nf, inv); }
    __device__ static T zero() { return 0u; }
};

// Split the element range [lo, lo+len) into an element-wise head up to the
// first 16-byte boundary, a body of 16-byte units, and an element-wise tail.
struct Span {
    size_t body;     // first element of the body
    size_t units;    // body length in units
    size_t tail;     // first tail element
    unsigned nhead;  // head elements, starting at lo
    unsigned ntail;  // tail elements
};

template <int EB, bool VEC>
__device__ __forceinline__ Span make_span(size_t lo, size_t len, unsigned mis) {
    Span s;
    if constexpr (VEC) {
        constexpr int kEpu = 16 / EB;
        const unsigned m = (unsigned)((mis + lo * EB) & 15u);
        size_t h = m ? (16u - m) / EB : 0;
        if (h > len) h = len;
        s.nhead = (unsigned)h;
        s.body = lo + h;
        s.units = (len - h) / kEpu;
        s.tail = s.body + s.units * kEpu;
        s.ntail = (unsigned)(lo + len - s.tail);
    } else {
        s.nhead = 0;
        s.body = lo;
        s.units = len;
        s.tail = lo + len;
        s.ntail = 0;
    }
    return s;
}

__device__ __forceinline__ void chunk_bounds(const Args& a, int c, size_t& lo, size_t& len) {
    size_t b0 = (size_t)c * a.per;
    if (b0 > a.count) b0 = a.count;
    size_t b1 = b0 + a.per;
    if (b1 > a.count) b1 = a.count;
    lo = b0;
    len = b1 - b0;
}

__device__ __forceinline__ char* rank_ptr(const Args& a, int r) {
    return reinterpret_cast<char*>(a.t.p[r]);
}

// ---------------------------------------------------------------- fused ring

// Units ubase, ubase+kFusedThreads, ... (kFusedUnroll of them, bounded by
// `units`) of the range starting at byte offset byte0 in every rank buffer.
// NR > 0 fixes the rank count at compile time (loops fully unrolled); NR == 0
// reads it from the arguments.
template <class Op, int MODE, bool VEC, int NR>
__device__ __forceinline__ void fused_units(const Args& a, int c, int start, size_t byte0,
                                            size_t ubase, size_t units) {
    using X = Unit<Op, VEC, kFusedNT>;
    using T = typename X::T;
    constexpr int U = kFusedUnroll;
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
        for (int j0 = 0; j0 < (NR > 0 ? NR : AR_MAX_RANKS); j0 += kBatch) {
            if (NR == 0 && j0 >= n) break;
            T v[kBatch][U];
            int rr = r;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (j0 + j < n) {
                    const char* src = rank_ptr(a, rr);
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        v[j][u] = ok[u] ? X::ld(src + off[u]) : X::zero();
                    rr = (rr + 1 == n) ? 0 : rr + 1;
                }
            }
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
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

template <class Op, int MODE, bool VEC, int NR>
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
    const size_t ubase = (size_t)tile * (kFusedThreads * kFusedUnroll) + threadIdx.x;
    if (ubase < sp.units)
        fused_units<Op, MODE, VEC, NR>(a, c, start, sp.body * EB, ubase, sp.units);
    if constexpr (VEC) {
        // heads have at most 15 bytes (< 8 elements), as do tails
        if (tile == 0) {
            const unsigned t = threadIdx.x;
            if (t < sp.nhead)
                fused_units<Op, MODE, false, NR>(a, c, start, (lo + t) * EB, 0, 1);
            else if (t >= kTailLane && t - kTailLane < sp.ntail)
                fused_units<Op, MODE, false, NR>(a, c, start, (sp.tail + (t - kTailLane)) * EB,
                                                 0, 1);
        }
    }
}

// ---------------------------------------------------------------- per-step ring and tree

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

// ---------------------------------------------------------------- host side

static int elem_bytes(ar_dtype d) { return d == AR_BFLOAT16 ? 2 : 4; }

static size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }

bool plan_shape(const Plan& p, Shape* out) {
    const size_t eb = (size_t)elem_bytes(p.dtype);
    const size_t epu = p.vec ? 16 / eb : 1;
    const bool fused = p.kind == KIND_FUSED_AR || p.kind == KIND_FUSED_RS || p.kind == KIND_FUSED_AG;
    const size_t threads = fused ? kFusedThreads : kThreads;
    const size_t per_tile = threads * (fused ? kFusedUnroll : kUnroll);
    size_t tiles, groups;
    if (p.kind == KIND_TREE_STEP) {
        tiles = ceil_div(ceil_div(p.count, epu), per_tile);
        groups = (size_t)p.nranks / 2;
    } else if (p.kind == KIND_DT_STEP) {
        int L = 0;
        while ((1 << L) < p.nranks) ++L;
        const int s = p.step;
        size_t nodes = 1;
        if (s < L - 1) nodes = (size_t)p.nranks >> (s + 2);
        else if (s > L) nodes = (size_t)p.nranks >> (2 * L - s + 1);
        tiles = ceil_div(ceil_div((p.count + 1) / 2, epu), per_tile);
        groups = 2 * nodes;
    } else if (p.kind == KIND_HD_RS_STEP || p.kind == KIND_HD_AG_STEP) {
        // a step moves d consecutive chunks per rank
        const size_t per = ceil_div(p.count, (size_t)p.nranks);
        const size_t d = p.kind == KIND_HD_RS_STEP ? ((size_t)p.nranks >> (p.step + 1))
                                                   : ((size_t)1 << p.step);
        tiles = ceil_div(ceil_div(per * d, epu), per_tile);
        groups = (size_t)p.nranks;
    } else {
        const size_t per = ceil_div(p.count, (size_t)p.nranks);
        tiles = ceil_div(ceil_div(per, epu), per_tile);
        groups = (size_t)p.nranks;
    }
    if (tiles == 0) tiles = 1;
    const size_t blocks = tiles * groups;
    if (blocks == 0 || blocks > 0x7fffffffu || tiles > 0xffffffffu) return false;
    out->blocks = (unsigned)blocks;
    out->threads = (unsigned)threads;
    out->tiles = (unsigned)tiles;
    return true;
}

template <class Op, int MODE, bool VEC>
static void launch_fused(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const dim3 block(kFusedThreads);
    if (AR_SPECIALIZE_N && VEC && p.nranks == 8)
        hipLaunchKernelGGL((k_fused<Op, MODE, VEC, 8>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((k_fused<Op, MODE, VEC, 0>), grid, block, 0, s, a);
}

template <class Op, bool VEC>
static hipError_t launch_kind(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const dim3 block(kThreads);
    switch (p.kind) {
        case KIND_FUSED_AR:
            launch_fused<Op, KIND_FUSED_AR, VEC>(p, a, grid, s);
            break;
        case KIND_FUSED_RS:
            launch_fused<Op, KIND_FUSED_RS, VEC>(p, a, grid, s);
            break;
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
static hipError_t launch_copy_kind(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    const dim3 block(kThreads);
    using Op = OpCopy<EB>;
    switch (p.kind) {
        case KIND_FUSED_AG:
            hipLaunchKernelGGL((k_fused<Op, KIND_FUSED_AG, VEC, 0>), dim3(grid), dim3(kFusedThreads),
                               0, s, a);
            break;
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
static hipError_t launch_op(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    return p.vec ? launch_kind<Op, true>(p, a, grid, s) : launch_kind<Op, false>(p, a, grid, s);
}

hipError_t launch(const Plan& p, const RankTable& t, hipStream_t stream) {
    Shape sh;
    if (!plan_shape(p, &sh)) return hipErrorInvalidConfiguration;
    Args a;
    a.t = t;
    a.count = p.count;
    a.per = ceil_div(p.count, (size_t)p.nranks);
    a.n = p.nranks;
    a.step = p.step;
    a.tiles = sh.tiles;
    a.mis = p.mis;
    a.avg = p.op == AR_AVG ? 1 : 0;
    a.nf = (float)p.nranks;
    a.inv = (p.nranks & (p.nranks - 1)) == 0 ? 1.0f / (float)p.nranks : 0.0f;
    const dim3 grid(sh.blocks);

    if (p.kind == KIND_FUSED_AG || p.kind == KIND_AG_STEP || p.kind == KIND_HD_AG_STEP) {
        if (elem_bytes(p.dtype) == 2)
            return p.vec ? launch_copy_kind<2, true>(p, a, grid, stream)
                         : launch_copy_kind<2, false>(p, a, grid, stream);
        return p.vec ? launch_copy_kind<4, true>(p, a, grid, stream)
                     : launch_copy_kind<4, false>(p, a, grid, stream);
    }
    const bool mx = p.op == AR_MAX;
    switch (p.dtype) {
        case AR_INT32:
            return mx ? launch_op<OpI32Max>(p, a, grid, stream)
                      : launch_op<OpI32Sum>(p, a, grid, stream);
        case AR_FLOAT32:
            return mx ? launch_op<OpF32Max>(p, a, grid, stream)
                      : launch_op<OpF32Sum>(p, a, grid, stream);
        case AR_BFLOAT16:
            return mx ? launch_op<OpBF16Max>(p, a, grid, stream)
                      : launch_op<OpBF16Sum>(p, a, grid, stream);
    }
    return hipErrorInvalidValue;
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

}  // namespace arlib
