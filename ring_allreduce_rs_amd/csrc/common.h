// common.h -- shared device-side building blocks of the AllReduce kernels
// (gfx950): launch-shape constants, the kernel argument block, 16-byte /
// element-wise memory units and the head / body / tail split of a range.
#pragma once

#include "elem.h"
#include "launch.h"

namespace arlib {

constexpr int kThreads = 256;       // per-step kernels: 4 wavefronts of 64
constexpr int kUnroll = 2;          // per-step kernels: 16-byte units per lane per tile
constexpr int kFusedThreads = 64;   // fused kernels: one wavefront per block
constexpr int kFusedUnroll = 4;     // fused WIDE shape: 16-byte units per lane
constexpr int kBatch = 8;           // ranks of loads issued before they are folded
// Fused-kernel shapes (units of 16 bytes per lane, ranks of loads in flight
// before folding).  WIDE suits up to 16 ranks; with many ranks the fold would
// wait on memory N/8 times, so DEEP keeps 32 ranks of loads in flight (a
// 64-rank fold waits twice).  fused_variant() picks one.
constexpr size_t kTinyMaxChunkBytes = 4096;        // TINY: chunks up to 4 KiB, > 32 ranks
constexpr size_t kDeepMaxChunkBytes = 256u << 10;  // 9-16 ranks: DEEP up to 256 KiB chunks
struct FusedWide {
    static constexpr int U = kFusedUnroll;
    static constexpr int B = kBatch;
    static constexpr bool kWrapLoads = false;
};
struct FusedDeep {
    static constexpr int U = 1;
    static constexpr int B = 32;
    static constexpr bool kWrapLoads = false;
};
// PACED: WIDE's 8-rank batches with one unit per lane (8 KiB of loads per
// wave per batch instead of 32), launched with an LDS reservation that caps
// the waves resident on a CU (fused_waves_per_cu).  On calls that stream far
// more than one round of waves, fewer and smaller requests in flight keep
// HBM busier than the WIDE shape's 12 waves x 32 KiB per CU; on smaller
// calls WIDE's all-at-once issue wins (measurements at fused_variant).
struct FusedPaced {
    static constexpr int U = 1;
    static constexpr int B = kBatch;
    static constexpr bool kWrapLoads = false;
};
// TINY: element-wise units with every rank's load in flight at once (one
// memory round trip for up to 64 ranks instead of DEEP's two); for chunks so
// small that latency, not bandwidth, sets the time.
struct FusedTiny {
    static constexpr int U = 1;
    static constexpr int B = AR_MAX_RANKS;
    static constexpr bool kWrapLoads = true;
};
enum { CFG_WIDE = 0, CFG_DEEP = 1, CFG_TINY = 2, CFG_PACED = 3 };
// Residency caps apply to calls that touch more than these many bytes over
// all ranks (N x bytes per rank): PACED replaces WIDE above the first, and
// DEEP is capped above the second; the AllGather over more than 8 ranks
// takes PACED above the third.
constexpr size_t kPacedMinBytes = size_t(128) << 20;
constexpr size_t kDeepCapMinBytes = size_t(256) << 20;
constexpr size_t kAgPacedMinBytes = size_t(512) << 20;
// Dynamic LDS per one-wave block that lets at most `waves` blocks share a CU:
// kLdsBytesPerCU / (waves + 1/2), rounded down to 256 bytes (waves fit,
// waves + 1 do not, with about half a block's share of slack either way).
constexpr unsigned lds_for_waves(unsigned waves) {
    return waves == 0 ? 0u : (2u * kLdsBytesPerCU / (2u * waves + 1u)) & ~255u;
}
// The PACED cap of the ring SUM / AVG AllReduce, which the calibration
// stream shares.
constexpr unsigned kPacedRingWaves = 5;
constexpr int kTailLane = 32;       // first lane that handles a chunk's tail elements
constexpr size_t kLeadUnits = 7;    // most idle 16-byte units before a chunk body (128-byte lines)
// Streaming (non-temporal) loads and stores.  The fused kernel touches every
// byte once, so caching it only evicts useful lines: on MI355X 8 x 25 MiB went
// from 86 us to 77 us with both loads and stores streaming.  The per-step
// kernels are the opposite case: each step re-reads what the previous step
// wrote, and a 200 MiB working set stays in the 256 MB Infinity Cache when
// the stores are ordinary (ring 8 x 25 MiB: 169 us with, 189 us without).
constexpr bool kFusedNT = true;
constexpr bool kStepNT = false;
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
    // in-register folds: fold hop by hop, then canon once (LazyFold)
    __device__ static T fold(T a, T b) {
        if constexpr (LazyFold<Op>::value) return fold4<Op>(a, b);
        else return comb4<Op>(a, b);
    }
    __device__ static T canon(T a) {
        if constexpr (LazyFold<Op>::value) return canon4<Op>(a);
        else return a;
    }
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
    // (LazyFold ops have 4-byte elements: an element is a word)
    __device__ static T fold(T a, T b) {
        if constexpr (LazyFold<Op>::value) return Op::fold_word(a, b);
        else return Op::comb_elem(a, b);
    }
    __device__ static T canon(T a) {
        if constexpr (LazyFold<Op>::value) return Op::canon_word(a);
        else return a;
    }
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

inline int elem_bytes(ar_dtype d) { return d == AR_BFLOAT16 ? 2 : 4; }

inline size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }

// Which fused shape (CFG_*) a plan runs (host side; dispatch.hip).
int fused_variant(const Plan& p);
int fused_units_per_lane(int cfg);
// Waves of a fused launch allowed per CU (0: no cap), and the dynamic LDS
// bytes per block that enforce it (0: none).
unsigned fused_waves_per_cu(const Plan& p);
unsigned fused_lds_reserve(const Plan& p);

// Launchers, one per translation unit.
hipError_t launch_fused_kind(const Plan& p, const Args& a, dim3 grid, hipStream_t s);
hipError_t launch_fused_i32(const Plan& p, const Args& a, dim3 grid, hipStream_t s);
hipError_t launch_fused_f32(const Plan& p, const Args& a, dim3 grid, hipStream_t s);
hipError_t launch_fused_bf16(const Plan& p, const Args& a, dim3 grid, hipStream_t s);
// the same for plans with p.vec && p.lead (line-aligned tiles)
hipError_t launch_fused_i32_lead(const Plan& p, const Args& a, dim3 grid, hipStream_t s);
hipError_t launch_fused_f32_lead(const Plan& p, const Args& a, dim3 grid, hipStream_t s);
hipError_t launch_fused_bf16_lead(const Plan& p, const Args& a, dim3 grid, hipStream_t s);
hipError_t launch_step_kind(const Plan& p, const Args& a, dim3 grid, hipStream_t s);

}  // namespace arlib
