// launch.h -- internal interface between the C-ABI host layer (ar_api.cpp)
// and the HIP kernels (fused.hip, steps.hip, copy.hip, dispatch.hip).  Not
// part of the public ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "ar.h"

namespace arlib {

// The N rank pointers travel by value in the kernel arguments.
struct RankTable {
    void* p[AR_MAX_RANKS];
};

enum Kind {
    KIND_FUSED_AR = 0,   // fold every chunk in ring order, write all N ranks
    KIND_FUSED_RS = 1,   // fold chunk r in ring order, write rank r only
    KIND_FUSED_AG = 2,   // copy chunk r of rank r to every other rank
    KIND_RS_STEP = 3,    // one ReduceScatter step of the ring
    KIND_AG_STEP = 4,    // one AllGather step of the ring
    KIND_TREE_STEP = 5,  // one recursive-doubling step
    KIND_HD_RS_STEP = 6, // one recursive-halving ReduceScatter step
    KIND_HD_AG_STEP = 7, // one recursive-doubling AllGather step
    KIND_DT_STEP = 8,    // one double-binary-tree step (reduce up / broadcast down)
};

// Fold order of the one-pass kernels.  RING: chunk c is folded over ranks
// c+1, ..., c (the ring's order).  PAIR: a pairwise tree over ranks 0..N-1 in
// index order (recursive doubling's result).  PAIR_BITREV: the same tree over
// ranks in bit-reversed order, i.e. partners at distance N/2 first
// (recursive halving-doubling's result).  DTREE: the double binary tree's
// in-order folds, the first ceil(count/2) elements over tree 0 and the rest
// over tree 1 (the double tree's result); its "chunks" are those two halves.
// The tree orders need a power-of-two N.
enum Order { ORDER_RING = 0, ORDER_PAIR = 1, ORDER_PAIR_BITREV = 2, ORDER_DTREE = 3 };

// LDS per CU on gfx950: a block that reserves a little over 1/(W+1) of it
// leaves room for at most W such blocks (one wave each) on the CU.  The
// residency caps rely on it; a context whose device reports another size
// keeps them off.
constexpr unsigned kLdsBytesPerCU = 160u << 10;

// Parts the fused kernels split a rank's vector into: N chunks, or the double
// tree's two halves.
inline int fused_parts(int order, int nranks) { return order == ORDER_DTREE ? 2 : nranks; }

struct Plan {
    Kind kind;
    ar_dtype dtype;
    ar_op op;
    int nranks;
    size_t count;
    int step;           // step index for the *_STEP kinds
    bool vec;           // 16-byte path (all buffers share their address mod 16)
    unsigned mis;       // that common address mod 16, in bytes
    int order = ORDER_RING;   // fold order of the fused kinds (Order)
    // Fused kinds: some chunk body may start off a 128-byte line of rank 0's
    // buffer.  The kernel then shifts its tiles back to the line (up to 7 idle
    // 16-byte units at the front) and the grid carries that slack.
    bool lead = false;
    // Fused kinds: residency caps allowed (the PACED shape and the LDS
    // reservations); off, large calls run the uncapped shapes
    bool caps = true;
};

// Grid / block shape a plan launches with (for logging and tests).
struct Shape {
    unsigned blocks;
    unsigned threads;
    unsigned tiles;     // tiles per chunk (or per pair for the tree)
};

// Returns false if the plan cannot be launched (grid too large).
bool plan_shape(const Plan& p, Shape* out);

hipError_t launch(const Plan& p, const RankTable& t, hipStream_t stream);

// 16-byte vector copy of `bytes` (multiple of 16, both pointers 16-byte aligned).
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

// Calibration stream: read `bytes` from each of nsrc buffers, write their XOR
// to each of ndst buffers (16-byte aligned pointers, bytes a multiple of 16),
// in the shape the fused AllReduce of the sources would run (`caps`: residency
// caps allowed).
hipError_t launch_stream(const void* const* src, int nsrc, void* const* dst, int ndst,
                         size_t bytes, bool caps, hipStream_t stream);

// The same stream in place over n buffers (each read, then written), in the
// PACED shape with `lds` bytes of dynamic LDS per block, recording block b's
// start and end on the device's real-time counter in ts[2b] and ts[2b + 1]
// (ts holds 2 * ceil(bytes / 1024) entries).
hipError_t launch_stream_timeline(void* const* bufs, int n, size_t bytes, unsigned lds,
                                  unsigned long long* ts, hipStream_t stream);

// On-device result checker (check.hip): pass 1 writes one partial record per
// block (at most kCheckMaxBlocks) to `part`, pass 2 folds them into `out`.
constexpr int kCheckThreads = 256;
constexpr unsigned kCheckMaxBlocks = AR_CHECK_MAX_RECORDS;
struct CheckArgs {
    RankTable t;
    size_t count;
    int n;
    int dtype;           // ar_dtype
    int eb;              // element bytes
    const double* ref;   // NULL: no error check
    const double* bound; // NULL: no bound check (needs ref)
};
struct CheckPartial {
    unsigned long long mismatched;
    unsigned long long first;
    unsigned long long over;
    double max_err;
    unsigned nan;
    unsigned pad;
};
unsigned check_blocks(size_t count);   // blocks of pass 1 (partial records written)
// The device address of the device-resident scratch (kCheckMaxBlocks
// records) on `device`, which must be current; looked up once per device.
hipError_t check_static_scratch(int device, CheckPartial** out);
hipError_t launch_check(const CheckArgs& a, CheckPartial* part, ar_check_result* out,
                        hipStream_t s);

}  // namespace arlib
