// ar_api.cpp -- the C ABI declared in include/ar.h: argument validation,
// chunk layout, algorithm dispatch, the cost model behind AR_ALGO_AUTO and
// error reporting.  Kernels live in fused.hip and steps.hip; this file only
// decides what to launch, in which order, on the context's stream.
//
// The ring AllReduce is ReduceScatter (N-1 steps) followed by AllGather (N-1
// steps) ("AllReduce 集合通信", zzmblog.top, sections 语义 and 两阶段流程); the
// tree is recursive doubling in log2 N steps ("集合通信基础AllReduce、Ring算法与
// NCCL全解析", section 4.1).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "ar.h"
#include "launch.h"
#include "probe.h"

// A pointer set that passed the device-memory checks, with the byte size it
// was checked for.
struct CheckedSet {
    std::vector<uintptr_t> ptrs;
    size_t bytes = 0;
    uint64_t stamp = 0;
};

// A recorded launch sequence.  `done` is recorded after every replay so the
// executable graph can be released only once its last replay has finished.
struct GraphEntry {
    std::vector<uint64_t> key;
    hipGraphExec_t exec = nullptr;
    hipEvent_t done = nullptr;
    uint64_t stamp = 0;
};

static constexpr size_t kGraphCacheSize = 64;

struct ar_ctx {
    int device = 0;
    hipStream_t stream = nullptr;
    std::string last_error;
    // Recently validated pointer sets (least recently used is replaced): a
    // training loop reduces the same few buckets every step, and checking 64
    // pointers with the runtime costs more than a small message's kernel.
    // Off unless the caller turns it on (ar_set_pointer_cache): a buffer freed
    // and re-allocated smaller at the same address would not be re-checked.
    bool ptr_cache = false;
    std::vector<CheckedSet> checked;
    // Residency caps of the fused kernels (ar_set_residency_caps): on unless
    // the caller turns them off or the device's LDS per CU is not the size
    // they are computed for
    bool caps = true;
    bool caps_supported = true;
    uint64_t clock = 0;
    // Graph replay of multi-launch collectives (ar_set_graphs): one
    // instantiated graph per (collective, algorithm, shape, pointer set),
    // recorded on a private stream and launched on `stream`.
    size_t graph_max_bytes = 0;   // replay collectives of at most this many bytes per rank
    hipStream_t capture = nullptr;
    std::vector<GraphEntry> graph_cache;
    // ar_check's per-block partial records (kCheckMaxBlocks of them),
    // allocated on the first ar_check
    arlib::CheckPartial* check_part = nullptr;
    // ar_check_noalloc's records: the device-resident array on this
    // context's device, looked up in ar_create (NULL if that failed)
    arlib::CheckPartial* check_static = nullptr;
    std::string check_static_error;
};

static constexpr size_t kCheckedSets = 32;

namespace {

thread_local std::string g_create_error;

bool debug_enabled() {
    static const bool on = [] {
        const char* v = std::getenv("AR_DEBUG");
        return v && *v && std::strcmp(v, "0") != 0;
    }();
    return on;
}

ar_status fail(ar_ctx* ctx, ar_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    if (ctx) ctx->last_error = buf;
    else g_create_error = buf;
    if (debug_enabled()) std::fprintf(stderr, "[ar] error: %s\n", buf);
    return st;
}

size_t elem_bytes(ar_dtype d) { return d == AR_BFLOAT16 ? 2 : 4; }

bool valid_dtype(int d) { return d == AR_INT32 || d == AR_FLOAT32 || d == AR_BFLOAT16; }
bool valid_op(int o) { return o == AR_SUM || o == AR_MAX || o == AR_AVG; }
bool valid_algo(int a) { return a >= AR_ALGO_RING_STEP && a <= AR_ALGO_DOUBLE_TREE_FUSED; }
// algorithms defined for power-of-two rank counts only
bool needs_pow2(int a) {
    return a == AR_ALGO_TREE || a == AR_ALGO_HALVING_DOUBLING || a == AR_ALGO_DOUBLE_TREE ||
           a == AR_ALGO_TREE_FUSED || a == AR_ALGO_HALVING_DOUBLING_FUSED ||
           a == AR_ALGO_DOUBLE_TREE_FUSED;
}
// algorithms that exist as AllReduce only
bool allreduce_only(int a) {
    return a == AR_ALGO_TREE || a == AR_ALGO_DOUBLE_TREE || a == AR_ALGO_TREE_FUSED ||
           a == AR_ALGO_DOUBLE_TREE_FUSED;
}
int log2_exact(int n) {
    int l = 0;
    while ((1 << l) < n) ++l;
    return l;
}
bool pow2(int n) { return n > 0 && (n & (n - 1)) == 0; }

// Makes ctx->device current for the lifetime of the guard.
struct DeviceGuard {
    int prev = -1;
    bool ok = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) {
            (void)hipGetLastError();
            return;
        }
        ok = prev == dev || hipSetDevice(dev) == hipSuccess;
        if (!ok) (void)hipGetLastError();
    }
    ~DeviceGuard() {
        int cur = -1;
        if (ok && hipGetDevice(&cur) == hipSuccess && cur != prev && prev >= 0)
            (void)hipSetDevice(prev);
    }
};

// ---------------------------------------------------------------- cost model
//
// T = t_call + launches * alpha + bytes / BW.  Fitted on MI355X (8 and 64
// ranks, fp32, 4 KiB .. 64 MiB per rank, inputs cold in HBM for >= 1 MiB):
//   t_call   host validation + first dispatch of a call
//   alpha    each further dependent launch (the per-step kernels wait for the
//            previous step)
//   BW       bytes-moved rate of each kernel family; the per-step kernels
//            re-read what the previous step wrote, partly from the Infinity
//            Cache, so their rate can exceed a cold stream's; the fused pass
//            slows as the number of concurrently written rank buffers grows
//            (its rates are those of the residency-capped kernels: 8 ranks
//            6.25 TB/s over 50 MB - 6.7 GB, 16 ranks 6.0-6.3, 32-64 ranks
//            5.6-6.1).
constexpr double kCallUs = 8.0;
constexpr double kLaunchUs = 3.4;
constexpr double kStepGBps = 6000.0;
constexpr double kTreeGBps = 5400.0;

double fused_gbps(int n) { return n <= 8 ? 6250.0 : n <= 16 ? 6000.0 : 5700.0; }

int log2_ceil(int n) {
    int l = 0;
    while ((1 << l) < n) ++l;
    return l;
}

double predict_allreduce_us(int algo, int n, size_t count, size_t eb) {
    const double k = (double)count * (double)eb;   // bytes per rank
    if (n == 1 || count == 0) return kCallUs;
    switch (algo) {
        case AR_ALGO_RING_FUSED:
        case AR_ALGO_TREE_FUSED:
        case AR_ALGO_HALVING_DOUBLING_FUSED:
        case AR_ALGO_DOUBLE_TREE_FUSED:
            return kCallUs + 2.0 * n * k / (fused_gbps(n) * 1e3);
        case AR_ALGO_RING_STEP:
            return kCallUs + (2.0 * (n - 1) - 1) * kLaunchUs + 5.0 * (n - 1) * k / (kStepGBps * 1e3);
        case AR_ALGO_HALVING_DOUBLING:
            return kCallUs + (2.0 * log2_ceil(n) - 1) * kLaunchUs +
                   5.0 * (n - 1) * k / (kStepGBps * 1e3);
        case AR_ALGO_TREE:
            return kCallUs + (log2_ceil(n) - 1) * kLaunchUs +
                   2.0 * n * k * log2_ceil(n) / (kTreeGBps * 1e3);
        case AR_ALGO_DOUBLE_TREE:
            // per tree (half the vector, H = K/2): N/2-1 interior nodes read 3H and
            // write H going up and read H / write 2H going down; the root steps
            // move 3H and 2H.  Both trees: (7 (N/2 - 1) + 5) K.
            return kCallUs + (2.0 * log2_ceil(n) - 1) * kLaunchUs +
                   (7.0 * (n / 2 - 1) + 5.0) * k / (kStepGBps * 1e3);
    }
    return 1e300;
}

// The argmin over every algorithm; ties keep the earlier candidate.  The
// one-pass forms share one prediction (one launch, 2NK bytes), so the fused
// ring, listed first, takes every tie: on MI355X the one-pass tree orders
// measured within 3 % of it either way, less than the spread between machines.
int auto_algo(int n, size_t count, size_t eb) {
    int best = AR_ALGO_RING_FUSED;
    double best_us = predict_allreduce_us(best, n, count, eb);
    const int cands[] = {AR_ALGO_TREE_FUSED,       AR_ALGO_HALVING_DOUBLING_FUSED,
                         AR_ALGO_DOUBLE_TREE_FUSED, AR_ALGO_RING_STEP,
                         AR_ALGO_HALVING_DOUBLING, AR_ALGO_TREE,
                         AR_ALGO_DOUBLE_TREE};
    for (int a : cands) {
        if (a != AR_ALGO_RING_STEP && !pow2(n)) continue;
        const double t = predict_allreduce_us(a, n, count, eb);
        if (t < best_us) {
            best_us = t;
            best = a;
        }
    }
    return best;
}

// Validates everything that can be checked without touching the data.  On
// success *vec and *mis describe the common 16-byte alignment of the buffers.
ar_status check_buffers(ar_ctx* ctx, void* const* bufs, int nranks, size_t count, int dtype,
                        bool* vec, unsigned* mis) {
    if (!bufs) return fail(ctx, AR_ERR_INVALID_ARG, "bufs is NULL");
    if (nranks < 1 || nranks > AR_MAX_RANKS)
        return fail(ctx, AR_ERR_INVALID_ARG, "nranks %d outside [1, %d]", nranks, AR_MAX_RANKS);
    if (!valid_dtype(dtype)) return fail(ctx, AR_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    const size_t eb = elem_bytes((ar_dtype)dtype);
    if (count > SIZE_MAX / eb / 2)
        return fail(ctx, AR_ERR_INVALID_ARG, "count %zu overflows the byte size", count);
    *vec = true;
    *mis = 0;
    if (count == 0) return AR_OK;
    const size_t bytes = count * eb;
    std::vector<std::pair<uintptr_t, int>> spans;
    spans.reserve((size_t)nranks);
    for (int r = 0; r < nranks; ++r) {
        const uintptr_t p = reinterpret_cast<uintptr_t>(bufs[r]);
        if (!p) return fail(ctx, AR_ERR_INVALID_ARG, "bufs[%d] is NULL", r);
        if (p % eb) return fail(ctx, AR_ERR_INVALID_ARG, "bufs[%d] is not %zu-byte aligned", r, eb);
        if (p > UINTPTR_MAX - bytes)
            return fail(ctx, AR_ERR_INVALID_ARG, "bufs[%d] + size wraps the address space", r);
        spans.emplace_back(p, r);
    }
    std::sort(spans.begin(), spans.end());
    for (size_t i = 1; i < spans.size(); ++i) {
        if (spans[i - 1].first + bytes > spans[i].first)
            return fail(ctx, AR_ERR_INVALID_ARG, "bufs[%d] and bufs[%d] overlap",
                        spans[i - 1].second, spans[i].second);
    }
    const unsigned m0 = (unsigned)(reinterpret_cast<uintptr_t>(bufs[0]) & 15u);
    for (int r = 1; r < nranks; ++r)
        if ((unsigned)(reinterpret_cast<uintptr_t>(bufs[r]) & 15u) != m0) *vec = false;
    *mis = *vec ? m0 : 0;

    // Device-memory checks: every buffer must be device memory of ctx->device
    // and lie inside its allocation.  With the pointer cache on, passing sets
    // are remembered (see ar_ctx).
    for (CheckedSet& cs : ctx->checked) {
        if (!ctx->ptr_cache) break;
        if (cs.ptrs.size() != (size_t)nranks || bytes > cs.bytes) continue;
        bool same = true;
        for (int r = 0; same && r < nranks; ++r)
            same = cs.ptrs[(size_t)r] == reinterpret_cast<uintptr_t>(bufs[r]);
        if (same) {
            cs.stamp = ++ctx->clock;
            return AR_OK;
        }
    }
    for (int r = 0; r < nranks; ++r) {
        hipPointerAttribute_t at;
        std::memset(&at, 0, sizeof at);
        if (hipPointerGetAttributes(&at, bufs[r]) != hipSuccess) {
            (void)hipGetLastError();
            return fail(ctx, AR_ERR_INVALID_ARG, "bufs[%d] is not a device pointer", r);
        }
        if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged)
            return fail(ctx, AR_ERR_INVALID_ARG, "bufs[%d] is not device memory (type %d)", r,
                        (int)at.type);
        if (at.device != ctx->device)
            return fail(ctx, AR_ERR_INVALID_ARG, "bufs[%d] lives on device %d, context on %d", r,
                        at.device, ctx->device);
        // fail closed: a buffer whose extent cannot be established is refused
        hipDeviceptr_t base = nullptr;
        size_t size = 0;
        if (hipMemGetAddressRange(&base, &size, bufs[r]) != hipSuccess || !base) {
            (void)hipGetLastError();
            return fail(ctx, AR_ERR_INVALID_ARG, "bufs[%d]: cannot determine its allocation", r);
        }
        const uintptr_t b = reinterpret_cast<uintptr_t>(base);
        const uintptr_t p = reinterpret_cast<uintptr_t>(bufs[r]);
        if (p < b || p + bytes > b + size)
            return fail(ctx, AR_ERR_INVALID_ARG,
                        "bufs[%d]: %zu bytes run past the end of its allocation", r, bytes);
    }
    if (!ctx->ptr_cache) return AR_OK;
    CheckedSet entry;
    entry.ptrs.resize((size_t)nranks);
    for (int r = 0; r < nranks; ++r) entry.ptrs[(size_t)r] = reinterpret_cast<uintptr_t>(bufs[r]);
    entry.bytes = bytes;
    entry.stamp = ++ctx->clock;
    if (ctx->checked.size() < kCheckedSets) {
        ctx->checked.push_back(std::move(entry));
    } else {
        size_t oldest = 0;
        for (size_t i = 1; i < ctx->checked.size(); ++i)
            if (ctx->checked[i].stamp < ctx->checked[oldest].stamp) oldest = i;
        ctx->checked[oldest] = std::move(entry);
    }
    return AR_OK;
}

// A device array of `bytes` bytes at p: device memory of ctx->device, inside
// its allocation (fail closed, like the rank buffers).
ar_status check_device_span(ar_ctx* ctx, const void* p, size_t bytes, const char* what) {
    hipPointerAttribute_t at;
    std::memset(&at, 0, sizeof at);
    if (hipPointerGetAttributes(&at, p) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, AR_ERR_INVALID_ARG, "%s is not a device pointer", what);
    }
    if (at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeManaged)
        return fail(ctx, AR_ERR_INVALID_ARG, "%s is not device memory", what);
    if (at.device != ctx->device)
        return fail(ctx, AR_ERR_INVALID_ARG, "%s lives on device %d, context on %d", what,
                    at.device, ctx->device);
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess || !base) {
        (void)hipGetLastError();
        return fail(ctx, AR_ERR_INVALID_ARG, "%s: cannot determine its allocation", what);
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    if (q < b || bytes > size || q - b > size - bytes)
        return fail(ctx, AR_ERR_INVALID_ARG, "%s: %zu bytes run past the end of its allocation",
                    what, bytes);
    return AR_OK;
}

ar_status run(ar_ctx* ctx, hipStream_t stream, const arlib::Plan& p, const arlib::RankTable& t) {
    if (debug_enabled()) {
        arlib::Shape sh{};
        arlib::plan_shape(p, &sh);
        std::fprintf(stderr,
                     "[ar] kind=%d dtype=%d op=%d n=%d count=%zu step=%d vec=%d mis=%u "
                     "grid=%u tiles=%u threads=%u\n",
                     (int)p.kind, (int)p.dtype, (int)p.op, p.nranks, p.count, p.step, (int)p.vec,
                     p.mis, sh.blocks, sh.tiles, sh.threads);
    }
    const hipError_t e = arlib::launch(p, t, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, AR_ERR_RUNTIME, "kernel launch failed: %s", hipGetErrorString(e));
    }
    return AR_OK;
}

arlib::RankTable table_of(void* const* bufs, int nranks) {
    arlib::RankTable t;
    std::memset(&t, 0, sizeof t);
    for (int r = 0; r < nranks; ++r) t.p[r] = bufs[r];
    return t;
}

arlib::Plan make_plan(arlib::Kind k, int dtype, int op, int nranks, size_t count, int step,
                      bool vec, unsigned mis, int order = arlib::ORDER_RING) {
    arlib::Plan p;
    p.kind = k;
    p.dtype = (ar_dtype)dtype;
    p.op = (ar_op)op;
    p.nranks = nranks;
    p.count = count;
    p.step = step;
    p.vec = vec;
    p.mis = mis;
    p.order = order;
    return p;
}

ar_status check_op(ar_ctx* ctx, int dtype, int op) {
    if (!valid_op(op)) return fail(ctx, AR_ERR_INVALID_ARG, "unknown op %d", op);
    if (op == AR_AVG && dtype == AR_INT32)
        return fail(ctx, AR_ERR_UNSUPPORTED, "AVG is defined for float32 and bfloat16 only");
    return AR_OK;
}

// The collective entry points share this body.
enum Coll { COLL_AR, COLL_RS, COLL_AG };

// A validated collective: everything its launch sequence depends on.
struct Launch {
    Coll coll;
    int algo;   // resolved (never AUTO)
    int dtype;
    int op;     // AR_SUM for AllGather
    int nranks;
    size_t count;
    bool vec;
    unsigned mis;
    arlib::RankTable t;
    bool caps;   // residency caps allowed (the fused kinds)
};

// The kernels of L, in launch order.
std::vector<arlib::Plan> plans_of(const Launch& L) {
    std::vector<arlib::Plan> ps;
    // a chunk body can start off a 128-byte line unless rank 0's buffer and
    // every chunk start are line-aligned (then the fused grid needs no slack)
    const size_t parts = (size_t)arlib::fused_parts(
        L.algo == AR_ALGO_DOUBLE_TREE_FUSED ? arlib::ORDER_DTREE : arlib::ORDER_RING, L.nranks);
    const size_t chunk_bytes = (L.count + parts - 1) / parts * (size_t)elem_bytes((ar_dtype)L.dtype);
    const bool lines = (reinterpret_cast<uintptr_t>(L.t.p[0]) & 127u) == 0 && chunk_bytes % 128 == 0;
    auto add = [&](arlib::Kind k, int st, int order = arlib::ORDER_RING) {
        ps.push_back(make_plan(k, L.dtype, L.op, L.nranks, L.count, st, L.vec, L.mis, order));
        const bool fused = k == arlib::KIND_FUSED_AR || k == arlib::KIND_FUSED_RS ||
                           k == arlib::KIND_FUSED_AG;
        ps.back().lead = fused && L.vec && !lines;
        ps.back().caps = L.caps;
    };
    const arlib::Kind fused = L.coll == COLL_AR   ? arlib::KIND_FUSED_AR
                              : L.coll == COLL_RS ? arlib::KIND_FUSED_RS
                                                  : arlib::KIND_FUSED_AG;
    const int levels = log2_exact(L.nranks);
    const bool rs = L.coll != COLL_AG, ag = L.coll != COLL_RS;
    switch (L.algo) {
        case AR_ALGO_RING_FUSED:
            add(fused, 0);
            break;
        case AR_ALGO_TREE_FUSED:
            add(fused, 0, arlib::ORDER_PAIR);
            break;
        case AR_ALGO_HALVING_DOUBLING_FUSED:
            // the AllGather half is a copy, whatever the order
            add(fused, 0, L.coll == COLL_AG ? arlib::ORDER_RING : arlib::ORDER_PAIR_BITREV);
            break;
        case AR_ALGO_DOUBLE_TREE_FUSED:
            add(fused, 0, arlib::ORDER_DTREE);
            break;
        case AR_ALGO_HALVING_DOUBLING:
            if (rs) for (int st = 0; st < levels; ++st) add(arlib::KIND_HD_RS_STEP, st);
            if (ag) for (int st = 0; st < levels; ++st) add(arlib::KIND_HD_AG_STEP, st);
            break;
        case AR_ALGO_DOUBLE_TREE:
            for (int st = 0; st < 2 * levels; ++st) add(arlib::KIND_DT_STEP, st);
            break;
        case AR_ALGO_TREE:
            for (int st = 0; st < levels; ++st) add(arlib::KIND_TREE_STEP, st);
            break;
        default:
            if (rs) for (int k = 0; k <= L.nranks - 2; ++k) add(arlib::KIND_RS_STEP, k);
            if (ag) for (int k = 0; k <= L.nranks - 2; ++k) add(arlib::KIND_AG_STEP, k);
            break;
    }
    return ps;
}

// Every kernel of L must fit one grid; checked before anything is launched.
ar_status check_shapes(ar_ctx* ctx, const std::vector<arlib::Plan>& ps) {
    for (const arlib::Plan& p : ps) {
        arlib::Shape sh;
        if (!arlib::plan_shape(p, &sh))
            return fail(ctx, AR_ERR_INVALID_ARG, "count %zu needs more blocks than one grid holds",
                        p.count);
    }
    return AR_OK;
}

// Enqueues the kernels of L on `stream`, in order.
ar_status enqueue(ar_ctx* ctx, hipStream_t stream, const Launch& L) {
    for (const arlib::Plan& p : plans_of(L)) {
        const ar_status s = run(ctx, stream, p, L.t);
        if (s != AR_OK) return s;
    }
    return AR_OK;
}

// ------------------------------------------------------------ graph replay
//
// A multi-launch collective pays the launch and inter-kernel gap once per
// step.  With graphs enabled the launch sequence is recorded once on a
// private stream into a HIP graph (the kernel arguments, pointer table
// included, are baked in) and later calls of the same collective on the same
// buffers replay it with one hipGraphLaunch.  Results are identical: the same
// kernels run in the same order.

std::vector<uint64_t> key_of(const Launch& L) {
    std::vector<uint64_t> k;
    k.reserve(8 + (size_t)L.nranks);
    k.push_back((uint64_t)L.coll);
    k.push_back((uint64_t)L.algo);
    k.push_back((uint64_t)L.dtype);
    k.push_back((uint64_t)L.op);
    k.push_back((uint64_t)L.nranks);
    k.push_back((uint64_t)L.count);
    k.push_back((uint64_t)L.vec);
    k.push_back((uint64_t)L.mis);
    k.push_back((uint64_t)L.caps);
    for (int r = 0; r < L.nranks; ++r) k.push_back(reinterpret_cast<uint64_t>(L.t.p[r]));
    return k;
}

// Waits for the entry's last replay, then frees it.
void release(GraphEntry& e) {
    if (e.done) {
        (void)hipEventSynchronize(e.done);
        (void)hipEventDestroy(e.done);
    }
    if (e.exec) (void)hipGraphExecDestroy(e.exec);
    (void)hipGetLastError();
    e.done = nullptr;
    e.exec = nullptr;
}

ar_status record(ar_ctx* ctx, const Launch& L, GraphEntry* out) {
    if (!ctx->capture &&
        hipStreamCreateWithFlags(&ctx->capture, hipStreamNonBlocking) != hipSuccess) {
        (void)hipGetLastError();
        ctx->capture = nullptr;
        return fail(ctx, AR_ERR_RUNTIME, "cannot create the capture stream");
    }
    hipError_t e = hipStreamBeginCapture(ctx->capture, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, AR_ERR_RUNTIME, "hipStreamBeginCapture: %s", hipGetErrorString(e));
    }
    const ar_status s = enqueue(ctx, ctx->capture, L);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(ctx->capture, &graph);
    if (s != AR_OK || e != hipSuccess || !graph) {
        if (graph) (void)hipGraphDestroy(graph);
        (void)hipGetLastError();
        if (s != AR_OK) return s;
        return fail(ctx, AR_ERR_RUNTIME, "hipStreamEndCapture: %s", hipGetErrorString(e));
    }
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess || !exec) {
        (void)hipGetLastError();
        return fail(ctx, AR_ERR_RUNTIME, "hipGraphInstantiate: %s", hipGetErrorString(e));
    }
    hipEvent_t done = nullptr;
    if (hipEventCreateWithFlags(&done, hipEventDisableTiming) != hipSuccess) {
        (void)hipGetLastError();
        (void)hipGraphExecDestroy(exec);
        return fail(ctx, AR_ERR_RUNTIME, "cannot create a graph event");
    }
    out->key = key_of(L);
    out->exec = exec;
    out->done = done;
    return AR_OK;
}

ar_status replay(ar_ctx* ctx, const Launch& L) {
    // A stream that is itself being captured (the caller builds its own
    // graph) gets the kernels directly, so they land in the caller's graph.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(ctx->stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return enqueue(ctx, ctx->stream, L);
    }
    if (cs != hipStreamCaptureStatusNone) return enqueue(ctx, ctx->stream, L);

    const std::vector<uint64_t> key = key_of(L);
    GraphEntry* hit = nullptr;
    for (GraphEntry& e : ctx->graph_cache)
        if (e.key == key) {
            hit = &e;
            break;
        }
    if (!hit) {
        GraphEntry fresh;
        const ar_status s = record(ctx, L, &fresh);
        if (s != AR_OK) return s;
        if (ctx->graph_cache.size() < kGraphCacheSize) {
            ctx->graph_cache.push_back(std::move(fresh));
            hit = &ctx->graph_cache.back();
        } else {
            size_t oldest = 0;
            for (size_t i = 1; i < ctx->graph_cache.size(); ++i)
                if (ctx->graph_cache[i].stamp < ctx->graph_cache[oldest].stamp) oldest = i;
            release(ctx->graph_cache[oldest]);
            ctx->graph_cache[oldest] = std::move(fresh);
            hit = &ctx->graph_cache[oldest];
        }
    }
    hit->stamp = ++ctx->clock;
    hipError_t e = hipGraphLaunch(hit->exec, ctx->stream);
    if (e == hipSuccess) e = hipEventRecord(hit->done, ctx->stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, AR_ERR_RUNTIME, "hipGraphLaunch: %s", hipGetErrorString(e));
    }
    return AR_OK;
}

void clear_graphs(ar_ctx* ctx) {
    for (GraphEntry& e : ctx->graph_cache) release(e);
    ctx->graph_cache.clear();
}

ar_status collective(ar_ctx* ctx, Coll coll, void* const* bufs, int nranks, size_t count,
                     int dtype, int op, int algo) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    try {
        if (!valid_algo(algo)) return fail(ctx, AR_ERR_INVALID_ARG, "unknown algo %d", algo);
        if (coll != COLL_AG) {
            const ar_status s = check_op(ctx, dtype, op);
            if (s != AR_OK && valid_dtype(dtype)) return s;
        }
        bool vec = true;
        unsigned mis = 0;
        ar_status s = check_buffers(ctx, bufs, nranks, count, dtype, &vec, &mis);
        if (s != AR_OK) return s;
        if (algo == AR_ALGO_AUTO) {
            // ReduceScatter / AllGather alone follow the AllReduce choice, minus TREE
            algo = auto_algo(nranks, count, elem_bytes((ar_dtype)dtype));
            if (allreduce_only(algo) && coll != COLL_AR) algo = AR_ALGO_RING_FUSED;
            if (debug_enabled()) std::fprintf(stderr, "[ar] AUTO -> algo %d\n", algo);
        }
        if (allreduce_only(algo) && coll != COLL_AR)
            return fail(ctx, AR_ERR_UNSUPPORTED,
                        "TREE, TREE_FUSED, DOUBLE_TREE and DOUBLE_TREE_FUSED are AllReduce "
                        "algorithms; use "
                        "RING_STEP, RING_FUSED, HALVING_DOUBLING or HALVING_DOUBLING_FUSED");
        if (needs_pow2(algo) && !pow2(nranks))
            return fail(ctx, AR_ERR_UNSUPPORTED, "algo %d needs a power-of-two nranks, got %d",
                        algo, nranks);
        if (count == 0 || nranks == 1) return AR_OK;
        const Launch L{coll, algo, dtype, coll == COLL_AG ? AR_SUM : op, nranks, count, vec, mis,
                       table_of(bufs, nranks), ctx->caps};
        const std::vector<arlib::Plan> plans = plans_of(L);
        s = check_shapes(ctx, plans);
        if (s != AR_OK) return s;

        DeviceGuard g(ctx->device);
        if (!g.ok) return fail(ctx, AR_ERR_RUNTIME, "cannot select device %d", ctx->device);
        if (count * elem_bytes((ar_dtype)dtype) <= ctx->graph_max_bytes && plans.size() > 1)
            return replay(ctx, L);
        return enqueue(ctx, ctx->stream, L);
    } catch (const std::bad_alloc&) {
        return fail(ctx, AR_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(ctx, AR_ERR_RUNTIME, "unexpected exception");
    }
}

ar_status single_step(ar_ctx* ctx, arlib::Kind kind, void* const* bufs, int nranks, size_t count,
                      int dtype, int op, int step) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    try {
        if (kind != arlib::KIND_AG_STEP && kind != arlib::KIND_HD_AG_STEP) {
            const ar_status s = check_op(ctx, dtype, op);
            if (s != AR_OK && valid_dtype(dtype)) return s;
        }
        bool vec = true;
        unsigned mis = 0;
        ar_status s = check_buffers(ctx, bufs, nranks, count, dtype, &vec, &mis);
        if (s != AR_OK) return s;
        int nsteps = nranks - 1;
        if (kind == arlib::KIND_TREE_STEP || kind == arlib::KIND_HD_RS_STEP ||
            kind == arlib::KIND_HD_AG_STEP || kind == arlib::KIND_DT_STEP) {
            if (!pow2(nranks))
                return fail(ctx, AR_ERR_UNSUPPORTED,
                            "this step needs a power-of-two nranks, got %d", nranks);
            nsteps = log2_exact(nranks) * (kind == arlib::KIND_DT_STEP ? 2 : 1);
        }
        if (step < 0 || step >= nsteps)
            return fail(ctx, AR_ERR_INVALID_ARG, "step %d outside [0, %d)", step, nsteps);
        if (count == 0) return AR_OK;
        const int o = (kind == arlib::KIND_AG_STEP || kind == arlib::KIND_HD_AG_STEP) ? AR_SUM : op;
        const arlib::Plan p = make_plan(kind, dtype, o, nranks, count, step, vec, mis);
        s = check_shapes(ctx, {p});
        if (s != AR_OK) return s;
        DeviceGuard g(ctx->device);
        if (!g.ok) return fail(ctx, AR_ERR_RUNTIME, "cannot select device %d", ctx->device);
        return run(ctx, ctx->stream, p, table_of(bufs, nranks));
    } catch (...) {
        return fail(ctx, AR_ERR_RUNTIME, "unexpected exception");
    }
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

ar_status ar_create(ar_ctx** out, int device, void* stream) {
    if (!out) return fail(nullptr, AR_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(nullptr, AR_ERR_RUNTIME, "no HIP device available");
    }
    if (device < 0 || device >= ndev)
        return fail(nullptr, AR_ERR_INVALID_ARG, "device %d outside [0, %d)", device, ndev);
    ar_ctx* c = new (std::nothrow) ar_ctx();
    if (!c) return fail(nullptr, AR_ERR_NO_MEMORY, "cannot allocate the context");
    c->device = device;
    c->stream = reinterpret_cast<hipStream_t>(stream);
    {
        // the residency caps size their LDS reservations for kLdsBytesPerCU
        int lds = 0;
        if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  device) != hipSuccess) {
            (void)hipGetLastError();
            lds = 0;
        }
        c->caps_supported = lds == (int)arlib::kLdsBytesPerCU;
        c->caps = c->caps_supported;
    }
    {
        // ar_check_noalloc's device-resident scratch on this device; a
        // failure here only disables that entry point
        DeviceGuard g(device);
        const hipError_t e = g.ok ? arlib::check_static_scratch(device, &c->check_static)
                                  : hipErrorInvalidDevice;
        if (e != hipSuccess) {
            (void)hipGetLastError();
            c->check_static = nullptr;
            c->check_static_error = hipGetErrorString(e);
        }
    }
    *out = c;
    return AR_OK;
}

ar_status ar_set_stream(ar_ctx* ctx, void* stream) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    ctx->stream = reinterpret_cast<hipStream_t>(stream);
    return AR_OK;
}

ar_status ar_set_graphs(ar_ctx* ctx, size_t max_bytes_per_rank) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    ctx->graph_max_bytes = max_bytes_per_rank;
    if (max_bytes_per_rank == 0) {
        DeviceGuard g(ctx->device);
        clear_graphs(ctx);
    }
    return AR_OK;
}

ar_status ar_set_residency_caps(ar_ctx* ctx, int enable) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    if (enable && !ctx->caps_supported)
        return fail(ctx, AR_ERR_UNSUPPORTED,
                    "the device's LDS per compute unit is not the %u bytes the caps assume",
                    arlib::kLdsBytesPerCU);
    ctx->caps = enable != 0;
    return AR_OK;
}

ar_status ar_residency_probe(ar_ctx* ctx, unsigned lds_bytes, unsigned blocks,
                             unsigned* max_per_cu, unsigned* min_per_cu, unsigned* cus) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    if (!max_per_cu || !min_per_cu || !cus)
        return fail(ctx, AR_ERR_INVALID_ARG, "NULL output");
    if (blocks == 0 || blocks > (1u << 20))
        return fail(ctx, AR_ERR_INVALID_ARG, "blocks %u outside [1, 2^20]", blocks);
    if (lds_bytes > (64u << 10))
        return fail(ctx, AR_ERR_INVALID_ARG, "lds_bytes %u above 64 KiB", lds_bytes);
    DeviceGuard g(ctx->device);
    if (!g.ok) return fail(ctx, AR_ERR_RUNTIME, "cannot select device %d", ctx->device);
    const size_t table = (size_t)arlib::kProbeSlots * sizeof(unsigned);
    unsigned* mem = nullptr;
    if (hipMalloc(reinterpret_cast<void**>(&mem), 2 * table) != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, AR_ERR_NO_MEMORY, "cannot allocate the probe's tables");
    }
    std::vector<unsigned> mx(arlib::kProbeSlots, 0u);
    hipError_t e = hipMemsetAsync(mem, 0, 2 * table, ctx->stream);
    if (e == hipSuccess)
        e = arlib::launch_residency_probe(mem, mem + arlib::kProbeSlots, lds_bytes, blocks, 100,
                                          ctx->stream);
    if (e == hipSuccess)
        e = hipMemcpyAsync(mx.data(), mem + arlib::kProbeSlots, table, hipMemcpyDeviceToHost,
                           ctx->stream);
    if (e == hipSuccess) e = hipStreamSynchronize(ctx->stream);
    (void)hipFree(mem);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, AR_ERR_RUNTIME, "residency probe: %s", hipGetErrorString(e));
    }
    unsigned hi = 0, lo = ~0u, n = 0;
    for (unsigned v : mx) {
        if (!v) continue;
        ++n;
        hi = v > hi ? v : hi;
        lo = v < lo ? v : lo;
    }
    *max_per_cu = hi;
    *min_per_cu = n ? lo : 0u;
    *cus = n;
    return AR_OK;
}

ar_status ar_set_pointer_cache(ar_ctx* ctx, int enable) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    ctx->ptr_cache = enable != 0;
    if (!ctx->ptr_cache) ctx->checked.clear();
    return AR_OK;
}

ar_status ar_allreduce(ar_ctx* ctx, void* const* bufs, int nranks, size_t count, ar_dtype dtype,
                       ar_op op, ar_algo algo) {
    return collective(ctx, COLL_AR, bufs, nranks, count, (int)dtype, (int)op, (int)algo);
}

ar_status ar_reduce_scatter(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                            ar_dtype dtype, ar_op op, ar_algo algo) {
    return collective(ctx, COLL_RS, bufs, nranks, count, (int)dtype, (int)op, (int)algo);
}

ar_status ar_allgather(ar_ctx* ctx, void* const* bufs, int nranks, size_t count, ar_dtype dtype,
                       ar_algo algo) {
    return collective(ctx, COLL_AG, bufs, nranks, count, (int)dtype, AR_SUM, (int)algo);
}

ar_status ar_ring_rs_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                          ar_dtype dtype, ar_op op, int step) {
    return single_step(ctx, arlib::KIND_RS_STEP, bufs, nranks, count, (int)dtype, (int)op, step);
}

ar_status ar_ring_ag_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                          ar_dtype dtype, int step) {
    return single_step(ctx, arlib::KIND_AG_STEP, bufs, nranks, count, (int)dtype, AR_SUM, step);
}

ar_status ar_tree_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count, ar_dtype dtype,
                       ar_op op, int step) {
    return single_step(ctx, arlib::KIND_TREE_STEP, bufs, nranks, count, (int)dtype, (int)op, step);
}

ar_status ar_hd_rs_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                        ar_dtype dtype, ar_op op, int step) {
    return single_step(ctx, arlib::KIND_HD_RS_STEP, bufs, nranks, count, (int)dtype, (int)op,
                       step);
}

ar_status ar_hd_ag_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                        ar_dtype dtype, int step) {
    return single_step(ctx, arlib::KIND_HD_AG_STEP, bufs, nranks, count, (int)dtype, AR_SUM,
                       step);
}

ar_status ar_dtree_step(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                        ar_dtype dtype, ar_op op, int step) {
    return single_step(ctx, arlib::KIND_DT_STEP, bufs, nranks, count, (int)dtype, (int)op, step);
}

ar_status ar_predict_us(ar_algo algo, int nranks, size_t count, ar_dtype dtype, double* us) {
    if (!us || nranks < 1 || nranks > AR_MAX_RANKS || !valid_dtype((int)dtype) ||
        !valid_algo((int)algo) || algo == AR_ALGO_AUTO)
        return AR_ERR_INVALID_ARG;
    if (needs_pow2((int)algo) && !pow2(nranks)) return AR_ERR_UNSUPPORTED;
    *us = predict_allreduce_us((int)algo, nranks, count, elem_bytes(dtype));
    return AR_OK;
}

ar_status ar_auto_algo(int nranks, size_t count, ar_dtype dtype, ar_algo* out) {
    if (!out || nranks < 1 || nranks > AR_MAX_RANKS || !valid_dtype((int)dtype))
        return AR_ERR_INVALID_ARG;
    *out = (ar_algo)auto_algo(nranks, count, elem_bytes(dtype));
    return AR_OK;
}

ar_status ar_chunk_range(size_t count, int nranks, int chunk, size_t* offset, size_t* len) {
    if (!offset || !len || nranks < 1 || nranks > AR_MAX_RANKS || chunk < 0 || chunk >= nranks)
        return AR_ERR_INVALID_ARG;
    // L = ceil(count / N) without forming count + N - 1; lo and hi are
    // clamped to count without forming chunk * L or lo + L when they would
    // pass it (both can exceed SIZE_MAX for counts near SIZE_MAX)
    const size_t per = count / (size_t)nranks + (count % (size_t)nranks ? 1 : 0);
    const size_t lo = per != 0 && (size_t)chunk > count / per ? count
                      : std::min((size_t)chunk * per, count);
    *offset = lo;
    *len = count - lo < per ? count - lo : per;
    return AR_OK;
}

ar_status ar_copy(ar_ctx* ctx, void* dst, const void* src, size_t bytes) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    if (bytes == 0) return AR_OK;
    if (!dst || !src) return fail(ctx, AR_ERR_INVALID_ARG, "NULL pointer");
    if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) | bytes) & 15u)
        return fail(ctx, AR_ERR_INVALID_ARG, "ar_copy needs 16-byte aligned pointers and size");
    void* const pair[2] = {dst, const_cast<void*>(src)};
    bool vec;
    unsigned mis;
    const ar_status s = check_buffers(ctx, pair, 2, bytes / 4, AR_INT32, &vec, &mis);
    if (s != AR_OK) return s;
    DeviceGuard g(ctx->device);
    if (!g.ok) return fail(ctx, AR_ERR_RUNTIME, "cannot select device %d", ctx->device);
    const hipError_t e = arlib::launch_copy(dst, src, bytes, ctx->stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(ctx, AR_ERR_RUNTIME, "copy launch failed: %s", hipGetErrorString(e));
    }
    return AR_OK;
}

ar_status ar_stream(ar_ctx* ctx, const void* const* src, int nsrc, void* const* dst, int ndst,
                    size_t bytes) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    try {
        if (nsrc < 0 || ndst < 0 || nsrc > AR_MAX_RANKS || ndst > AR_MAX_RANKS ||
            nsrc + ndst < 1)
            return fail(ctx, AR_ERR_INVALID_ARG, "nsrc %d / ndst %d outside [0, %d], or both 0",
                        nsrc, ndst, AR_MAX_RANKS);
        if ((nsrc && !src) || (ndst && !dst)) return fail(ctx, AR_ERR_INVALID_ARG, "NULL array");
        if (bytes % 16) return fail(ctx, AR_ERR_INVALID_ARG, "bytes %zu is not a multiple of 16",
                                    bytes);
        if (bytes == 0) return AR_OK;
        // every buffer: device memory of this device, 16-byte aligned, no
        // overlap -- except that dst[i] may be src[i] itself (the in-place
        // pattern of an AllReduce: each block reads its tile of every source
        // before it writes, and blocks own disjoint tiles)
        std::vector<void*> all;
        for (int i = 0; i < nsrc; ++i) all.push_back(const_cast<void*>(src[i]));
        for (int i = 0; i < ndst; ++i)
            if (!(i < nsrc && dst[i] == src[i])) all.push_back(dst[i]);
        if (all.size() > (size_t)AR_MAX_RANKS)
            return fail(ctx, AR_ERR_INVALID_ARG, "%zu distinct buffers, at most %d", all.size(),
                        AR_MAX_RANKS);
        for (size_t i = 0; i < all.size(); ++i)
            if (reinterpret_cast<uintptr_t>(all[i]) & 15u)
                return fail(ctx, AR_ERR_INVALID_ARG, "buffer %zu is not 16-byte aligned", i);
        bool vec;
        unsigned mis;
        const ar_status s =
            check_buffers(ctx, all.data(), (int)all.size(), bytes / 4, AR_INT32, &vec, &mis);
        if (s != AR_OK) return s;
        DeviceGuard g(ctx->device);
        if (!g.ok) return fail(ctx, AR_ERR_RUNTIME, "cannot select device %d", ctx->device);
        const hipError_t e = arlib::launch_stream(src, nsrc, dst, ndst, bytes, ctx->caps, ctx->stream);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(ctx, AR_ERR_RUNTIME, "stream launch failed: %s", hipGetErrorString(e));
        }
        return AR_OK;
    } catch (const std::bad_alloc&) {
        return fail(ctx, AR_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(ctx, AR_ERR_RUNTIME, "unexpected exception");
    }
}

ar_status ar_stream_timeline(ar_ctx* ctx, void* const* bufs, int nbufs, size_t bytes,
                             unsigned lds_bytes, unsigned long long* ts, size_t ts_len,
                             size_t* blocks, unsigned* clock_khz) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    try {
        if (!bufs || !ts) return fail(ctx, AR_ERR_INVALID_ARG, "NULL bufs or ts");
        if (nbufs < 1 || nbufs > AR_MAX_RANKS)
            return fail(ctx, AR_ERR_INVALID_ARG, "nbufs %d outside [1, %d]", nbufs, AR_MAX_RANKS);
        if (bytes == 0 || bytes % 16)
            return fail(ctx, AR_ERR_INVALID_ARG, "bytes %zu is 0 or not a multiple of 16", bytes);
        if (lds_bytes > (64u << 10))
            return fail(ctx, AR_ERR_INVALID_ARG, "lds_bytes %u above 64 KiB", lds_bytes);
        if (reinterpret_cast<uintptr_t>(ts) & 7u)
            return fail(ctx, AR_ERR_INVALID_ARG, "ts is not 8-byte aligned");
        const size_t nblk = (bytes + 1023) / 1024;   // one 1 KiB tile per buffer per block
        if (nblk > 0x7fffffffu)
            return fail(ctx, AR_ERR_INVALID_ARG, "bytes %zu needs more than 2^31 blocks", bytes);
        if (ts_len < 2 * nblk)
            return fail(ctx, AR_ERR_INVALID_ARG, "ts_len %zu below 2 x %zu blocks", ts_len, nblk);
        for (int i = 0; i < nbufs; ++i)
            if (reinterpret_cast<uintptr_t>(bufs[i]) & 15u)
                return fail(ctx, AR_ERR_INVALID_ARG, "bufs[%d] is not 16-byte aligned", i);
        bool vec;
        unsigned mis;
        ar_status st = check_buffers(ctx, bufs, nbufs, bytes / 4, AR_INT32, &vec, &mis);
        if (st != AR_OK) return st;
        void* tsp = ts;
        const size_t ts_bytes = 2 * nblk * sizeof(unsigned long long);
        st = check_buffers(ctx, &tsp, 1, ts_bytes / 4, AR_INT32, &vec, &mis);
        if (st != AR_OK) return st;
        const uintptr_t t0 = reinterpret_cast<uintptr_t>(ts);
        for (int i = 0; i < nbufs; ++i) {
            const uintptr_t b = reinterpret_cast<uintptr_t>(bufs[i]);
            if (t0 < b + bytes && b < t0 + ts_bytes)
                return fail(ctx, AR_ERR_INVALID_ARG, "ts overlaps bufs[%d]", i);
        }
        DeviceGuard g(ctx->device);
        if (!g.ok) return fail(ctx, AR_ERR_RUNTIME, "cannot select device %d", ctx->device);
        if (clock_khz) {
            int khz = 0;
            if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, ctx->device) !=
                    hipSuccess ||
                khz <= 0) {
                (void)hipGetLastError();
                return fail(ctx, AR_ERR_RUNTIME, "cannot read the wall-clock rate");
            }
            *clock_khz = (unsigned)khz;
        }
        const hipError_t e =
            arlib::launch_stream_timeline(bufs, nbufs, bytes, lds_bytes, ts, ctx->stream);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(ctx, AR_ERR_RUNTIME, "timeline launch failed: %s", hipGetErrorString(e));
        }
        if (blocks) *blocks = nblk;
        return AR_OK;
    } catch (const std::bad_alloc&) {
        return fail(ctx, AR_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(ctx, AR_ERR_RUNTIME, "unexpected exception");
    }
}

namespace {

// ar_check and ar_check_noalloc: the same validation and kernels; the
// partial records go to the context's allocated array or to the
// device-resident one.
ar_status check_impl(ar_ctx* ctx, void* const* bufs, int nranks, size_t count, ar_dtype dtype,
                     const double* ref, const double* bound, ar_check_result* result,
                     bool noalloc) {
    if (!ctx) return fail(nullptr, AR_ERR_INVALID_ARG, "ctx is NULL");
    try {
        if (!result) return fail(ctx, AR_ERR_INVALID_ARG, "result is NULL");
        if (reinterpret_cast<uintptr_t>(result) & 7u)
            return fail(ctx, AR_ERR_INVALID_ARG, "result is not 8-byte aligned");
        if (bound && !ref) return fail(ctx, AR_ERR_INVALID_ARG, "bound given without ref");
        bool vec;
        unsigned mis;
        ar_status s = check_buffers(ctx, bufs, nranks, count, (int)dtype, &vec, &mis);
        if (s != AR_OK) return s;
        s = check_device_span(ctx, result, sizeof(ar_check_result), "result");
        if (s != AR_OK) return s;
        if (count > 0) {
            if (count > SIZE_MAX / sizeof(double))
                return fail(ctx, AR_ERR_INVALID_ARG, "count %zu overflows the reference", count);
            if (ref && (reinterpret_cast<uintptr_t>(ref) & 7u))
                return fail(ctx, AR_ERR_INVALID_ARG, "ref is not 8-byte aligned");
            if (bound && (reinterpret_cast<uintptr_t>(bound) & 7u))
                return fail(ctx, AR_ERR_INVALID_ARG, "bound is not 8-byte aligned");
            if (ref && (s = check_device_span(ctx, ref, count * sizeof(double), "ref")) != AR_OK)
                return s;
            if (bound && (s = check_device_span(ctx, bound, count * sizeof(double), "bound")) != AR_OK)
                return s;
        }
        DeviceGuard g(ctx->device);
        if (!g.ok) return fail(ctx, AR_ERR_RUNTIME, "cannot select device %d", ctx->device);
        if (noalloc && !ctx->check_static)
            return fail(ctx, AR_ERR_RUNTIME, "the device-resident scratch is unavailable: %s",
                        ctx->check_static_error.c_str());
        if (noalloc && arlib::check_blocks(count) > arlib::kCheckMaxBlocks)
            return fail(ctx, AR_ERR_INVALID_ARG, "count %zu needs more than %u partial records",
                        count, arlib::kCheckMaxBlocks);   // unreachable: the grid is capped
        if (!noalloc && !ctx->check_part) {
            void* p = nullptr;
            if (hipMalloc(&p, sizeof(arlib::CheckPartial) * arlib::kCheckMaxBlocks) != hipSuccess ||
                !p) {
                (void)hipGetLastError();
                return fail(ctx, AR_ERR_NO_MEMORY, "cannot allocate the checker's scratch array");
            }
            ctx->check_part = static_cast<arlib::CheckPartial*>(p);
        }
        arlib::CheckArgs a;
        a.t = table_of(bufs, nranks);
        a.count = count;
        a.n = nranks;
        a.dtype = (int)dtype;
        a.eb = (int)elem_bytes(dtype);
        a.ref = count ? ref : nullptr;
        a.bound = count ? bound : nullptr;
        const hipError_t e = arlib::launch_check(
            a, noalloc ? ctx->check_static : ctx->check_part, result, ctx->stream);
        if (e != hipSuccess) {
            (void)hipGetLastError();
            return fail(ctx, AR_ERR_RUNTIME, "check launch failed: %s", hipGetErrorString(e));
        }
        return AR_OK;
    } catch (const std::bad_alloc&) {
        return fail(ctx, AR_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(ctx, AR_ERR_RUNTIME, "unexpected exception");
    }
}

}  // namespace

ar_status ar_check(ar_ctx* ctx, void* const* bufs, int nranks, size_t count, ar_dtype dtype,
                   const double* ref, const double* bound, ar_check_result* result) {
    return check_impl(ctx, bufs, nranks, count, dtype, ref, bound, result, false);
}

ar_status ar_check_noalloc(ar_ctx* ctx, void* const* bufs, int nranks, size_t count,
                           ar_dtype dtype, const double* ref, const double* bound,
                           ar_check_result* result) {
    return check_impl(ctx, bufs, nranks, count, dtype, ref, bound, result, true);
}

const char* ar_status_string(ar_status s) {
    switch (s) {
        case AR_OK: return "AR_OK";
        case AR_ERR_INVALID_ARG: return "AR_ERR_INVALID_ARG";
        case AR_ERR_UNSUPPORTED: return "AR_ERR_UNSUPPORTED";
        case AR_ERR_RUNTIME: return "AR_ERR_RUNTIME";
        case AR_ERR_NO_MEMORY: return "AR_ERR_NO_MEMORY";
    }
    return "AR_ERR_UNKNOWN";
}

const char* ar_last_error(const ar_ctx* ctx) {
    return ctx ? ctx->last_error.c_str() : g_create_error.c_str();
}

ar_status ar_destroy(ar_ctx* ctx) {
    if (!ctx) return AR_OK;
    if (!ctx->graph_cache.empty() || ctx->capture || ctx->check_part) {
        DeviceGuard g(ctx->device);
        clear_graphs(ctx);
        if (ctx->capture) (void)hipStreamDestroy(ctx->capture);
        // the checker's scratch may still be in use by enqueued work
        if (ctx->check_part) {
            (void)hipStreamSynchronize(ctx->stream);
            (void)hipFree(ctx->check_part);
        }
        (void)hipGetLastError();
    }
    delete ctx;
    return AR_OK;
}

}  // extern "C"
#pragma GCC visibility pop
