// fake_hip.cpp -- a CPU-only stand-in for the HIP runtime and for the kernel
// launchers, used to run the library's host code (argument validation, chunk
// layout, launch planning, graph-replay cache) under AddressSanitizer and
// UndefinedBehaviorSanitizer without a GPU.  Test infrastructure only.
//
// * "Device memory" is a registry of address ranges; the ranges are never
//   dereferenced, so they may be arbitrarily large.
// * Kernel launchers record each launch (its plan, arguments and grid) and
//   check on the host that the grid covers every element the kernel is meant
//   to touch, with the rule each kernel family uses to map blocks to work.
// * Streams, events, graphs and stream capture are modelled just far enough
//   for the library's graph cache: a launch on a capturing stream is recorded
//   into the capture, a graph launch replays the recorded launches.
// Every object the fake hands out is heap-allocated, so LeakSanitizer reports
// any stream, event or graph the library fails to release.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <vector>

#include "common.h"
#include "fake_hip.h"

namespace {

struct Range {
    uintptr_t base;
    size_t size;
    int device;
};
std::vector<Range> g_ranges;

struct FakeStream {
    bool capturing = false;
    std::vector<FakeLaunch>* sink = nullptr;   // capture target
};
struct FakeGraph {
    std::vector<FakeLaunch> launches;
};
struct FakeEvent {
    int dummy = 0;
};

FakeStream g_null_stream;
std::vector<FakeLaunch> g_executed;
FakeCounters g_count;
int g_device = 0;
int g_lds_per_cu = 160 << 10;   // gfx950
hipError_t g_last = hipSuccess;
bool g_coverage_ok = true;
char g_coverage_msg[512];

FakeStream* S(hipStream_t s) { return s ? reinterpret_cast<FakeStream*>(s) : &g_null_stream; }

hipError_t set(hipError_t e) {
    if (e != hipSuccess) g_last = e;
    return e;
}

void coverage_fail(const char* what, const arlib::Args& a, dim3 grid) {
    if (g_coverage_ok)
        std::snprintf(g_coverage_msg, sizeof g_coverage_msg,
                      "%s: n=%d count=%zu per=%zu step=%d tiles=%u grid=%u", what, a.n, a.count,
                      a.per, a.step, a.tiles, grid.x);
    g_coverage_ok = false;
}

// Elements one group (chunk, pair, tree node, ...) of the launch must cover,
// and the number of groups, for each kernel family.
void expected_work(const arlib::Plan& p, const arlib::Args& a, size_t* elems, size_t* groups) {
    const size_t n = (size_t)p.nranks;
    const size_t per = (p.count + n - 1) / n;
    int L = 0;
    while ((1 << L) < p.nranks) ++L;
    switch (p.kind) {
        case arlib::KIND_TREE_STEP:
            *elems = p.count;
            *groups = n / 2;
            break;
        case arlib::KIND_DT_STEP: {
            const int s = p.step;
            size_t nodes = 1;
            if (s < L - 1) nodes = n >> (s + 2);
            else if (s > L) nodes = n >> (2 * L - s + 1);
            *elems = (p.count + 1) / 2;
            *groups = 2 * nodes;
            break;
        }
        case arlib::KIND_HD_RS_STEP:
            *elems = per * (n >> (p.step + 1));
            *groups = n;
            break;
        case arlib::KIND_HD_AG_STEP:
            *elems = per * ((size_t)1 << p.step);
            *groups = n;
            break;
        default:
            if (p.order == arlib::ORDER_DTREE) {   // fused double tree: two halves
                *elems = (p.count + 1) / 2;
                *groups = 2;
            } else {
                *elems = per;
                *groups = n;
            }
            break;
    }
    (void)a;
}

void record(const arlib::Plan& p, const arlib::Args& a, dim3 grid, hipStream_t s, bool fused) {
    FakeLaunch l;
    l.plan = p;
    l.args = a;
    l.grid = grid.x;
    FakeStream* fs = S(s);
    if (fs->capturing) fs->sink->push_back(l);
    else g_executed.push_back(l);
    ++g_count.kernel_launches;

    // the grid must cover the work: blocks = tiles x groups, and tiles x
    // (threads x units per lane x elements per unit) >= elements per group
    size_t elems = 0, groups = 0;
    expected_work(p, a, &elems, &groups);
    const size_t eb = (size_t)arlib::elem_bytes(p.dtype);
    size_t threads, upl, epu;
    if (fused) {
        const int cfg = arlib::fused_variant(p);
        threads = arlib::kFusedThreads;
        upl = (size_t)arlib::fused_units_per_lane(cfg);
        epu = (p.vec && cfg != arlib::CFG_TINY) ? 16 / eb : 1;
    } else {
        threads = arlib::kThreads;
        upl = arlib::kUnroll;
        epu = p.vec ? 16 / eb : 1;
    }
    // a fused plan whose chunk bodies can start off a 128-byte line shifts its
    // tiles back by up to kLeadUnits idle units: the grid must cover those too
    const size_t lead = fused && p.lead && epu > 1 ? arlib::kLeadUnits * epu : 0;
    if (a.tiles == 0 || (size_t)grid.x != (size_t)a.tiles * groups)
        coverage_fail("grid is not tiles x groups", a, grid);
    else if ((size_t)a.tiles * threads * upl * epu < elems + lead)
        coverage_fail("tiles do not cover the group's elements", a, grid);
    else if (elems > 0 && ((size_t)a.tiles - 1) * threads * upl * epu >= elems + lead + threads * upl * epu)
        coverage_fail("more tiles than the work needs", a, grid);
    const size_t parts = fused ? (size_t)arlib::fused_parts(p.order, p.nranks) : (size_t)p.nranks;
    if (a.n != p.nranks || a.count != p.count || a.per != (p.count + parts - 1) / parts)
        coverage_fail("kernel arguments disagree with the plan", a, grid);
    for (int r = 0; r < p.nranks; ++r)
        if (!a.t.p[r]) coverage_fail("NULL rank pointer passed to a kernel", a, grid);
}

}  // namespace

// ----------------------------------------------------------- test controls
void fake_register(const void* base, size_t size, int device) {
    g_ranges.push_back({reinterpret_cast<uintptr_t>(base), size, device});
}
void fake_reset_ranges() { g_ranges.clear(); }
const std::vector<FakeLaunch>& fake_executed() { return g_executed; }
void fake_clear_executed() { g_executed.clear(); }
FakeCounters& fake_counters() { return g_count; }
bool fake_coverage_ok(const char** msg) {
    if (msg) *msg = g_coverage_msg;
    return g_coverage_ok;
}
void fake_set_lds_per_cu(int bytes) { g_lds_per_cu = bytes; }
void fake_set_null_stream_capturing(bool on, std::vector<FakeLaunch>* sink) {
    g_null_stream.capturing = on;
    g_null_stream.sink = sink;
}

// ------------------------------------------------------------ kernel side
namespace arlib {
hipError_t launch_fused_kind(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    record(p, a, grid, s, true);
    return hipSuccess;
}
hipError_t launch_step_kind(const Plan& p, const Args& a, dim3 grid, hipStream_t s) {
    record(p, a, grid, s, false);
    return hipSuccess;
}
hipError_t launch_copy(void*, const void*, size_t, hipStream_t) {
    ++g_count.kernel_launches;
    return hipSuccess;
}
hipError_t launch_residency_probe(unsigned*, unsigned*, unsigned, unsigned, int, hipStream_t) {
    ++g_count.kernel_launches;
    return hipSuccess;
}
hipError_t launch_stream(const void* const*, int, void* const*, int, size_t, bool, hipStream_t) {
    ++g_count.kernel_launches;
    return hipSuccess;
}
hipError_t launch_stream_timeline(void* const*, int, size_t, unsigned, unsigned long long*,
                                  hipStream_t) {
    ++g_count.kernel_launches;
    return hipSuccess;
}
unsigned check_blocks(size_t count) {
    const size_t want = (count + kCheckThreads - 1) / kCheckThreads;
    return (unsigned)(want == 0 ? 1 : want < kCheckMaxBlocks ? want : kCheckMaxBlocks);
}
hipError_t check_static_scratch(int device, CheckPartial** out) {
    // a fixed stand-in address; never dereferenced
    *out = device == 0 ? reinterpret_cast<CheckPartial*>(uintptr_t(1) << 41) : nullptr;
    return device == 0 ? hipSuccess : hipErrorInvalidDevice;
}
hipError_t launch_check(const CheckArgs& a, CheckPartial* part, ar_check_result* out, hipStream_t) {
    g_count.kernel_launches += a.count > 0 ? 2 : 1;
    if (!part || !out) coverage_fail("checker launched without scratch or result", Args{}, dim3(0));
    return hipSuccess;
}
}  // namespace arlib

// ------------------------------------------------------------- HIP runtime
extern "C" {

hipError_t hipGetDeviceCount(int* count) {
    *count = 1;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int device) {
    if (device != 0) return set(hipErrorInvalidDevice);
    if (attr == hipDeviceAttributeWallClockRate) {
        *value = 100000;   // a 100 MHz clock
        return hipSuccess;
    }
    if (attr != hipDeviceAttributeMaxSharedMemoryPerMultiprocessor) return set(hipErrorInvalidValue);
    *value = g_lds_per_cu;
    return hipSuccess;
}
hipError_t hipGetDevice(int* d) {
    *d = g_device;
    return hipSuccess;
}
hipError_t hipSetDevice(int d) {
    if (d != 0) return set(hipErrorInvalidDevice);
    g_device = d;
    return hipSuccess;
}
hipError_t hipGetLastError(void) {
    const hipError_t e = g_last;
    g_last = hipSuccess;
    return e;
}
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "ok" : "fake error"; }

hipError_t hipPointerGetAttributes(hipPointerAttribute_t* at, const void* ptr) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(ptr);
    for (const Range& r : g_ranges)
        if (p >= r.base && p - r.base < r.size) {
            at->type = hipMemoryTypeDevice;
            at->device = r.device;
            at->devicePointer = const_cast<void*>(ptr);
            return hipSuccess;
        }
    return set(hipErrorInvalidValue);
}
hipError_t hipMemGetAddressRange(hipDeviceptr_t* base, size_t* size, hipDeviceptr_t ptr) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(ptr);
    for (const Range& r : g_ranges)
        if (p >= r.base && p - r.base < r.size) {
            *base = reinterpret_cast<hipDeviceptr_t>(r.base);
            *size = r.size;
            return hipSuccess;
        }
    return set(hipErrorInvalidValue);
}

hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
    *s = reinterpret_cast<hipStream_t>(new FakeStream());
    ++g_count.streams_created;
    return hipSuccess;
}
hipError_t hipStreamDestroy(hipStream_t s) {
    delete reinterpret_cast<FakeStream*>(s);
    ++g_count.streams_destroyed;
    return hipSuccess;
}
hipError_t hipStreamBeginCapture(hipStream_t s, hipStreamCaptureMode) {
    FakeStream* fs = S(s);
    if (fs->capturing) return set(hipErrorIllegalState);
    fs->capturing = true;
    fs->sink = new std::vector<FakeLaunch>();
    ++g_count.captures;
    return hipSuccess;
}
hipError_t hipStreamEndCapture(hipStream_t s, hipGraph_t* graph) {
    FakeStream* fs = S(s);
    if (!fs->capturing) return set(hipErrorIllegalState);
    FakeGraph* g = new FakeGraph();
    g->launches = *fs->sink;
    delete fs->sink;
    fs->sink = nullptr;
    fs->capturing = false;
    *graph = reinterpret_cast<hipGraph_t>(g);
    ++g_count.graphs_created;
    return hipSuccess;
}
hipError_t hipStreamIsCapturing(hipStream_t s, hipStreamCaptureStatus* st) {
    *st = S(s)->capturing ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
    return hipSuccess;
}
hipError_t hipGraphInstantiate(hipGraphExec_t* exec, hipGraph_t graph, hipGraphNode_t*, char*,
                               size_t) {
    FakeGraph* g = new FakeGraph(*reinterpret_cast<FakeGraph*>(graph));
    *exec = reinterpret_cast<hipGraphExec_t>(g);
    ++g_count.execs_created;
    return hipSuccess;
}
hipError_t hipGraphDestroy(hipGraph_t graph) {
    delete reinterpret_cast<FakeGraph*>(graph);
    ++g_count.graphs_destroyed;
    return hipSuccess;
}
hipError_t hipGraphExecDestroy(hipGraphExec_t exec) {
    delete reinterpret_cast<FakeGraph*>(exec);
    ++g_count.execs_destroyed;
    return hipSuccess;
}
hipError_t hipGraphLaunch(hipGraphExec_t exec, hipStream_t s) {
    const FakeGraph* g = reinterpret_cast<const FakeGraph*>(exec);
    FakeStream* fs = S(s);
    for (const FakeLaunch& l : g->launches) {
        if (fs->capturing) fs->sink->push_back(l);
        else g_executed.push_back(l);
    }
    ++g_count.graph_launches;
    return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
    *e = reinterpret_cast<hipEvent_t>(new FakeEvent());
    ++g_count.events_created;
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipMalloc(void** p, size_t size) {
    // host memory stands in for the allocation; kernels never run here
    *p = new char[size ? size : 1];
    ++g_count.device_allocs;
    return hipSuccess;
}
hipError_t hipFree(void* p) {
    if (p) {
        delete[] static_cast<char*>(p);
        ++g_count.device_frees;
    }
    return hipSuccess;
}
hipError_t hipMemsetAsync(void* p, int value, size_t size, hipStream_t) {
    // fake "device" memory is host memory (hipMalloc above)
    std::memset(p, value, size);
    return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t size, hipMemcpyKind, hipStream_t) {
    std::memcpy(dst, src, size);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) {
    ++g_count.stream_syncs;
    return hipSuccess;
}
hipError_t hipEventSynchronize(hipEvent_t) {
    ++g_count.event_syncs;
    return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t e) {
    delete reinterpret_cast<FakeEvent*>(e);
    ++g_count.events_destroyed;
    return hipSuccess;
}

}  // extern "C"
