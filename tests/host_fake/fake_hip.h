// fake_hip.h -- controls of the CPU-only HIP stand-in (test infrastructure).
#pragma once

#include <vector>

#include "common.h"

struct FakeLaunch {
    arlib::Plan plan;
    arlib::Args args;
    unsigned grid;
};

struct FakeCounters {
    long kernel_launches = 0;
    long streams_created = 0, streams_destroyed = 0;
    long captures = 0;
    long graphs_created = 0, graphs_destroyed = 0;
    long execs_created = 0, execs_destroyed = 0;
    long graph_launches = 0;
    long events_created = 0, events_destroyed = 0, event_syncs = 0;
    long device_allocs = 0, device_frees = 0, stream_syncs = 0;
};

// Registers [base, base + size) as device memory of `device` (never touched).
void fake_register(const void* base, size_t size, int device);
void fake_reset_ranges();
// Launches that ran (directly or from a graph), in order.
const std::vector<FakeLaunch>& fake_executed();
void fake_clear_executed();
FakeCounters& fake_counters();
// False once any launch's grid failed to cover its work; *msg says which.
bool fake_coverage_ok(const char** msg);
// Makes the null stream a capturing stream whose launches go to `sink`.
void fake_set_null_stream_capturing(bool on, std::vector<FakeLaunch>* sink);
// LDS per compute unit the fake device reports (gfx950: 160 KiB)
void fake_set_lds_per_cu(int bytes);
