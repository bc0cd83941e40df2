// probe.h -- the residency probe (probe.hip), a diagnostic of the LDS
// reservations that cap the fused kernels' resident waves.  Not part of the
// public ABI; ar_residency_probe wraps it.
#pragma once

#include <hip/hip_runtime_api.h>

namespace arlib {

constexpr unsigned kProbeSlots = 4096;   // per-CU table entries (12-bit CU key)

// Launches `blocks` one-wave blocks with `lds_bytes` of dynamic LDS.  Each
// block's first lane counts itself in cur[key] while it sleeps for a bounded
// time (about `spin` x 8 K cycles) and records the count it saw in mx[key];
// key identifies the compute unit (XCC and hardware id).  cur and mx hold
// kProbeSlots entries each and must be zero on entry.
hipError_t launch_residency_probe(unsigned* cur, unsigned* mx, unsigned lds_bytes,
                                  unsigned blocks, int spin, hipStream_t s);

}  // namespace arlib
