"""Benchmark of the single-GPU AllReduce hot path on MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--algo ALGO]

One step is one in-place AllReduce (ReduceScatter + AllGather, fused into one
pass by default) of N logical ranks held in HBM.  The default workload is the
DDP gradient bucket: 8 ranks x 25 MiB fp32 (6,553,600 values ~ N(0, 1e-3)),
op AVG.  Steps rotate over several independent bucket sets whose combined
footprint is several times the 256 MB Infinity Cache, so every step reads its
inputs from HBM, as a DDP step reducing many different buckets does.

Printed (one JSON line):
  value      algorithmic HBM GB/s of the whole timed run: 2*N*K bytes per
             AllReduce (every input read once, every output written once; K =
             bytes per rank) x K steps / wall time between the two
             synchronisations
  roofline   the dominant kernel's GB/s from HIP events recorded on its stream
             at both ends of the timed region (mean per launch), against the
             8 TB/s HBM peak; the median and minimum of per-launch event times
             from a second pass over the same buckets beside it; `traffic` is
             the HBM bytes per launch measured with rocprofv3 counters (scaled
             by a plain copy of known size) when the kernel source is
             unchanged since they were taken, else null
  others     the other algorithms on the same buckets, the fused ReduceScatter
             and AllGather alone, the plain copy and the R-read / W-write
             calibration streams (ar_stream) over the same bytes per buffer
  cpu_baseline  the CPU oracle (message-passing simulation, numpy, one core)
             on the whole workload when it fits the host comfortably, else on
             the workload's first elements of every rank (the sample is
             named); the GPU result is checked against the oracle bitwise,
             whole or at sampled positions
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
INFINITY_CACHE_BYTES = 256 << 20
ALWAYS_REPLAY = 1 << 62         # graph-replay threshold that covers every size measured
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
# the sources the fused kernel and the calibration copy are built from, and
# the host code that picks their shape and residency cap
KERNEL_SOURCES = [os.path.join(ROOT, "ring_allreduce_rs_amd", "csrc", f)
                  for f in ("common.h", "elem.h", "launch.h", "fused_impl.h", "fused.hip",
                            "fused_f32.hip", "fused_bf16.hip", "fused_i32.hip", "fused_f32_lead.hip",
                            "fused_bf16_lead.hip", "fused_i32_lead.hip", "copy.hip", "dispatch.hip")]


def strip_comments(src: str) -> str:
    """C / C++ source without its comments, whitespace runs collapsed: what
    the compiler sees, so that editing a comment keeps measurements valid."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash() -> str:
    """Hash of the fused kernels' sources (comments excluded): the committed
    byte counters are reported only while it matches theirs."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch from the committed counter runs, if still valid."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(key)
    if not ent or ent.get("kernel_source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def parse():
    import workloads as W
    names = {w.name: w for w in W.ALL}
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default=W.DDP_BUCKET.name, choices=sorted(names))
    ap.add_argument("--algo", default="ring_fused",
                    choices=["ring_fused", "ring_step", "tree", "halving_doubling",
                             "double_tree", "tree_fused", "halving_doubling_fused",
                             "double_tree_fused"])
    ap.add_argument("--sets", type=int, default=0,
                    help="bucket sets to rotate over (0: enough to exceed the Infinity Cache 4x)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the secondary per-step ring / tree / copy measurements")
    ap.add_argument("--no-residency-caps", action="store_true",
                    help="run the one-pass kernels without their residency caps "
                         "(ar_set_residency_caps off: uncapped shapes, for comparison)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum CPU time spent timing the oracle")
    ap.add_argument("--sweep", action="store_true",
                    help="time every algorithm over the 64-rank message-size sweep, fit the "
                         "latency/bandwidth model T = a + b*K per algorithm and report the "
                         "ring/tree crossover (one JSON line per point, then one fit line)")
    ap.add_argument("--size-sweep", action="store_true",
                    help="time the fused AllReduce, the in-place N-read / N-write calibration "
                         "stream and the plain copy over the same bytes, for the workload's rank "
                         "count and dtype at sizes per rank from 0.78 to 400 MiB, and fit "
                         "T = a + bytes / BW to each (one JSON line per size, then one fit line)")
    ap.add_argument("--timeline", action="store_true",
                    help="per-block timeline of the in-place N-read / N-write calibration stream "
                         "at the workload's size (ar_stream_timeline), under the one-pass ring's "
                         "residency cap and without: steady streaming rate, ramp and drain (one "
                         "JSON line per launch)")
    a = ap.parse_args()
    return a, names[a.workload]


def time_algo(ar, sets, w, algo, steps, warmup, kind="allreduce"):
    """Time `steps` back-to-back launches of one collective (`kind`).

    Returns (wall seconds between the two synchronisations, mean ms per
    launch from HIP events recorded on the launch stream at the start and the
    end of the timed region)."""
    import torch
    calls = [ar.bind(ts, op=w.op, algo=algo, kind=kind) for ts in sets]
    # every bucket set at least once before timing (with graph replay on, the
    # first call on a set records its graph)
    for i in range(max(warmup, len(calls))):
        calls[i % len(calls)]()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        calls[i % len(calls)]()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, start.elapsed_time(end) / steps


def copy_ceiling(ar, nbytes, reps=50):
    """GB/s (read + write) of the plain 16-byte copy kernel over nbytes,
    rotating over buffer pairs that together exceed the Infinity Cache."""
    import torch
    nb = (nbytes // 16) * 16
    npairs = max(2, -(-4 * INFINITY_CACHE_BYTES // (2 * nb)))
    pairs = [(torch.empty(nb, dtype=torch.uint8, device="cuda"),
              torch.empty(nb, dtype=torch.uint8, device="cuda")) for _ in range(npairs)]
    for d, s in pairs:
        s.fill_(1)
        ar.copy_(d, s)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(reps):
        d, s = pairs[i % len(pairs)]
        ar.copy_(d, s)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    return 2 * nb / (ms * 1e-3) / 1e9, ms


LAUNCH_GROUP = 10               # launches between two events of the per-launch pass


def launch_stats(ar, sets, w, algo, groups):
    """Per-launch HIP-event times (ms): `groups` groups of LAUNCH_GROUP
    back-to-back launches rotating over the bucket sets, one event on the
    launch stream between consecutive groups; each group's time / LAUNCH_GROUP
    is one sample.  (A timing event after every single launch costs a few
    microseconds of its own, more than the spread being measured.)  Returns
    (median, min, mean) over the groups."""
    import statistics

    import torch
    calls = [ar.bind(ts, op=w.op, algo=algo) for ts in sets]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(groups + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    i = 0
    for g in range(groups):
        for _ in range(LAUNCH_GROUP):
            calls[i % len(calls)]()
            i += 1
        evs[g + 1].record()
    torch.cuda.synchronize()
    ms = [evs[g].elapsed_time(evs[g + 1]) / LAUNCH_GROUP for g in range(groups)]
    return statistics.median(ms), min(ms), sum(ms) / len(ms)


def stream_ceiling(ar, nsrc, ndst, nbytes, reps=40, in_place=False):
    """GB/s of the calibration stream reading nsrc and writing ndst buffers of
    nbytes each (ar_stream: the fused kernel's tiling, no reduction), rotating
    over buffer sets that together exceed the Infinity Cache 4x.  in_place:
    the destinations are the sources themselves, as in an AllReduce."""
    import torch
    nb = (nbytes // 16) * 16
    per_set = (nsrc + ndst) * nb
    nsets = max(1, min(8, -(-4 * INFINITY_CACHE_BYTES // (nsrc if in_place else nsrc + ndst)
                            // nb)))
    sets = []
    for _ in range(nsets):
        srcs = [torch.ones(nb // 4, dtype=torch.int32, device="cuda") for _ in range(nsrc)]
        dsts = (srcs[:ndst] if in_place else
                [torch.empty(nb // 4, dtype=torch.int32, device="cuda") for _ in range(ndst)])
        sets.append((srcs, dsts))
    for srcs, dsts in sets:
        ar.stream_(srcs, dsts)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(reps):
        srcs, dsts = sets[i % nsets]
        ar.stream_(srcs, dsts)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    del sets
    torch.cuda.empty_cache()
    return per_set / (ms * 1e-3) / 1e9, ms


def host_mem_available_gib():
    try:
        with open("/proc/meminfo", encoding="ascii") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return round(int(line.split()[1]) / (1 << 20), 1)
    except OSError:
        pass
    return None


def oracle_allreduce(algo):
    """The oracle's message-passing simulation of `algo` (test infrastructure)."""
    import oracle
    if algo in ("tree", "tree_fused"):
        return oracle.simulate_tree_allreduce
    if algo in ("halving_doubling", "halving_doubling_fused"):
        return oracle.simulate_hd_allreduce
    if algo in ("double_tree", "double_tree_fused"):
        return oracle.simulate_double_tree_allreduce
    return oracle.simulate_ring_allreduce


def cpu_baseline(w, algo, sets_host, gpu_first, min_seconds, sample_count=None):
    """Time the CPU oracle on the workload (or, when sample_count is given, on
    the first sample_count elements of every rank: the same per-element work
    at a size the host finishes in seconds); also check the GPU's first
    result when it is given for the same input."""
    import numpy as np
    sim = oracle_allreduce(algo)
    reps, t_total = 0, 0.0
    out = None
    while t_total < min_seconds or reps == 0:
        t0 = time.perf_counter()
        out = sim(sets_host, w.dtype, w.op).state
        t_total += time.perf_counter() - t0
        reps += 1
    ok = None
    if gpu_first is not None:
        ok = all(np.array_equal(np.ascontiguousarray(g).view(np.uint8),
                                np.ascontiguousarray(o).view(np.uint8))
                 for g, o in zip(gpu_first, out))
    per = t_total / reps
    count = sample_count or w.count
    nbytes = 2 * w.nranks * count * (w.bytes_per_rank // w.count)
    gbps = nbytes / per / 1e9
    what = (f"whole workload ({w.nranks} ranks x {w.count} {w.dtype}, {w.op})" if not sample_count
            else f"the first {sample_count} of {w.count} {w.dtype} elements of each of the "
                 f"{w.nranks} ranks (bucket set 0, {w.op}), an AllReduce of that count; the "
                 f"whole workload needs {2 * w.nranks * w.bytes_per_rank / 2**30:.0f} GiB of "
                 "host arrays for inputs and state")
    return {
        "value": round(gbps, 4),
        "unit": "GB/s",
        "cores": 1,
        "kind": "oracle",
        "sample": (f"{what} through oracle.{sim.__name__}, {reps} run(s), {per:.3f} s each; "
                   "numpy elementwise kernels, single thread"),
        "seconds_per_allreduce": round(per, 4),
    }, ok


def sampled_parity(w, algo, vals, idx, got):
    """The oracle's per-position fold at sampled positions against the GPU
    result there (full-size workloads whose whole oracle run would not fit)."""
    import numpy as np

    import oracle
    per = -(-w.count // w.nranks)
    if algo in ("ring_fused", "ring_step"):
        want = oracle.ring_fold_at(vals, (idx // per).astype(np.int64), w.nranks, w.dtype, w.op)
    elif algo in ("tree", "tree_fused"):
        want = oracle.tree_fold_at(vals, w.dtype, w.op)
    elif algo in ("halving_doubling", "halving_doubling_fused"):
        want = oracle.hd_fold_at(vals, w.dtype, w.op)
    else:
        half = (w.count + 1) // 2
        want = np.where(idx < half, oracle.dtree_fold_at(vals, 0, w.dtype, w.op),
                        oracle.dtree_fold_at(vals, 1, w.dtype, w.op))
    return bool(np.array_equal(np.ascontiguousarray(got).view(np.uint8),
                               np.ascontiguousarray(want).view(np.uint8)))


DTYPE_TAG = {"float32": "f32", "bfloat16": "bf16", "int32": "i32"}
SAMPLE_COUNT = 1 << 22          # elements per rank of the CPU baseline's sample (large workloads)
METRIC = "AllReduce GB/s + % of HBM peak, N=8 ranks \u00d7 25 MB fp32, 1 MI355X"


def step_bytes(w, algo):
    """HBM bytes one AllReduce moves with each algorithm (K = bytes per rank)."""
    n, k = w.nranks, w.bytes_per_rank
    if algo.endswith("_fused"):
        return 2 * n * k                      # one pass: N*K read + N*K written
    if algo in ("ring_step", "halving_doubling"):
        return 5 * (n - 1) * k                # ReduceScatter 3(N-1)K + AllGather 2(N-1)K
    if algo == "double_tree":
        return (7 * (n // 2 - 1) + 5) * k     # two trees, each over half the vector
    return 2 * n * k * (n.bit_length() - 1)   # log2 N steps of 2*N*K


def sweep(args):
    """64 ranks, fp32 U[-1, 1], SUM, 4 KiB .. 64 MiB per rank: time each
    algorithm and fit T(K) = a + b*K (the alpha-beta model: a = launches x
    alpha, b = bytes-per-K / bandwidth)."""
    import numpy as np
    import torch

    import ring_allreduce_rs_amd as ar
    import workloads as W
    base = ("ring_step", "tree", "halving_doubling", "double_tree", "ring_fused", "tree_fused",
            "halving_doubling_fused", "double_tree_fused")
    # "+graph": the same algorithm replayed from a library-recorded HIP graph
    algos = base + tuple(a + "+graph" for a in base[:4])
    launches = {"ring_step": 2 * 63, "tree": 6, "halving_doubling": 12, "double_tree": 12,
                "ring_fused": 1, "tree_fused": 1, "halving_doubling_fused": 1,
                "double_tree_fused": 1}
    launches.update({a + "+graph": launches[a] for a in base[:4]})
    rows = {a: [] for a in algos}
    for w in W.SWEEP:
        set_bytes = w.nranks * w.bytes_per_rank
        nsets = max(2, min(16, -(-4 * INFINITY_CACHE_BYTES // set_bytes)))
        sets = [W.device_inputs(w, seed=s) for s in range(nsets)]
        steps = max(10, min(200, int(2e9 // max(set_bytes, 1))))
        for algo in algos:
            name, graph = algo.split("+")[0], algo.endswith("+graph")
            ar.set_graphs(graph, max_bytes_per_rank=ALWAYS_REPLAY)
            wall, ms = time_algo(ar, sets, w, name, steps, 5)
            ar.set_graphs(False)
            t = wall / steps
            rows[algo].append((w.bytes_per_rank, t))
            print(json.dumps({"sweep": w.name, "algo": algo, "nranks": w.nranks,
                              "bytes_per_rank": w.bytes_per_rank, "rotating_sets": nsets,
                              "steps": steps, "us_per_allreduce": round(t * 1e6, 3),
                              "event_us": round(ms * 1e3, 3),
                              "GBps_algorithmic": round(2 * set_bytes / t / 1e9, 2),
                              "GBps_bytes_moved": round(step_bytes(w, name) / t / 1e9, 2)}),
                  flush=True)
        del sets
        torch.cuda.empty_cache()
    fit = {}
    for algo in algos:
        k = np.array([r[0] for r in rows[algo]], dtype=np.float64)
        t = np.array([r[1] for r in rows[algo]], dtype=np.float64)
        b, a = np.polyfit(k, t, 1)
        fit[algo] = {"a_us": round(a * 1e6, 3), "b_us_per_MiB": round(b * 1e6 * (1 << 20), 4),
                     "alpha_us_per_launch": round(a * 1e6 / launches[algo], 3),
                     "launches": launches[algo],
                     "bytes_moved_GBps": round(step_bytes(W.SWEEP[-1], algo.split("+")[0])
                                               / W.SWEEP[-1].bytes_per_rank / b / 1e9, 1)}
    cross = {}
    for x, y in (("ring_step", "tree"), ("halving_doubling", "tree"), ("ring_step", "ring_fused"),
                 ("ring_step+graph", "tree+graph")):
        ax, bx = fit[x]["a_us"], fit[x]["b_us_per_MiB"]
        ay, by = fit[y]["a_us"], fit[y]["b_us_per_MiB"]
        cross[f"{x}_vs_{y}_MiB"] = (round((ay - ax) / (bx - by), 3) if bx != by else None)
    print(json.dumps({"sweep_fit": fit, "crossover_bytes_per_rank": cross,
                      "model": "T(K) = a + b*K fitted over the five sizes; a / launches = alpha"}),
          flush=True)


def size_sweep(w):
    """The fused AllReduce against its access pattern's ceiling over sizes."""
    import numpy as np
    import torch

    import ring_allreduce_rs_amd as ar
    import workloads as W

    def ev_time(fn, nsets, reps):
        for i in range(nsets):
            fn(i)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for i in range(reps):
            fn(i % nsets)
        e.record()
        torch.cuda.synchronize()
        return s.elapsed_time(e) / reps * 1e3

    n, eb = w.nranks, w.itemsize
    rows = []
    for mib in (0.78125, 1.5625, 3.125, 6.25, 12.5, 25, 50, 100, 200, 400):
        count = int(mib * (1 << 20)) // eb
        kb = count * eb
        ws = W.Workload(f"{w.name}@{mib}MiB", n, count, w.dtype, w.dist, w.op)
        # at most 32 sets: the binding's pointer-set cache holds 32, and a call
        # whose set fell out of it re-validates its pointers through the
        # runtime, which at the small sizes takes longer than the kernel
        nsets = min(32, max(2, -(-4 * INFINITY_CACHE_BYTES // (n * kb))))
        sets = [W.device_inputs(ws, seed=s) for s in range(nsets)]
        calls = [ar.bind(ts, op=w.op, algo="ring_fused") for ts in sets]
        streams = [ar.bind_stream(ts, ts) for ts in sets]
        reps = max(20, min(400, int(4e9 // (2 * n * kb))))
        t_f = ev_time(lambda i: calls[i](), nsets, reps)
        t_s = ev_time(lambda i: streams[i](), nsets, reps)
        flat = [torch.empty(n * kb, dtype=torch.uint8, device="cuda") for _ in range(2 * nsets)]
        t_c = ev_time(lambda i: ar.copy_(flat[2 * i], flat[2 * i + 1]), nsets, reps)
        del sets, calls, streams, flat
        torch.cuda.empty_cache()
        nbytes = 2 * n * kb
        rows.append((nbytes, t_f, t_s, t_c))
        print(json.dumps({"size_sweep": w.name, "MiB_per_rank": mib, "bytes": nbytes,
                          "rotating_sets": nsets, "launches": reps,
                          "fused_us": round(t_f, 2), "stream_in_place_us": round(t_s, 2),
                          "copy_us": round(t_c, 2),
                          "fused_frac": round(nbytes / t_f / 1e3 / HBM_PEAK_GBPS, 4),
                          "stream_frac": round(nbytes / t_s / 1e3 / HBM_PEAK_GBPS, 4),
                          "copy_frac": round(nbytes / t_c / 1e3 / HBM_PEAK_GBPS, 4),
                          "fused_vs_stream": round(t_s / t_f, 4)}), flush=True)
    r = np.array(rows)
    sel = r[:, 0] >= 5e7
    fit = {}
    for j, name in ((1, "fused"), (2, "stream_in_place"), (3, "copy")):
        b, a = np.polyfit(r[sel, 0], r[sel, j], 1)
        fit[name] = {"a_us": round(a, 2), "GBps": round(1 / b / 1e3, 1),
                     "frac": round(1 / b / 1e3 / HBM_PEAK_GBPS, 4)}
    print(json.dumps({"size_sweep_fit": fit,
                      "model": "T = a + bytes / GBps, fitted over sizes with >= 50 MB moved"}),
          flush=True)


def lds_for_waves(waves):
    """The LDS reservation that holds a compute unit at `waves` one-wave blocks:
    160 KiB / (waves + 1/2), rounded down to 256 bytes (0: no reservation)."""
    return 0 if waves == 0 else (2 * (160 << 10) // (2 * waves + 1)) & ~255


def timeline(w, caps=(5, 0), launches=24, keep=4):
    """Where a one-pass launch spends its time: the in-place calibration stream
    over the workload's buffers (the fused AllReduce's access pattern without
    the reduction) with a per-block start / end on the device's wall clock."""
    import numpy as np
    import torch

    import ring_allreduce_rs_amd as ar

    n = w.nranks
    nbytes = w.count * w.itemsize // 16 * 16
    nsets = max(2, -(-4 * INFINITY_CACHE_BYTES // (n * nbytes)))
    sets = [[torch.full((nbytes // 4,), s * n + r, dtype=torch.int32, device="cuda")
             for r in range(n)] for s in range(nsets)]
    blocks = -(-nbytes // 1024)
    ts = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
    per_block = 2 * n * 1024          # bytes one block reads and writes
    for waves in caps:
        lds = lds_for_waves(waves)
        for it in range(launches):
            nblk, khz = ar.stream_timeline(sets[it % nsets], lds, ts)
            if it < launches - keep:
                continue
            torch.cuda.synchronize()
            t = ts.view(-1, 2).cpu().numpy().astype(np.float64) / (khz / 1e3)   # us
            t -= t[:, 0].min()
            start, end = t[:, 0], t[:, 1]
            span = float(end.max())
            lo, hi = 0.25 * span, 0.75 * span
            rate = float(((end >= lo) & (end < hi)).sum()) / (hi - lo)          # blocks per us
            resident = float((np.clip(end, lo, hi) - np.clip(start, lo, hi)).sum()) / (hi - lo)
            edges = np.linspace(0.0, span, 21)
            active = [int(((start <= x) & (end > x)).sum()) for x in edges[:-1]]
            steady = rate * per_block / 1e3                                    # GB/s
            print(json.dumps({
                "timeline": w.name, "waves_per_cu_cap": waves or None, "lds_bytes": lds,
                "blocks": nblk, "bytes_moved": 2 * n * nbytes, "span_us": round(span, 2),
                "span_frac_hbm_peak": round(2 * n * nbytes / span / 1e3 / HBM_PEAK_GBPS, 4),
                "steady_blocks_per_us": round(rate, 1), "steady_GBps": round(steady, 1),
                "steady_frac_hbm_peak": round(steady / HBM_PEAK_GBPS, 4),
                "us_over_steady": round(span - nblk / rate, 2),
                "first_block_done_us": round(float(end.min()), 2),
                "last_block_start_us": round(float(start.max()), 2),
                "block_us_p10_p50_p90": [round(float(np.percentile(end - start, q)), 2)
                                         for q in (10, 50, 90)],
                "resident_blocks_mid": round(resident, 1),
                "active_blocks_per_5pct_of_span": active}), flush=True)


def main():
    args, w = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: every logical rank lives in one GPU's HBM, so "
              f"--gpus {args.gpus} is not a configuration of this path (use --gpus 1).",
              file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        return sweep(args)
    if args.size_sweep:
        return size_sweep(w)
    if args.timeline:
        return timeline(w)
    import numpy as np
    import torch

    import ring_allreduce_rs_amd as ar
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.algo not in ("ring_fused", "ring_step") and w.nranks & (w.nranks - 1):
        print(f"{args.algo} needs a power-of-two rank count", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    ar.set_residency_caps(not args.no_residency_caps)
    set_bytes = w.nranks * w.bytes_per_rank
    # enough sets to exceed the Infinity Cache 4x; at most 32 (small workloads
    # are cache-resident anyway) and at most 64 GiB of buffers
    nsets = args.sets or min(32, max(2, -(-4 * INFINITY_CACHE_BYTES // set_bytes)))
    nsets = max(1, min(nsets, (64 << 30) // max(set_bytes, 1)))
    host = W.host_inputs(w, seed=args.seed) if set_bytes <= (1 << 30) else None
    torch_dt = {"int32": torch.int32, "float32": torch.float32, "bfloat16": torch.bfloat16}[w.dtype]

    def upload(x):
        if w.dtype == "bfloat16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda")
        return torch.from_numpy(x).to("cuda")

    def download(t):
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).cpu().numpy().view(np.uint16)
        return t.cpu().numpy()

    sets = []
    for s in range(nsets):
        if s == 0 and host is not None:
            sets.append([upload(x) for x in host])
        else:
            sets.append(W.device_inputs(w, seed=args.seed + s))
    assert all(t.dtype == torch_dt for ts in sets for t in ts)

    # Full-size workloads too large for a whole oracle run: keep the first
    # SAMPLE_COUNT inputs of every rank (the CPU baseline's sample) and the
    # inputs at sampled positions (the parity check), both taken before the
    # first AllReduce, which works in place.
    sample_host = idx = vals = None
    if host is None:
        rng = np.random.Generator(np.random.PCG64(args.seed + 99))
        idx = np.unique(np.concatenate([
            rng.integers(0, w.count, size=4096),
            np.array([0, w.count - 1, (w.count + 1) // 2 - 1, (w.count + 1) // 2]),
            # both sides of every chunk boundary (ceil(count / N) apart)
            np.array([c * -(-w.count // w.nranks) + d for c in range(1, w.nranks)
                      for d in (-1, 0) if 0 <= c * -(-w.count // w.nranks) + d < w.count],
                     dtype=np.int64)])).astype(np.int64)
        ti = torch.from_numpy(idx).to("cuda")
        vals = np.stack([download(t.index_select(0, ti)) for t in sets[0]])
        if not args.no_cpu_baseline:
            sample_host = [download(t[:SAMPLE_COUNT]) for t in sets[0]]

    # first AllReduce of set 0, kept for the parity check
    ar.allreduce(sets[0], op=w.op, algo=args.algo)
    torch.cuda.synchronize()
    gpu_first = [download(t) for t in sets[0]] if host is not None else None
    got_at = same = None
    if host is None:
        got_at = download(sets[0][0].index_select(0, torch.from_numpy(idx).to("cuda")))
        same = all(torch.equal(t, sets[0][0]) for t in sets[0][1:])

    wall, ms = time_algo(ar, sets, w, args.algo, args.steps, args.warmup)
    alg_bytes = 2 * w.nranks * w.bytes_per_rank
    value = alg_bytes * args.steps / wall / 1e9
    t_step = wall / args.steps
    stat_groups = max(5, min(args.steps // LAUNCH_GROUP, 40))
    med, mn, _ = launch_stats(ar, sets, w, args.algo, stat_groups)
    achieved = alg_bytes / (ms * 1e-3) / 1e9
    key = f"{w.name}/{args.algo}"
    # the committed counters were taken on the capped kernels
    traffic = None if args.no_residency_caps else measured_traffic(key)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE_TAG[w.dtype],
        "data": "synthetic",
        "config": {
            "workload": w.name, "nranks": w.nranks, "count_per_rank": w.count,
            "bytes_per_rank": w.bytes_per_rank, "op": w.op, "algo": args.algo,
            "distribution": list(w.dist), "rotating_sets": nsets, "seed": args.seed,
            "residency_caps": not args.no_residency_caps,
        },
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "algbw_GBps": round(w.bytes_per_rank / t_step / 1e9, 2),
        "busbw_GBps": round(2 * (w.nranks - 1) / w.nranks * w.bytes_per_rank / t_step / 1e9, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel": {"ring_fused": "k_fused", "ring_step": "k_rs_step/k_ag_step",
                       "tree": "k_tree_step",
                       "halving_doubling": "k_hd_rs_step/k_hd_ag_step",
                       "double_tree": "k_dtree_step", "tree_fused": "k_fused",
                       "halving_doubling_fused": "k_fused",
                       "double_tree_fused": "k_fused"}[args.algo],
            "us_per_launch": round(ms * 1e3, 3),
            "us_per_launch_median": round(med * 1e3, 3),
            "us_per_launch_min": round(mn * 1e3, 3),
            "frac_median": round(alg_bytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "per_launch_pass": (f"{stat_groups} groups of {LAUNCH_GROUP} launches over the same "
                                "bucket sets after the timed region, one HIP event between "
                                "groups; median and min over the groups of time / launches"),
            "algorithmic_bytes_per_launch": alg_bytes,
        },
        "gpu": torch.cuda.get_device_properties(0).name,
    }
    if not args.no_others:
        others = {}
        for algo in ("ring_fused", "ring_step", "tree", "halving_doubling", "double_tree",
                     "tree_fused", "halving_doubling_fused", "double_tree_fused"):
            if algo == args.algo or (algo not in ("ring_fused", "ring_step")
                                     and w.nranks & (w.nranks - 1)):
                continue
            reps = max(5, min(args.steps // 4, 100))
            for graph in ((False, True) if not algo.endswith("_fused") else (False,)):
                ar.set_graphs(graph, max_bytes_per_rank=ALWAYS_REPLAY)
                wl, m = time_algo(ar, sets, w, algo, reps, 3)
                ar.set_graphs(False)
                others[algo + ("_graph" if graph else "")] = {
                    "us_per_allreduce": round(wl / reps * 1e6, 2),
                    "GBps_algorithmic": round(alg_bytes * reps / wl / 1e9, 2),
                    "GBps_bytes_moved": round(step_bytes(w, algo) * reps / wl / 1e9, 2),
                    "event_us_per_allreduce": round(m * 1e3, 2),
                }
        # the two halves on their own (fused kernels): ReduceScatter reads every
        # rank's chunks and writes the owner's (N*K + K bytes); AllGather reads
        # the owners' chunks and writes the other N-1 copies (N*K bytes)
        for kind, nbytes in (("reduce_scatter", (w.nranks + 1) * w.bytes_per_rank),
                             ("allgather", w.nranks * w.bytes_per_rank)):
            reps = max(5, min(args.steps // 4, 100))
            wl, m = time_algo(ar, sets, w, "ring_fused", reps, 3, kind=kind)
            others[kind + "_fused"] = {
                "us_per_call": round(wl / reps * 1e6, 2),
                "algorithmic_bytes": nbytes,
                "GBps_algorithmic": round(nbytes * reps / wl / 1e9, 2),
                "event_us_per_call": round(m * 1e3, 2),
                "frac_hbm_peak": round(nbytes / (m * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            }
        cg, cms = copy_ceiling(ar, w.nranks * w.bytes_per_rank)
        others["copy_ceiling"] = {"GBps": round(cg, 2), "bytes": 2 * w.nranks * w.bytes_per_rank,
                                  "us": round(cms * 1e3, 2),
                                  "frac_hbm_peak": round(cg / HBM_PEAK_GBPS, 4)}
        # R-read / W-write streams of K bytes per buffer with the fused
        # kernel's tiling and no reduction: N/N is the ceiling of the fused
        # AllReduce's access pattern; the others separate reads from writes
        n = w.nranks
        streams = {}
        for ns, nd, inpl in ((n, n, True), (n, n, False), (1, 1, False), (n, 0, False),
                             (0, n, False), (n, 1, False), (1, n, False)):
            if ns + nd > 64 and not inpl:
                continue
            g, sms = stream_ceiling(ar, ns, nd, w.bytes_per_rank, in_place=inpl)
            streams[f"{ns}R{nd}W" + ("_in_place" if inpl else "")] = {
                "GBps": round(g, 2), "us": round(sms * 1e3, 2),
                "frac_hbm_peak": round(g / HBM_PEAK_GBPS, 4)}
        others["stream_ceiling"] = streams
        if args.algo.endswith("_fused"):
            # event time of the in-place N-read / N-write stream over the
            # fused AllReduce's mean event time: 1.0 = at that ceiling
            others["fused_vs_stream"] = round(streams[f"{n}R{n}W_in_place"]["us"] / (ms * 1e3), 4)
        out["others"] = others
    parity = None
    if not args.no_cpu_baseline:
        # the CPU leg: the oracle timed, and the GPU's first result checked
        # against it (whole, or at the sampled positions)
        if host is not None:
            cb, ok = cpu_baseline(w, args.algo, host, gpu_first, args.cpu_seconds)
            parity = "bitwise (whole workload)" if ok else "MISMATCH"
        else:
            cb, _ = cpu_baseline(w, args.algo, sample_host, None, args.cpu_seconds,
                                 sample_count=SAMPLE_COUNT)
            parity = (f"bitwise at {idx.size} sampled positions (rank 0), every rank identical"
                      if sampled_parity(w, args.algo, vals, idx, got_at) and same
                      else "MISMATCH")
        cb["host_cpus"] = os.cpu_count()
        cb["host_mem_available_GiB"] = host_mem_available_gib()
        out["cpu_baseline"] = cb
    out["parity_vs_oracle"] = parity
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
