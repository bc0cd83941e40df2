"""Graph replay inside the library (ar_set_graphs): the multi-launch
algorithms record their kernel sequence once per pointer set and shape and
replay it as one HIP graph.  Every replay is checked against the oracle, with
fresh inputs loaded eagerly and the stream synchronised between replays; the
graph cache's eviction and the fallback under a caller's own capture are
covered too."""

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_rs_amd as ar
from tests.gpu_helpers import assert_bits_equal, to_gpu, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

AR_SIMS = {"ring_step": oracle.simulate_ring_allreduce,
           "tree": oracle.simulate_tree_allreduce,
           "halving_doubling": oracle.simulate_hd_allreduce,
           "double_tree": oracle.simulate_double_tree_allreduce}
RS_SIMS = {"ring_step": oracle.simulate_ring_reduce_scatter,
           "halving_doubling": oracle.simulate_hd_reduce_scatter}
AG_SIMS = {"ring_step": oracle.simulate_ring_allgather,
           "halving_doubling": oracle.simulate_hd_allgather}


def _inputs(n, count, dtype, seed, reps=3):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(reps):
        if dtype == "int32":
            xs = [rng.integers(-10**6, 10**6, size=count).astype(np.int32) for _ in range(n)]
        else:
            f = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
            xs = f if dtype == "float32" else [
                torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                for x in f]
        out.append(xs)
    return out


@pytest.fixture
def graphs_on():
    ar.set_graphs(True)
    yield
    ar.set_graphs(False)


def _replays(kind, algo, n, count, dtype, op, want_of):
    inputs = _inputs(n, count, dtype, seed=count * 7 + n)
    src = [to_gpu(xs, dtype) for xs in inputs]
    ts = [torch.empty_like(t) for t in src[0]]
    for rep, xs in enumerate(inputs):
        for t, s in zip(ts, src[rep]):                 # eager work between replays
            t.copy_(s)
        torch.cuda.synchronize()
        if kind == "allreduce":
            ar.allreduce(ts, op=op, algo=algo)
        elif kind == "reduce_scatter":
            ar.reduce_scatter(ts, op=op, algo=algo)
        else:
            ar.allgather(ts, algo=algo)
        torch.cuda.synchronize()
        want_of(xs, [to_np(t) for t in ts], f"{kind} {algo} replay {rep}")


@pytest.mark.parametrize("algo", sorted(AR_SIMS))
@pytest.mark.parametrize("dtype,op", [("float32", "avg"), ("bfloat16", "sum"), ("int32", "max")])
@pytest.mark.parametrize("count", [1, 4099, 65_537])
def test_replayed_allreduce_matches_oracle(graphs_on, algo, dtype, op, count):
    n = 8

    def check(xs, got, what):
        want = AR_SIMS[algo](xs, dtype, op).state
        for r in range(n):
            assert_bits_equal(got[r], want[r], f"{what} rank {r}")

    _replays("allreduce", algo, n, count, dtype, op, check)


@pytest.mark.parametrize("algo", sorted(RS_SIMS))
@pytest.mark.parametrize("n,count", [(4, 1001), (16, 70_001)])
def test_replayed_reduce_scatter_matches_oracle(graphs_on, algo, n, count):
    layout = oracle.chunk_layout(count, n)

    def check(xs, got, what):
        want = RS_SIMS[algo](xs, "float32", "sum").state
        for r, (lo, ln) in enumerate(layout):       # the owner's chunk is specified
            assert_bits_equal(got[r][lo:lo + ln], want[r][lo:lo + ln], f"{what} rank {r}")

    _replays("reduce_scatter", algo, n, count, "float32", "sum", check)


@pytest.mark.parametrize("algo", sorted(AG_SIMS))
@pytest.mark.parametrize("n,count", [(4, 1001), (16, 70_001)])
def test_replayed_allgather_matches_oracle(graphs_on, algo, n, count):
    def check(xs, got, what):
        want = AG_SIMS[algo](xs, "bfloat16").state
        for r in range(n):
            assert_bits_equal(got[r], want[r], f"{what} rank {r}")

    _replays("allgather", algo, n, count, "bfloat16", None, check)


def test_cache_eviction_rerecords(graphs_on):
    """More distinct shapes than the cache holds (64): evicted graphs are
    released and recorded again on their next call."""
    n, base = 4, 200
    counts = list(range(base, base + 70)) + list(range(base, base + 8))
    xs_full = [np.random.Generator(np.random.PCG64(r)).integers(-1000, 1000, size=base + 80)
               .astype(np.int32) for r in range(n)]
    src = to_gpu(xs_full, "int32")
    ts = [torch.empty_like(t) for t in src]
    for count in counts:
        for t, s in zip(ts, src):
            t.copy_(s)
        views = [t[:count] for t in ts]
        ar.allreduce(views, op="sum", algo="ring_step")
        torch.cuda.synchronize()
        want = oracle.exact_int_sum([x[:count] for x in xs_full])
        for r in range(n):
            assert_bits_equal(to_np(ts[r])[:count], want, f"count {count} rank {r}")
            assert_bits_equal(to_np(ts[r])[count:], xs_full[r][count:],
                              f"count {count} rank {r} beyond the view")


def test_caller_capture_falls_back_to_direct_launches(graphs_on):
    """With graphs on, a call on a stream the caller is capturing launches its
    kernels directly, so they become part of the caller's graph."""
    n, count, dtype, op, algo = 8, 12_347, "float32", "avg", "double_tree"
    inputs = _inputs(n, count, dtype, seed=5)
    src = [to_gpu(xs, dtype) for xs in inputs]
    ts = [torch.empty_like(t) for t in src[0]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for t, s in zip(ts, src[0]):
            t.copy_(s)
        ar.allreduce(ts, op=op, algo=algo)          # records a library graph (not capturing)
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            ar.allreduce(ts, op=op, algo=algo)
    torch.cuda.synchronize()
    for rep, xs in enumerate(inputs):
        for t, s in zip(ts, src[rep]):
            t.copy_(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = AR_SIMS[algo](xs, dtype, op).state
        for r in range(n):
            assert_bits_equal(to_np(ts[r]), want[r], f"caller graph replay {rep} rank {r}")


def test_turning_graphs_off_releases_and_keeps_results(graphs_on):
    n, count = 8, 3001
    inputs = _inputs(n, count, "float32", seed=11, reps=2)
    ts = to_gpu(inputs[0], "float32")
    ar.allreduce(ts, op="sum", algo="halving_doubling")       # recorded and replayed
    torch.cuda.synchronize()
    ar.set_graphs(False)                                      # releases the graphs
    ts2 = to_gpu(inputs[1], "float32")
    ar.allreduce(ts2, op="sum", algo="halving_doubling")      # direct launches
    torch.cuda.synchronize()
    for xs, t in ((inputs[0], ts), (inputs[1], ts2)):
        want = oracle.simulate_hd_allreduce(xs, "float32", "sum").state
        for r in range(n):
            assert_bits_equal(to_np(t[r]), want[r], f"rank {r}")


def test_threshold_limits_replay_to_small_collectives():
    """Above the per-rank byte threshold the call launches directly; both
    sides of the threshold give the oracle's bits."""
    n = 8
    ar.set_graphs(True, max_bytes_per_rank=4096)
    try:
        for count in (1024, 1025, 50_000):          # 4096 B (replayed), 4100 B, 200 KB
            xs = _inputs(n, count, "float32", seed=count, reps=1)[0]
            for rep in range(2):
                ts = to_gpu(xs, "float32")
                ar.allreduce(ts, op="avg", algo="ring_step")
                torch.cuda.synchronize()
                want = oracle.simulate_ring_allreduce(xs, "float32", "avg").state
                for r in range(n):
                    assert_bits_equal(to_np(ts[r]), want[r], f"count {count} call {rep} rank {r}")
    finally:
        ar.set_graphs(False)
