"""The library's calls can be captured in a HIP graph and replayed: they
allocate nothing, never synchronise and record only kernel launches on the
caller's stream.  Every replay is checked against the oracle, with eager work
(re-loading the inputs) and synchronisations between replays."""

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_rs_amd as ar
from tests.gpu_helpers import assert_bits_equal, to_gpu, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SIMS = {"ring_step": oracle.simulate_ring_allreduce, "ring_fused": oracle.simulate_ring_allreduce,
        "tree": oracle.simulate_tree_allreduce, "halving_doubling": oracle.simulate_hd_allreduce,
        "double_tree": oracle.simulate_double_tree_allreduce}


@pytest.mark.parametrize("algo", sorted(SIMS))
@pytest.mark.parametrize("dtype,op", [("float32", "avg"), ("bfloat16", "sum"), ("int32", "max")])
def test_captured_allreduce_replays_match_oracle(algo, dtype, op):
    n, count = 8, 12_347
    rng = np.random.Generator(np.random.PCG64(count))
    inputs = []
    for rep in range(3):
        if dtype == "int32":
            xs = [rng.integers(-10**6, 10**6, size=count).astype(np.int32) for _ in range(n)]
        else:
            f = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
            xs = f if dtype == "float32" else [
                torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                for x in f]
        inputs.append(xs)
    src = [to_gpu(xs, dtype) for xs in inputs]
    ts = [torch.empty_like(t) for t in src[0]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for t, s in zip(ts, src[0]):
            t.copy_(s)
        ar.allreduce(ts, op=op, algo=algo)         # warm-up on the capture stream
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            ar.allreduce(ts, op=op, algo=algo)
    torch.cuda.synchronize()
    for rep, xs in enumerate(inputs):
        for t, s in zip(ts, src[rep]):                # eager work between replays
            t.copy_(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = SIMS[algo](xs, dtype, op).state
        for r in range(n):
            assert_bits_equal(to_np(ts[r]), want[r], f"{algo} replay {rep} rank {r}")


@pytest.mark.parametrize("dtype,op,count", [("float32", "avg", (4 << 20) + 3),
                                            ("bfloat16", "sum", (8 << 20) + 13)])
def test_captured_capped_allreduce_replays_match_oracle(dtype, op, count):
    """A call just above 128 MiB runs the residency-capped kernel, whose LDS
    reservation is part of the recorded launch: every replay matches."""
    n = 8
    rng = np.random.Generator(np.random.PCG64(count + 1))
    inputs = []
    for rep in range(3):
        f = [rng.standard_normal(count, dtype=np.float32) for _ in range(n)]
        inputs.append(f if dtype == "float32" else [
            torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            for x in f])
    src = [to_gpu(xs, dtype) for xs in inputs]
    ts = [torch.empty_like(t) for t in src[0]]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for t, s in zip(ts, src[0]):
            t.copy_(s)
        ar.allreduce(ts, op=op, algo="ring_fused")      # warm-up on the capture stream
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            ar.allreduce(ts, op=op, algo="ring_fused")
    torch.cuda.synchronize()
    for rep, xs in enumerate(inputs):
        for t, s in zip(ts, src[rep]):                # eager work between replays
            t.copy_(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.ordered_ring_fold(xs, dtype, op)
        for r in (0, n - 1):
            assert_bits_equal(to_np(ts[r]), want, f"capped replay {rep} rank {r}")
        assert ar.check(ts)["mismatched"] == 0
    del src, ts, g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("coll", ["allgather", "reduce_scatter"])
def test_captured_capped_allgather_and_reduce_scatter_replay(coll):
    """The AllGather and ReduceScatter just above 128 MiB run their own capped
    PACED kernels (14 and 10 waves per CU); captured by the caller, every
    replay matches the oracle."""
    n, count, dtype = 8, (4 << 20) + 3, "float32"
    rng = np.random.Generator(np.random.PCG64(count + len(coll)))
    inputs = [[rng.standard_normal(count, dtype=np.float32) for _ in range(n)] for _ in range(3)]
    src = [to_gpu(xs, dtype) for xs in inputs]
    ts = [torch.empty_like(t) for t in src[0]]

    def call():
        if coll == "allgather":
            ar.allgather(ts, algo="ring_fused")
        else:
            ar.reduce_scatter(ts, op="sum", algo="ring_fused")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for t, s in zip(ts, src[0]):
            t.copy_(s)
        call()                                          # warm-up on the capture stream
        side.synchronize()
        with torch.cuda.graph(g, stream=side):
            call()
    torch.cuda.synchronize()
    for rep, xs in enumerate(inputs):
        for t, s in zip(ts, src[rep]):                  # eager work between replays
            t.copy_(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if coll == "allgather":
            want = oracle.simulate_ring_allgather(xs, dtype).state
            for r in (0, 3, n - 1):
                assert_bits_equal(to_np(ts[r]), want[r], f"AllGather replay {rep} rank {r}")
        else:
            want = oracle.ordered_ring_fold(xs, dtype, "sum")
            for r, (lo, ln) in enumerate(oracle.chunk_layout(count, n)):
                assert_bits_equal(to_np(ts[r][lo:lo + ln]), want[lo:lo + ln],
                                  f"ReduceScatter replay {rep} owner {r}")
    del src, ts, g
    torch.cuda.empty_cache()
