"""Poison test: no kernel writes outside the rank buffers it is given.

Every rank buffer is a view into a larger allocation whose leading and
trailing guard regions hold a sentinel bit pattern; after each collective the
guards must be bit-for-bit unchanged and the views must hold the oracle's
result.  Counts cover ragged chunks, counts below N and empty chunks, and the
views start at several element offsets from a 16-byte boundary, so the
element-wise head and tail paths run next to the guards.  The residency-capped
shapes of the AllReduce, AllGather and ReduceScatter run at the sizes that
select them."""

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_rs_amd as ar
from tests.gpu_helpers import assert_bits_equal, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

GUARD = 67                                     # elements on each side
SENTINEL = {"int32": np.int32(0x7BADBEEF),
            "float32": np.uint32(0x7FBADBAD).view(np.float32),
            "bfloat16": np.uint16(0x7FBB)}

AR_SIMS = {"ring_step": oracle.simulate_ring_allreduce, "ring_fused": oracle.simulate_ring_allreduce,
           "tree": oracle.simulate_tree_allreduce, "halving_doubling": oracle.simulate_hd_allreduce,
           "double_tree": oracle.simulate_double_tree_allreduce,
           "tree_fused": oracle.simulate_tree_allreduce,
           "halving_doubling_fused": oracle.simulate_hd_allreduce,
           "double_tree_fused": oracle.simulate_double_tree_allreduce}


def _inputs(dtype, n, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    if dtype == "int32":
        return [rng.integers(-10**6, 10**6, size=count).astype(np.int32) for _ in range(n)]
    f = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    if dtype == "float32":
        return f
    return [torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            for x in f]


def _guarded(xs, dtype, shift):
    """Per rank: an allocation of GUARD + shift + count + GUARD elements filled
    with the sentinel, with the input copied into the middle; returns the
    full tensors and the views handed to the library."""
    fulls, views = [], []
    for x in xs:
        host = np.full(GUARD + shift + x.size + GUARD, SENTINEL[dtype])
        host[GUARD + shift:GUARD + shift + x.size] = x
        if dtype == "bfloat16":
            t = torch.from_numpy(host.view(np.int16)).view(torch.bfloat16).cuda()
        else:
            t = torch.from_numpy(host).cuda()
        fulls.append(t)
        views.append(t[GUARD + shift:GUARD + shift + x.size])
    return fulls, views


def _check_guards(fulls, dtype, shift, count, what):
    for r, t in enumerate(fulls):
        h = to_np(t)
        assert_bits_equal(h[:GUARD + shift], np.full(GUARD + shift, SENTINEL[dtype]),
                          f"{what}: leading guard of rank {r}")
        assert_bits_equal(h[GUARD + shift + count:], np.full(GUARD, SENTINEL[dtype]),
                          f"{what}: trailing guard of rank {r}")


CASES = [(8, 1), (8, 7), (8, 1001), (3, 10007), (16, 4099), (64, 130), (64, 70_001)]


@pytest.mark.parametrize("algo", sorted(AR_SIMS))
@pytest.mark.parametrize("dtype,op", [("float32", "avg"), ("bfloat16", "sum"), ("int32", "max")])
@pytest.mark.parametrize("n,count", CASES)
def test_allreduce_writes_only_its_buffers(algo, dtype, op, n, count):
    if algo not in ("ring_step", "ring_fused") and n & (n - 1):
        pytest.skip("needs a power-of-two rank count")
    xs = _inputs(dtype, n, count, seed=n * 613 + count)
    want = AR_SIMS[algo](xs, dtype, op).state
    for shift in (0, 1, 3):
        fulls, views = _guarded(xs, dtype, shift)
        ar.allreduce(views, op=op, algo=algo)
        torch.cuda.synchronize()
        what = f"{algo} {dtype} {op} n={n} count={count} shift={shift}"
        _check_guards(fulls, dtype, shift, count, what)
        for r in range(n):
            assert_bits_equal(to_np(views[r]), want[r], f"{what} rank {r}")


@pytest.mark.parametrize("algo", ["ring_step", "ring_fused", "halving_doubling",
                                  "halving_doubling_fused"])
@pytest.mark.parametrize("n,count", CASES)
def test_reduce_scatter_and_allgather_write_only_their_buffers(algo, n, count):
    if algo.startswith("halving_doubling") and n & (n - 1):
        pytest.skip("needs a power-of-two rank count")
    dtype, op = "float32", "sum"
    xs = _inputs(dtype, n, count, seed=n * 919 + count)
    for shift in (0, 2):
        fulls, views = _guarded(xs, dtype, shift)
        ar.reduce_scatter(views, op=op, algo=algo)
        torch.cuda.synchronize()
        _check_guards(fulls, dtype, shift, count, f"RS {algo} n={n} count={count} shift={shift}")
        ar.allgather(views, algo=algo)
        torch.cuda.synchronize()
        _check_guards(fulls, dtype, shift, count, f"AG {algo} n={n} count={count} shift={shift}")
        want = AR_SIMS[algo](xs, dtype, op).state
        for r in range(n):
            assert_bits_equal(to_np(views[r]), want[r], f"RS+AG {algo} n={n} rank {r}")


# The residency-capped shapes (calls above 128 MiB; the AllGather beyond 8
# ranks above 512 MiB; the ReduceScatter's capped DEEP shape beyond 16 ranks
# above 256 MiB), next to guards, with chunk bodies on and off 16-byte units
BIG = [("allreduce", 8, "float32", (4 << 20) + 3, 0), ("allreduce", 8, "float32", (4 << 20) + 3, 3),
       ("allreduce", 16, "int32", (2 << 20) + 5, 1), ("allgather", 8, "float32", (4 << 20) + 3, 2),
       ("allgather", 16, "int32", (8 << 20) + 5, 0), ("reduce_scatter", 8, "float32", (4 << 20) + 3, 1),
       ("reduce_scatter", 32, "int32", (2 << 20) + 7, 2)]


@pytest.mark.parametrize("coll,n,dtype,count,shift", BIG,
                         ids=[f"{c[0]}-n{c[1]}-{c[2]}-s{c[4]}" for c in BIG])
def test_capped_kernels_write_only_their_buffers(coll, n, dtype, count, shift):
    xs = _inputs(dtype, n, count, seed=n * 1000 + count + shift)
    fulls, views = _guarded(xs, dtype, shift)
    op = "avg" if dtype == "float32" and coll == "allreduce" else "sum"
    if coll == "allreduce":
        ar.allreduce(views, op=op, algo="ring_fused")
    elif coll == "allgather":
        ar.allgather(views, algo="ring_fused")
    else:
        ar.reduce_scatter(views, op=op, algo="ring_fused")
    torch.cuda.synchronize()
    _check_guards(fulls, dtype, shift, count, f"{coll} n={n} shift={shift}")
    if coll == "allgather":
        want = oracle.simulate_ring_allgather(xs, dtype).state
        for r in (0, n - 1):
            assert_bits_equal(to_np(views[r]), want[r], f"AllGather rank {r}")
    else:
        want = oracle.ordered_ring_fold(xs, dtype, op)
        if coll == "allreduce":
            for r in (0, n - 1):
                assert_bits_equal(to_np(views[r]), want, f"AllReduce rank {r}")
        else:
            for r, (lo, ln) in enumerate(oracle.chunk_layout(count, n)):
                assert_bits_equal(to_np(views[r][lo:lo + ln]), want[lo:lo + ln], f"RS owner {r}")
    del fulls, views
    torch.cuda.empty_cache()
