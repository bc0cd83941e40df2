"""GPU parity of the residency-capped fused shapes against the oracle.

The PACED shape (one 16-byte unit per lane, an LDS reservation capping the
waves per compute unit) and the capped DEEP shape only run on calls above a
size threshold: more than 128 MiB over all ranks for PACED, 256 MiB for the
DEEP cap, 512 MiB for the AllGather's PACED shape beyond 8 ranks.  Each case
here sits just above its threshold and picks one kernel form: the compiled
8-rank loop or the run-time rank count, plain or line-aligned indexing (ragged
counts put chunk starts off 16-byte units and off 128-byte lines), every fold
order, ReduceScatter, AllGather under each of its caps, every dtype and op,
and AVG with a rank count that is not a power of two.  For the AllReduce every
position of rank 0 is compared bit for bit with the oracle's fold and the
on-device checker confirms that every rank holds the same bits; the
AllGather compares every rank with the oracle's ring AllGather.
"""

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_rs_amd as ar
from tests.gpu_helpers import assert_bits_equal, to_gpu, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MIB = 1 << 20


def inputs(dtype, n, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    if dtype == "int32":
        return [rng.integers(-2**31, 2**31, size=count, dtype=np.int64).astype(np.int32)
                for _ in range(n)]
    f = [rng.standard_normal(count, dtype=np.float32) * np.float32(rng.choice([1e-3, 1.0]))
         for _ in range(n)]
    if dtype == "float32":
        return f
    return [torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            for x in f]


def total_bytes(dtype, n, count):
    return n * count * (2 if dtype == "bfloat16" else 4)


# (ranks, dtype, op, count): the count puts the call just above its threshold
RING_CASES = [
    (8, "float32", "sum", 4 * MIB + 3),            # 8-rank loop, line-aligned (ragged)
    (8, "float32", "max", 4 * MIB + 8192),         # 8-rank loop, plain indexing
    (8, "int32", "max", 4 * MIB + 77),
    (8, "bfloat16", "sum", 8 * MIB + 1024),        # bf16 PACED, plain indexing
    (8, "bfloat16", "avg", 8 * MIB + 13),          # bf16 PACED, line-aligned
    (8, "bfloat16", "max", 8 * MIB + 13),          # bf16 MAX: DEEP without a cap
    (10, "float32", "avg", 3355457),               # run-time N, AVG by division
    (12, "int32", "sum", 2796208),                 # run-time N, 256 B over the threshold
    (32, "float32", "max", 2 * MIB + 3),           # DEEP capped (fp32 MAX)
    (64, "int32", "sum", MIB + 5),                 # DEEP capped
    (32, "bfloat16", "sum", 4 * MIB + 7),          # DEEP capped (bf16)
    (16, "bfloat16", "avg", 8 * MIB + 3),          # DEEP capped (bf16, 16 ranks)
]


def run_allreduce(xs, dtype, op, algo):
    ts = to_gpu(xs, dtype)
    ar.allreduce(ts, op=op, algo=algo)
    torch.cuda.synchronize()
    r = ar.check(ts)
    assert r["mismatched"] == 0, (algo, r)
    got = to_np(ts[0])
    del ts
    torch.cuda.empty_cache()
    return got


@pytest.mark.parametrize("n,dtype,op,count", RING_CASES,
                         ids=[f"n{c[0]}-{c[1]}-{c[2]}-{c[3]}" for c in RING_CASES])
def test_capped_ring_allreduce_matches_oracle(n, dtype, op, count):
    threshold = 256 * MIB if n > 16 or (n == 16 and dtype == "bfloat16") else 128 * MIB
    assert total_bytes(dtype, n, count) > threshold
    xs = inputs(dtype, n, count, seed=n * 131 + count)
    want = oracle.ordered_ring_fold(xs, dtype, op)
    assert_bits_equal(run_allreduce(xs, dtype, op, "ring_fused"), want, f"n={n} {dtype} {op}")


# The one-pass tree orders over 8 ranks (their PACED 8-rank kernels), ragged
@pytest.mark.parametrize("dtype,op", [("float32", "sum"), ("float32", "max"), ("int32", "sum")])
def test_capped_tree_orders_match_oracle(dtype, op):
    n, count = 8, 4 * MIB + 3
    xs = inputs(dtype, n, count, seed=77 + len(op))
    cases = [("tree_fused", oracle.pairwise_tree_fold(xs, dtype, op)),
             ("halving_doubling_fused", oracle.simulate_hd_allreduce(xs, dtype, op).state[0]),
             ("double_tree_fused", oracle.double_tree_fold(xs, dtype, op))]
    for algo, want in cases:
        assert_bits_equal(run_allreduce(xs, dtype, op, algo), want, f"{algo} {dtype} {op}")


# ReduceScatter over PACED and over capped DEEP (beyond 16 ranks and 256 MiB):
# each owner's chunk
@pytest.mark.parametrize("n,dtype,op,count", [(8, "float32", "sum", 4 * MIB + 3),
                                              (16, "int32", "max", 2 * MIB + 9),
                                              (8, "int32", "sum", 4 * MIB + 4096),
                                              (32, "float32", "avg", 2 * MIB + 3),
                                              (64, "float32", "max", MIB + 5),
                                              (32, "bfloat16", "sum", 4 * MIB + 7),
                                              (24, "int32", "max", 2796203)])
def test_capped_reduce_scatter_matches_oracle(n, dtype, op, count):
    assert total_bytes(dtype, n, count) > 128 * MIB
    xs = inputs(dtype, n, count, seed=n + count)
    want = oracle.ordered_ring_fold(xs, dtype, op)
    ts = to_gpu(xs, dtype)
    ar.reduce_scatter(ts, op=op, algo="ring_fused")
    torch.cuda.synchronize()
    for r, (lo, ln) in enumerate(oracle.chunk_layout(count, n)):
        assert_bits_equal(to_np(ts[r][lo:lo + ln]), want[lo:lo + ln], f"RS owner {r}")
        # a ReduceScatter leaves the other chunks of rank r as they were
        other = np.ones(count, dtype=bool)
        other[lo:lo + ln] = False
        got = to_np(ts[r])
        assert np.array_equal(got[other].view(np.uint8), np.asarray(xs[r])[other].view(np.uint8))
    del ts
    torch.cuda.empty_cache()


# AllGather over PACED: (ranks, dtype, count), each just above its threshold
# (8 ranks: 128 MiB over all ranks; more ranks: 512 MiB): the 8-rank loop, the
# run-time rank count with plain and line-aligned indexing, every cap
AG_CASES = [
    (8, "float32", 4 * MIB + 3),            # 8-rank loop, ragged chunks
    (8, "bfloat16", 8 * MIB + 1024),        # 8-rank loop, aligned chunks
    (16, "int32", 8 * MIB + 512),           # run-time N, plain indexing (cap 8)
    (16, "float32", 8 * MIB + 5),           # run-time N, line-aligned (cap 8)
    (24, "int32", 5592406),                 # cap 5
    (32, "bfloat16", 8 * MIB + 77),         # cap 4
    (64, "float32", 2 * MIB + 7),           # cap 3
]


@pytest.mark.parametrize("n,dtype,count", AG_CASES,
                         ids=[f"n{c[0]}-{c[1]}-{c[2]}" for c in AG_CASES])
def test_capped_allgather_matches_oracle(n, dtype, count):
    threshold = 128 * MIB if n == 8 else 512 * MIB
    assert total_bytes(dtype, n, count) > threshold
    xs = inputs(dtype, n, count, seed=n * 7 + count)
    want = oracle.simulate_ring_allgather(xs, dtype).state
    ts = to_gpu(xs, dtype)
    del xs
    ar.allgather(ts, algo="ring_fused")
    torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_np(ts[r]), want[r], f"AllGather rank {r}")
    del ts
    torch.cuda.empty_cache()


def test_threshold_neighbours_agree():
    """The same AllReduce just below (uncapped WIDE) and just above (PACED)
    the threshold: both equal the oracle, so the shape switch is invisible."""
    n, dtype, op = 8, "float32", "avg"
    for count in (4 * MIB - 16, 4 * MIB + 16):
        xs = inputs(dtype, n, count, seed=count)
        want = oracle.ordered_ring_fold(xs, dtype, op)
        assert_bits_equal(run_allreduce(xs, dtype, op, "ring_fused"), want, f"count {count}")


def test_caps_off_gives_the_same_bits():
    """ar_set_residency_caps(0): the same large calls run the uncapped shapes
    (no LDS reservation) and return the same bits; the calibration stream
    follows the setting and still writes the XOR of its sources."""
    n, count = 8, 4 * MIB + 3
    xs = inputs("float32", n, count, seed=4242)
    want = oracle.ordered_ring_fold(xs, "float32", "avg")
    try:
        ar.set_residency_caps(False)
        assert_bits_equal(run_allreduce(xs, "float32", "avg", "ring_fused"), want, "caps off")
        stream_xor_ok()
        allgather_ok(xs)
    finally:
        ar.set_residency_caps(True)
    assert_bits_equal(run_allreduce(xs, "float32", "avg", "ring_fused"), want, "caps on")
    stream_xor_ok()
    allgather_ok(xs)


def allgather_ok(xs):
    want = oracle.simulate_ring_allgather(xs, "float32").state
    ts = to_gpu(xs, "float32")
    ar.allgather(ts, algo="ring_fused")
    torch.cuda.synchronize()
    for r in range(len(xs)):
        assert_bits_equal(to_np(ts[r]), want[r], f"AllGather rank {r}")


def stream_xor_ok():
    # 8 sources just over 128 MiB in all: the paced shape when caps are on
    srcs = to_gpu(inputs("int32", 8, 4 * MIB + 16, seed=7), "int32")
    dsts = [torch.empty_like(srcs[0]) for _ in range(2)]
    ar.stream_(srcs, dsts)
    torch.cuda.synchronize()
    x = srcs[0].clone()
    for t in srcs[1:]:
        x ^= t
    assert all(torch.equal(d, x) for d in dsts)
