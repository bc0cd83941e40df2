"""The on-device result checker (ar_check) against the same quantities
computed on the host with numpy: positions where some rank's bits differ
from rank 0's (count and first), the largest |rank 0 - reference| in
binary64, and the positions over a per-position bound.  Counts span many
blocks of the grid-stride pass and a partial last block."""

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_rs_amd as ar
from ring_allreduce_rs_amd import _lib
from tests.gpu_helpers import to_gpu, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def rand_inputs(dtype, n, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    if dtype == "int32":
        return [rng.integers(-2**20, 2**20, size=count).astype(np.int32) for _ in range(n)]
    f = [(rng.standard_normal(count) * 1e-2).astype(np.float32) for _ in range(n)]
    if dtype == "float32":
        return f
    return [torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
            for x in f]


def widen(x, dtype):
    if dtype == "bfloat16":
        return oracle.bf16_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def host_view(ts):
    a = np.stack([to_np(t) for t in ts])
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.int32 if a.dtype == np.int32
                                                                  else np.uint16)


@pytest.mark.parametrize("dtype", ["int32", "float32", "bfloat16"])
@pytest.mark.parametrize("n,count", [(1, 5), (2, 1000), (8, 2048 * 256 * 2 + 1234), (64, 3001)])
def test_identical_ranks_and_planted_differences(dtype, n, count):
    xs = rand_inputs(dtype, n, count, seed=n + count)
    ts = to_gpu(xs, dtype)
    ar.allreduce(ts, op="sum", algo="ring_fused")
    torch.cuda.synchronize()
    r = ar.check(ts)
    assert r["mismatched"] == 0 and r["first_mismatch"] == count
    assert r["over_bound"] == 0 and r["max_abs_err"] == 0.0
    if n == 1:
        return
    # plant differences in other ranks (bit flips of the low bit)
    plant = {1: [count - 1, 3], n - 1: [count // 2, 3]}
    for rank, pos in plant.items():
        for p in pos:
            if dtype == "bfloat16":
                ts[rank].view(torch.int16)[p] ^= 1
            else:
                ts[rank].view(torch.int32)[p] ^= 1
    torch.cuda.synchronize()
    a = host_view(ts)
    bad = np.nonzero((a != a[0]).any(axis=0))[0]
    r = ar.check(ts)
    assert r["mismatched"] == bad.size
    assert r["first_mismatch"] == int(bad[0])


@pytest.mark.parametrize("dtype", ["int32", "float32", "bfloat16"])
@pytest.mark.parametrize("count", [1, 777, 2048 * 256 * 3 + 17])
def test_error_against_reference_and_bound(dtype, count):
    n = 4
    xs = rand_inputs(dtype, n, count, seed=count)
    ts = to_gpu(xs, dtype)
    ar.allreduce(ts, op="sum", algo="ring_fused")
    torch.cuda.synchronize()
    got = widen(to_np(ts[0]), dtype)
    ref = oracle.fp64_sum(xs, dtype)
    err = np.abs(got - ref)
    rng = np.random.Generator(np.random.PCG64(5))
    bound = err * rng.choice([0.5, 1.0, 2.0], size=count)      # some over, some equal, some under
    r = ar.check(ts, ref=torch.from_numpy(ref).cuda(), bound=torch.from_numpy(bound).cuda())
    assert r["mismatched"] == 0
    assert r["max_abs_err"] == float(err.max())
    assert r["over_bound"] == int((err > bound).sum())
    # without a bound nothing is over it; the maximum is the same
    r2 = ar.check(ts, ref=torch.from_numpy(ref).cuda())
    assert r2["over_bound"] == 0 and r2["max_abs_err"] == r["max_abs_err"]


def test_nan_difference_is_reported():
    count = 5000
    xs = rand_inputs("float32", 2, count, seed=3)
    ts = to_gpu(xs, "float32")
    ts[0][1234] = float("nan")
    ts[1][1234] = float("nan")
    ref = np.zeros(count)
    r = ar.check(ts, ref=torch.from_numpy(ref).cuda(),
                 bound=torch.full((count,), 1e9, dtype=torch.float64, device="cuda"))
    assert np.isnan(r["max_abs_err"])
    assert r["over_bound"] == 1
    assert r["mismatched"] == int((host_view(ts)[0] != host_view(ts)[1]).sum())


def test_empty_and_rejected_arguments():
    ts = [torch.zeros(0, device="cuda") for _ in range(3)]
    r = ar.check(ts)
    assert r == {"mismatched": 0, "first_mismatch": 0, "over_bound": 0, "max_abs_err": 0.0}
    ctx = ar.Context(0, torch.cuda.current_stream().cuda_stream)
    bufs = [torch.zeros(100, device="cuda") for _ in range(2)]
    p = [b.data_ptr() for b in bufs]
    ref = torch.zeros(100, dtype=torch.float64, device="cuda")
    out = torch.zeros(4, dtype=torch.int64, device="cuda")
    # (a reference shorter than count inside a larger allocation is not seen:
    # the runtime reports torch's whole segment; the host-side tests cover it)
    cases = {
        "NULL result": lambda: ctx.check_ptrs(p, 100, "float32", 0, 0, 0),
        "misaligned result": lambda: ctx.check_ptrs(p, 100, "float32", 0, 0, out.data_ptr() + 4),
        "bound without ref": lambda: ctx.check_ptrs(p, 100, "float32", 0, ref.data_ptr(),
                                                    out.data_ptr()),
        "host result": lambda: ctx.check_ptrs(p, 100, "float32", 0, 0,
                                              np.zeros(4, np.int64).ctypes.data),
    }
    for what, fn in cases.items():
        with pytest.raises(ar.ArError) as e:
            fn()
        assert e.value.status == _lib.AR_ERR_INVALID_ARG, what
    ctx.close()
