"""ar_check_noalloc (the checker with a device-resident scratch array, for
callers that cannot allocate) against ar_check, through the C ABI: every
field equal, on two calls in a row, the second with a smaller input, so the
second call runs over records the first one left behind."""

import numpy as np
import pytest
import torch

import ring_allreduce_rs_amd as ar
from tests.gpu_helpers import to_gpu

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def inputs(n, count, seed, plant):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = (rng.standard_normal(count) * 1e-2).astype(np.float32)
    xs = [x.copy() for _ in range(n)]
    for rank, pos in plant:
        xs[rank][pos] = np.float32(xs[rank][pos] + 1.0)
    ref = x.astype(np.float64) + rng.standard_normal(count) * 1e-7
    bound = np.abs(rng.standard_normal(count)) * 1e-7
    return to_gpu(xs, "float32"), torch.from_numpy(ref).cuda(), torch.from_numpy(bound).cuda()


def run_both(ctx, ts, ref, bound):
    p = [t.data_ptr() for t in ts]
    a = torch.full((4,), -1, dtype=torch.int64, device="cuda")
    b = torch.full((4,), -2, dtype=torch.int64, device="cuda")
    ctx.check_ptrs(p, ts[0].numel(), "float32", ref.data_ptr(), bound.data_ptr(), a.data_ptr())
    ctx.check_noalloc_ptrs(p, ts[0].numel(), "float32", ref.data_ptr(), bound.data_ptr(),
                           b.data_ptr())
    torch.cuda.synchronize()
    return a.cpu(), b.cpu()


def test_noalloc_checker_matches_the_allocating_one():
    ctx = ar.Context(0, torch.cuda.current_stream().cuda_stream)
    # first call: every one of the 2048 partial records in use
    big = 2048 * 256 * 3 + 77
    ts, ref, bound = inputs(8, big, 1, [(3, 5), (7, big - 1), (1, 700_000)])
    a, b = run_both(ctx, ts, ref, bound)
    assert torch.equal(a, b), (a, b)
    assert a[0] == 3 and a[1] == 5 and 0 < a[2] < big
    # second call, smaller: 4 records, over what the first call left
    small = 1000
    ts, ref, bound = inputs(4, small, 2, [(2, 999)])
    a, b = run_both(ctx, ts, ref, bound)
    assert torch.equal(a, b), (a, b)
    assert a[0] == 1 and a[1] == 999
    # and no mismatch at all
    ts, ref, bound = inputs(2, 513, 3, [])
    a, b = run_both(ctx, ts, ref, bound)
    assert torch.equal(a, b) and a[0] == 0 and a[1] == 513
    ctx.close()
