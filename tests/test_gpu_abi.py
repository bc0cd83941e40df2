"""C-ABI behaviour on the GPU: every invalid argument is rejected with the
documented status before anything is launched; no-op cases; context life
cycle; stream binding.  Nothing here launches a kernel on bad input."""

import ctypes

import numpy as np
import pytest
import torch

import ring_allreduce_rs_amd as ar
from ring_allreduce_rs_amd import _lib

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

INVALID, UNSUPPORTED = _lib.AR_ERR_INVALID_ARG, _lib.AR_ERR_UNSUPPORTED


@pytest.fixture()
def ctx():
    c = ar.Context(0, torch.cuda.current_stream().cuda_stream)
    yield c
    c.close()


def status_of(fn):
    try:
        fn()
    except ar.ArError as e:
        return e.status
    return 0


def bufs(n, count=64, dtype=torch.float32):
    return [torch.arange(count, device="cuda").to(dtype) + r for r in range(n)]


def test_invalid_arguments_are_rejected_before_launch(ctx):
    ts = bufs(4)
    before = [t.clone() for t in ts]
    p = [t.data_ptr() for t in ts]
    cases = {
        "nranks 0": lambda: ctx.allreduce_ptrs([], 64, "float32", "sum", "ring_fused"),
        "nranks 65": lambda: ctx.allreduce_ptrs([p[0]] * 65, 1, "float32", "sum", "ring_fused"),
        "NULL entry": lambda: ctx.allreduce_ptrs([p[0], 0, p[2], p[3]], 64, "float32", "sum",
                                                 "ring_fused"),
        "misaligned": lambda: ctx.allreduce_ptrs([p[0] + 1, p[1], p[2], p[3]], 16, "float32",
                                                 "sum", "ring_fused"),
        "overlap same": lambda: ctx.allreduce_ptrs([p[0], p[0], p[2], p[3]], 64, "float32",
                                                   "sum", "ring_step"),
        "overlap partial": lambda: ctx.allreduce_ptrs([p[0], p[0] + 128, p[2], p[3]], 64,
                                                      "float32", "sum", "ring_fused"),
        "count overflow": lambda: ctx.allreduce_ptrs(p, 2**62, "float32", "sum", "ring_fused"),
        # 4 GiB per rank from 256-byte tensors: past the end of any allocation
        "past allocation": lambda: ctx.allreduce_ptrs(p, 2**30, "float32", "sum", "ring_fused"),
        "past allocation step": lambda: ctx.ring_ag_step_ptrs(p, 2**30, "float32", 0),
        "host pointer": lambda: ctx.allreduce_ptrs(
            [np.zeros(64, np.float32).ctypes.data] + p[1:], 64, "float32", "sum", "ring_fused"),
        "rs step range": lambda: ctx.ring_rs_step_ptrs(p, 64, "float32", "sum", 3),
        "rs step negative": lambda: ctx.ring_rs_step_ptrs(p, 64, "float32", "sum", -1),
        "ag step range": lambda: ctx.ring_ag_step_ptrs(p, 64, "float32", 3),
        "tree step range": lambda: ctx.tree_step_ptrs(p, 64, "float32", "sum", 2),
        "hd rs step range": lambda: ctx.hd_rs_step_ptrs(p, 64, "float32", "sum", 2),
        "hd ag step range": lambda: ctx.hd_ag_step_ptrs(p, 64, "float32", -1),
        "dtree step range": lambda: ctx.dtree_step_ptrs(p, 64, "float32", "sum", 4),
    }
    for name, fn in cases.items():
        assert status_of(fn) == INVALID, name
        assert ctx.last_error(), name
    # raw enum values out of range
    arr = (ctypes.c_void_p * 4)(*p)
    assert _lib.lib.ar_allreduce(ctx.handle, arr, 4, 64, 7, 0, 1) == INVALID
    assert _lib.lib.ar_allreduce(ctx.handle, arr, 4, 64, 1, 9, 1) == INVALID
    assert _lib.lib.ar_allreduce(ctx.handle, arr, 4, 64, 1, 0, 9) == INVALID
    assert _lib.lib.ar_allreduce(ctx.handle, None, 4, 64, 1, 0, 1) == INVALID
    torch.cuda.synchronize()
    for t, b in zip(ts, before):
        assert torch.equal(t, b)


def test_unsupported_combinations(ctx):
    ti = bufs(4, dtype=torch.int32)
    pi = [t.data_ptr() for t in ti]
    assert status_of(lambda: ctx.allreduce_ptrs(pi, 64, "int32", "avg", "ring_fused")) == UNSUPPORTED
    assert status_of(lambda: ctx.ring_rs_step_ptrs(pi, 64, "int32", "avg", 0)) == UNSUPPORTED
    t3 = bufs(3)
    p3 = [t.data_ptr() for t in t3]
    assert status_of(lambda: ctx.allreduce_ptrs(p3, 64, "float32", "sum", "tree")) == UNSUPPORTED
    assert status_of(lambda: ctx.tree_step_ptrs(p3, 64, "float32", "sum", 0)) == UNSUPPORTED
    t4 = bufs(4)
    p4 = [t.data_ptr() for t in t4]
    assert status_of(lambda: ctx.reduce_scatter_ptrs(p4, 64, "float32", "sum", "tree")) == UNSUPPORTED
    assert status_of(lambda: ctx.allgather_ptrs(p4, 64, "float32", "tree")) == UNSUPPORTED
    for call in (lambda: ctx.allreduce_ptrs(p3, 64, "float32", "sum", "halving_doubling"),
                 lambda: ctx.reduce_scatter_ptrs(p3, 64, "float32", "sum", "halving_doubling"),
                 lambda: ctx.allgather_ptrs(p3, 64, "float32", "halving_doubling"),
                 lambda: ctx.hd_rs_step_ptrs(p3, 64, "float32", "sum", 0),
                 lambda: ctx.hd_ag_step_ptrs(p3, 64, "float32", 0),
                 lambda: ctx.allreduce_ptrs(p3, 64, "float32", "sum", "double_tree"),
                 lambda: ctx.dtree_step_ptrs(p3, 64, "float32", "sum", 0),
                 lambda: ctx.reduce_scatter_ptrs(p4, 64, "float32", "sum", "double_tree"),
                 lambda: ctx.allgather_ptrs(p4, 64, "float32", "double_tree")):
        assert status_of(call) == UNSUPPORTED


def test_noops(ctx):
    # count 0: nothing is read, NULL entries are allowed
    ctx.allreduce_ptrs([0, 0, 0], 0, "float32", "avg", "ring_fused")
    ctx.allreduce_ptrs([0, 0, 0, 0], 0, "float32", "avg", "tree")
    # one rank: AVG over one rank is the identity
    (t,) = bufs(1, count=1001)
    before = t.clone()
    for algo in ("ring_step", "ring_fused", "tree", "halving_doubling", "double_tree", "auto"):
        ar.allreduce([t], op="avg", algo=algo)
    torch.cuda.synchronize()
    assert torch.equal(t, before)


def test_context_life_cycle():
    for _ in range(50):
        c = ar.Context(0)
        c.close()
    assert _lib.lib.ar_destroy(None) == 0
    h = ctypes.c_void_p()
    assert _lib.lib.ar_create(ctypes.byref(h), 99, None) == INVALID
    assert _lib.lib.ar_last_error(None)


def test_torch_wrapper_checks_inputs():
    ts = bufs(2)
    with pytest.raises(ValueError):
        ar.allreduce([ts[0], ts[1][:10]])
    with pytest.raises(ValueError):
        ar.allreduce([ts[0], ts[1].double()])
    with pytest.raises(ValueError):
        ar.allreduce([ts[0], ts[1].cpu()])
    m = torch.zeros(8, 8, device="cuda")
    with pytest.raises(ValueError):
        ar.allreduce([m.t(), m.t().clone()])
    with pytest.raises(ValueError):
        ar.allreduce([])


def test_stream_binding_orders_work():
    """Work enqueued on a side stream after a producer on the same stream sees
    the producer's writes."""
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ts = [torch.empty(100_003, device="cuda") for _ in range(8)]
        for r, t in enumerate(ts):
            t.fill_(float(r))
        ar.allreduce(ts, op="sum", algo="ring_fused")
        ar.allreduce(ts, op="avg", algo="ring_step")
    s.synchronize()
    for t in ts:
        assert (t.cpu() == 28.0).all()


@pytest.mark.parametrize("nsrc,ndst", [(1, 1), (8, 8), (3, 5), (16, 16), (0, 2), (4, 0), (1, 8)])
def test_calibration_stream_writes_the_xor(nsrc, ndst):
    """ar_stream: every destination receives the XOR of the sources (zeros
    with no source); the sources are left unchanged; sizes span several 4 KiB
    tiles and a partial last tile."""
    nbytes = 3 * 4096 + 48
    g = torch.Generator(device="cpu").manual_seed(nsrc * 100 + ndst)
    srcs = [torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32).cuda()
            for _ in range(nsrc)]
    keep = [s.clone() for s in srcs]
    dsts = [torch.full((nbytes // 4,), -1, dtype=torch.int32, device="cuda") for _ in range(ndst)]
    ar.stream_(srcs, dsts)
    torch.cuda.synchronize()
    want = np.zeros(nbytes // 4, np.int32)
    for s in keep:
        want ^= s.cpu().numpy()
    for d in dsts:
        assert np.array_equal(d.cpu().numpy(), want)
    for s, k in zip(srcs, keep):
        assert torch.equal(s, k)
    # the pre-bound form (timing loops) issues the same call
    for d in dsts:
        d.fill_(-1)
    call = ar.bind_stream(srcs, dsts)
    call()
    call()
    torch.cuda.synchronize()
    for d in dsts:
        assert np.array_equal(d.cpu().numpy(), want)


def test_calibration_stream_in_place():
    """dst[i] == src[i]: every buffer ends with the XOR of all the inputs."""
    n, nbytes = 8, 5 * 4096 + 32
    g = torch.Generator(device="cpu").manual_seed(7)
    bufs = [torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g, dtype=torch.int32).cuda()
            for _ in range(n)]
    want = np.zeros(nbytes // 4, np.int32)
    for b in bufs:
        want ^= b.cpu().numpy()
    ar.stream_(bufs, bufs)
    torch.cuda.synchronize()
    for b in bufs:
        assert np.array_equal(b.cpu().numpy(), want)


def test_calibration_stream_rejects_bad_arguments(ctx):
    a = torch.zeros(1024, dtype=torch.int32, device="cuda")
    b = torch.zeros(1024, dtype=torch.int32, device="cuda")
    pa, pb = a.data_ptr(), b.data_ptr()
    cases = {
        "nothing": lambda: ctx.stream_ptrs([], [], 4096),
        "65 sources": lambda: ctx.stream_ptrs([pa] * 65, [], 16),
        "65 distinct buffers": lambda: ctx.stream_ptrs([pa] * 33, [pb] * 32, 16),
        "bytes not a multiple of 16": lambda: ctx.stream_ptrs([pa], [pb], 4000 + 8),
        "misaligned": lambda: ctx.stream_ptrs([pa + 4], [pb], 1024),
        "overlap": lambda: ctx.stream_ptrs([pa], [pa + 16], 1024),
        "dst is another source": lambda: ctx.stream_ptrs([pa, pb], [pb], 1024),
        "past allocation": lambda: ctx.stream_ptrs([pa], [pb], 8192),
        "host pointer": lambda: ctx.stream_ptrs([np.zeros(256, np.int32).ctypes.data], [pb],
                                                1024),
    }
    for what, fn in cases.items():
        assert status_of(fn) == INVALID, what
    ctx.stream_ptrs([pa], [pb], 0)          # zero bytes: a no-op
