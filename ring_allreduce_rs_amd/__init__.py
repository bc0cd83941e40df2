"""Single-GPU AllReduce of N logical ranks on MI355X -- Python binding.

N "ranks" are N equal-length torch tensors in one GPU's HBM.  Every call
marshals tensor pointers into the C ABI of libar.so (include/ar.h); the HIP
kernels do all the work, in place, on torch's current stream.  There is no
CPU fallback: if libar.so is missing, importing this package raises.

    import ring_allreduce_rs_amd as ar
    ar.allreduce(tensors, op="avg", algo="ring_fused")

The API mirrors ``torch.distributed.all_reduce`` semantics ("Allreduce：大模型
分布式训练的核心通信算法与优化实践", section 3.2: in place, every participant
ends with the same reduced tensor), with the participants given as a list.
"""

from __future__ import annotations

import ctypes

from . import _lib
from ._lib import (  # noqa: F401
    ALGOS, AR_GRAPHS_MAX_BYTES_DEFAULT, AR_MAX_RANKS, DTYPES, EXPORTS, LIB_PATH, OPS, ArError,
    Context, auto_algo, chunk_range, lib, predict_us,
)

__all__ = [
    "ArError", "Context", "allreduce", "reduce_scatter", "allgather", "ring_rs_step",
    "ring_ag_step", "tree_step", "hd_rs_step", "hd_ag_step", "dtree_step", "copy_", "stream_",
    "check", "chunk_range", "bind", "bind_stream", "stream_timeline",
    "context", "LIB_PATH", "predict_us", "auto_algo", "set_graphs", "set_residency_caps",
]

_ctx: dict = {}


def _torch():
    import torch
    return torch


def _dtype_name(t) -> str:
    torch = _torch()
    m = {torch.int32: "int32", torch.float32: "float32", torch.bfloat16: "bfloat16"}
    if t.dtype not in m:
        raise ValueError(f"unsupported dtype {t.dtype}; use int32, float32 or bfloat16")
    return m[t.dtype]


def _check(tensors):
    """Same checks the pages ask of all_reduce inputs: on the GPU, contiguous,
    same shape and dtype on every participant (pwwt.cn page, sections 3.3
    and 5.3)."""
    ts = list(tensors)
    if not 1 <= len(ts) <= AR_MAX_RANKS:
        raise ValueError(f"need 1..{AR_MAX_RANKS} rank tensors, got {len(ts)}")
    t0 = ts[0]
    dt = _dtype_name(t0)
    for i, t in enumerate(ts):
        if not t.is_cuda:
            raise ValueError(f"tensor {i} is not on a GPU")
        if t.device != t0.device:
            raise ValueError(f"tensor {i} is on {t.device}, tensor 0 on {t0.device}")
        if t.dtype != t0.dtype:
            raise ValueError(f"tensor {i} has dtype {t.dtype}, tensor 0 {t0.dtype}")
        if t.numel() != t0.numel():
            raise ValueError(f"tensor {i} has {t.numel()} elements, tensor 0 {t0.numel()}")
        if not t.is_contiguous():
            raise ValueError(f"tensor {i} is not contiguous")
    return ts, dt, t0.numel(), t0.device.index or 0


def context(device: int = 0) -> Context:
    """The per-device context, rebound to torch's current stream."""
    torch = _torch()
    c = _ctx.get(device)
    if c is None:
        c = Context(device, torch.cuda.current_stream(device).cuda_stream)
        _ctx[device] = c
    c.set_stream(torch.cuda.current_stream(device).cuda_stream)
    return c


def set_graphs(enable: bool = True, device: int = 0,
               max_bytes_per_rank: int = AR_GRAPHS_MAX_BYTES_DEFAULT) -> None:
    """Turn graph replay of the multi-launch algorithms on (for collectives of
    at most ``max_bytes_per_rank`` bytes per rank) or off, for the device's
    context (see ar_set_graphs)."""
    context(device).set_graphs(max_bytes_per_rank if enable else 0)


def set_residency_caps(enable: bool = True, device: int = 0) -> None:
    """Residency caps of the large one-pass calls on or off for the device's
    context (see ar_set_residency_caps): off for callers that overlap the
    collective with kernels needing LDS."""
    context(device).set_residency_caps(enable)


def allreduce(tensors, op: str = "sum", algo: str = "ring_fused"):
    """In-place AllReduce over the rank tensors; returns them."""
    ts, dt, count, dev = _check(tensors)
    context(dev).allreduce_ptrs([t.data_ptr() for t in ts], count, dt, op, algo)
    return ts


def reduce_scatter(tensors, op: str = "sum", algo: str = "ring_fused"):
    """In-place ReduceScatter: tensor r ends with the finished chunk r at its
    own offset (``chunk_range``); its other chunks are unspecified."""
    ts, dt, count, dev = _check(tensors)
    context(dev).reduce_scatter_ptrs([t.data_ptr() for t in ts], count, dt, op, algo)
    return ts


def allgather(tensors, algo: str = "ring_fused"):
    """In-place AllGather: chunk r of tensor r is copied to every tensor."""
    ts, dt, count, dev = _check(tensors)
    context(dev).allgather_ptrs([t.data_ptr() for t in ts], count, dt, algo)
    return ts


def ring_rs_step(tensors, op: str, step: int):
    ts, dt, count, dev = _check(tensors)
    context(dev).ring_rs_step_ptrs([t.data_ptr() for t in ts], count, dt, op, step)
    return ts


def ring_ag_step(tensors, step: int):
    ts, dt, count, dev = _check(tensors)
    context(dev).ring_ag_step_ptrs([t.data_ptr() for t in ts], count, dt, step)
    return ts


def tree_step(tensors, op: str, step: int):
    ts, dt, count, dev = _check(tensors)
    context(dev).tree_step_ptrs([t.data_ptr() for t in ts], count, dt, op, step)
    return ts


def hd_rs_step(tensors, op: str, step: int):
    ts, dt, count, dev = _check(tensors)
    context(dev).hd_rs_step_ptrs([t.data_ptr() for t in ts], count, dt, op, step)
    return ts


def hd_ag_step(tensors, step: int):
    ts, dt, count, dev = _check(tensors)
    context(dev).hd_ag_step_ptrs([t.data_ptr() for t in ts], count, dt, step)
    return ts


def dtree_step(tensors, op: str, step: int):
    ts, dt, count, dev = _check(tensors)
    context(dev).dtree_step_ptrs([t.data_ptr() for t in ts], count, dt, op, step)
    return ts


def copy_(dst, src):
    """16-byte vector copy of src into dst (same byte size), on the current stream."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("copy_ needs equal byte sizes")
    context(src.device.index or 0).copy_ptrs(dst.data_ptr(), src.data_ptr(), nbytes)
    return dst


def check(tensors, ref=None, bound=None) -> dict:
    """On-device check of an AllReduce result (ar_check): positions where some
    rank's bits differ from rank 0's, the first of them, and -- given a
    float64 reference (and per-position bounds) on the same device -- the
    largest |rank 0 - ref| and the positions over their bound.  Waits for the
    result on the current stream."""
    torch = _torch()
    ts, dt, count, dev = _check(tensors)
    for name, t in (("ref", ref), ("bound", bound)):
        if t is not None and (t.dtype != torch.float64 or t.numel() != count
                              or t.device != ts[0].device or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous float64 tensor of {count} elements "
                             "on the buffers' device")
    out = torch.zeros(4, dtype=torch.int64, device=ts[0].device)
    context(dev).check_ptrs([t.data_ptr() for t in ts], count, dt,
                            ref.data_ptr() if ref is not None else 0,
                            bound.data_ptr() if bound is not None else 0, out.data_ptr())
    torch.cuda.current_stream(ts[0].device).synchronize()
    v = out.cpu()
    return {"mismatched": int(v[0]), "first_mismatch": int(v[1]), "over_bound": int(v[2]),
            "max_abs_err": float(v[3:4].view(torch.float64)[0])}


def stream_(srcs, dsts):
    """Calibration stream (ar_stream): the XOR of the source tensors written to
    every destination tensor, all of one byte size, on the current stream."""
    bufs = list(srcs) + list(dsts)      # dsts[i] may be srcs[i] itself (in place)
    if not bufs:
        raise ValueError("stream_ needs at least one buffer")
    nbytes = bufs[0].numel() * bufs[0].element_size()
    for t in bufs:
        if t.numel() * t.element_size() != nbytes or not t.is_contiguous():
            raise ValueError("stream_ needs contiguous buffers of one byte size")
    context(bufs[0].device.index or 0).stream_ptrs([t.data_ptr() for t in srcs],
                                                  [t.data_ptr() for t in dsts], nbytes)
    return list(dsts)


class _Bound:
    """A pre-marshalled call: the pointer array and enums are converted to
    ctypes objects once and passed to the entry point as they are."""

    def __init__(self, fn, args, ctx, *keep):
        self._fn = fn
        self._args = args
        self._ctx = ctx
        self._keep = keep   # the pointer arrays the arguments point into

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise ArError(st, self._fn.__name__, self._ctx.last_error())


def bind(tensors, op: str = "sum", algo: str = "ring_fused", kind: str = "allreduce"):
    """Return a zero-argument callable that re-issues the same collective on
    the context's current stream (for timing loops)."""
    ts, dt, count, dev = _check(tensors)
    ctx = context(dev)
    arr = (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])
    c_int, h = ctypes.c_int, ctypes.c_void_p(ctx.handle.value)
    head = (h, arr, c_int(len(ts)), ctypes.c_size_t(count), c_int(DTYPES[dt]))
    if kind == "allreduce":
        return _Bound(_lib.raw_fn("ar_allreduce"), head + (c_int(OPS[op]), c_int(ALGOS[algo])),
                      ctx, arr)
    if kind == "reduce_scatter":
        return _Bound(_lib.raw_fn("ar_reduce_scatter"),
                      head + (c_int(OPS[op]), c_int(ALGOS[algo])), ctx, arr)
    if kind == "allgather":
        return _Bound(_lib.raw_fn("ar_allgather"), head + (c_int(ALGOS[algo]),), ctx, arr)
    raise ValueError(kind)


def stream_timeline(bufs, lds_bytes, ts):
    """Timeline of the in-place calibration stream over `bufs` (ar_stream_timeline):
    each buffer is overwritten with the XOR of all of them, block b writes its
    start and end on the device's wall clock to ts[2b], ts[2b + 1] (ts: an int64
    tensor on the same device).  Returns (blocks, clock rate in kHz)."""
    bufs = list(bufs)
    if not bufs:
        raise ValueError("stream_timeline needs at least one buffer")
    nbytes = bufs[0].numel() * bufs[0].element_size()
    for t in bufs:
        if t.numel() * t.element_size() != nbytes or not t.is_contiguous():
            raise ValueError("stream_timeline needs contiguous buffers of one byte size")
    if not ts.is_contiguous() or ts.element_size() != 8:
        raise ValueError("ts must be a contiguous 8-byte tensor")
    return context(bufs[0].device.index or 0).stream_timeline_ptrs(
        [t.data_ptr() for t in bufs], nbytes, lds_bytes, ts.data_ptr(), ts.numel())


def bind_stream(srcs, dsts):
    """Return a zero-argument callable that re-issues the same calibration
    stream (ar_stream) on the context's current stream (for timing loops)."""
    bufs = list(srcs) + list(dsts)
    if not bufs:
        raise ValueError("bind_stream needs at least one buffer")
    nbytes = bufs[0].numel() * bufs[0].element_size()
    for t in bufs:
        if t.numel() * t.element_size() != nbytes or not t.is_contiguous():
            raise ValueError("bind_stream needs contiguous buffers of one byte size")
    ctx = context(bufs[0].device.index or 0)
    sa = (ctypes.c_void_p * max(1, len(srcs)))(*[t.data_ptr() for t in srcs])
    da = (ctypes.c_void_p * max(1, len(dsts)))(*[t.data_ptr() for t in dsts])
    c_int = ctypes.c_int
    return _Bound(_lib.raw_fn("ar_stream"),
                  (ctypes.c_void_p(ctx.handle.value), sa, c_int(len(srcs)), da, c_int(len(dsts)),
                   ctypes.c_size_t(nbytes)), ctx, sa, da)
