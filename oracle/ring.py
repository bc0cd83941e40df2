"""Message-passing simulation of Ring AllReduce -- oracle (test infrastructure only).

The ring is the two-phase algorithm the pages describe: N ranks in a one-way
ring r -> r+1 (mod N), each vector split into N chunks; a ReduceScatter phase
of N-1 steps in which every rank sends one chunk to its successor, which
folds it into its own copy of that chunk; then an AllGather phase of N-1
steps in which every rank forwards a finished chunk to its successor, which
stores it unchanged.  Sources: "AllReduce" (compassingai.com), section 3
技术原理; "Allreduce：大模型分布式训练的核心通信算法与优化实践", section 2.2;
"AllReduce算法详解", sections 4.2.1-4.2.3; "AllReduce 集合通信"
(zzmblog.top), sections 两阶段流程 and 通信量推导; "集合通信基础AllReduce、Ring
算法与NCCL全解析", section 3.1.

Schedule (a reading: the pages name no formula).  Section 2.2 of the pwwt.cn
page says that after ReduceScatter rank 0 holds the reduced chunk 0, rank 1
chunk 1, and so on, and that in the AllGather rank 0 starts by sending chunk 0
while receiving chunk N-1.  Hence, with ``rotation`` = 0:

* ReduceScatter step k (k = 0..N-2): rank r sends chunk (r-k-1) mod N;
* AllGather step k (k = 0..N-2): rank r sends chunk (r-k) mod N;

so chunk c is folded in rank order c+1, c+2, ..., c-1, c and ends on rank c.
``rotation`` = 1 gives the other reading of the same section (rank r starts
by sending chunk r and ends owning chunk r+1); it exists only so tests can
show that the two readings give different fp32 bits.

Every step first builds all N messages from a snapshot of the senders' state,
then delivers them; the simulation asserts that no chunk a step reads is also
written in that step.  Per-rank bytes sent and received and the number of
steps are counted for the closed-form checks.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .elementops import avg_epilogue, hop, np_dtype_of
from .layout import chunk_layout


class BrokenRing(RuntimeError):
    """A message was lost: the ring cannot complete (no partial result)."""


@dataclass
class RingTrace:
    state: list            # per-rank vectors after the simulated phases
    sent: list             # bytes sent per rank
    recv: list             # bytes received per rank
    steps: int = 0         # communication steps taken
    snapshots: list = field(default_factory=list)  # state after every step


def _itemsize(dtype: str) -> int:
    return np.dtype(np_dtype_of(dtype)).itemsize


def _init(xs, dtype):
    n = len(xs)
    if n < 1:
        raise ValueError("need at least one rank")
    arrs = [np.array(x, dtype=np_dtype_of(dtype), copy=True).reshape(-1) for x in xs]
    count = arrs[0].size
    if any(a.size != count for a in arrs):
        raise ValueError("all ranks must hold the same number of elements")
    return arrs


def _run_reduce_scatter(tr, dtype, op, rotation, record, drop, step0):
    n = len(tr.state)
    count = tr.state[0].size
    layout = chunk_layout(count, n)
    isz = _itemsize(dtype)
    for k in range(n - 1):
        msgs = []
        for r in range(n):
            c = (r - k - 1 + rotation) % n
            lo, ln = layout[c]
            msgs.append((r, (r + 1) % n, c, tr.state[r][lo:lo + ln].copy()))
        reads = {(src, c) for src, _, c, _ in msgs}
        writes = {(dst, c) for _, dst, c, _ in msgs}
        assert not (reads & writes), "a ring step read and wrote the same chunk"
        for src, dst, c, payload in msgs:
            if drop is not None and drop == (src, step0 + k):
                raise BrokenRing(f"message from rank {src} lost at step {step0 + k}")
            lo, ln = layout[c]
            # the travelling partial sum is folded with the receiver's term
            tr.state[dst][lo:lo + ln] = hop(payload, tr.state[dst][lo:lo + ln], dtype, op)
            tr.sent[src] += ln * isz
            tr.recv[dst] += ln * isz
        tr.steps += 1
        if op == "avg" and k == n - 2:
            _apply_avg(tr, dtype, rotation)
        if record:
            tr.snapshots.append([s.copy() for s in tr.state])
    if op == "avg" and n == 1:
        _apply_avg(tr, dtype, rotation)


def _apply_avg(tr, dtype, rotation):
    """The owner of a finished chunk divides it by N (once, after the SUM)."""
    n = len(tr.state)
    layout = chunk_layout(tr.state[0].size, n)
    for r in range(n):
        lo, ln = layout[(r + rotation) % n]
        tr.state[r][lo:lo + ln] = avg_epilogue(tr.state[r][lo:lo + ln], n, dtype)


def _run_allgather(tr, dtype, rotation, record, drop, step0):
    n = len(tr.state)
    count = tr.state[0].size
    layout = chunk_layout(count, n)
    isz = _itemsize(dtype)
    for k in range(n - 1):
        msgs = []
        for r in range(n):
            c = (r - k + rotation) % n
            lo, ln = layout[c]
            msgs.append((r, (r + 1) % n, c, tr.state[r][lo:lo + ln].copy()))
        reads = {(src, c) for src, _, c, _ in msgs}
        writes = {(dst, c) for _, dst, c, _ in msgs}
        assert not (reads & writes), "a ring step read and wrote the same chunk"
        for src, dst, c, payload in msgs:
            if drop is not None and drop == (src, step0 + k):
                raise BrokenRing(f"message from rank {src} lost at step {step0 + k}")
            lo, ln = layout[c]
            tr.state[dst][lo:lo + ln] = payload       # stored unchanged
            tr.sent[src] += ln * isz
            tr.recv[dst] += ln * isz
        tr.steps += 1
        if record:
            tr.snapshots.append([s.copy() for s in tr.state])


def simulate_ring_reduce_scatter(xs, dtype, op, rotation=0, record=False, drop=None):
    """Ring ReduceScatter: rank r ends holding the reduced chunk r (rotation 0).

    The other chunks of each rank hold partial results afterwards.
    ``drop=(rank, step)`` loses that rank's message at that step.
    """
    st = _init(xs, dtype)
    n = len(st)
    tr = RingTrace(state=st, sent=[0] * n, recv=[0] * n)
    _run_reduce_scatter(tr, dtype, op, rotation, record, drop, 0)
    return tr


def simulate_ring_allgather(xs, dtype, rotation=0, record=False, drop=None):
    """Ring AllGather: rank r's chunk r is copied to every other rank."""
    st = _init(xs, dtype)
    n = len(st)
    tr = RingTrace(state=st, sent=[0] * n, recv=[0] * n)
    _run_allgather(tr, dtype, rotation, record, drop, 0)
    return tr


def simulate_ring_allreduce(xs, dtype, op, rotation=0, record=False, drop=None):
    """Ring AllReduce = Ring ReduceScatter followed by Ring AllGather.

    Returns a RingTrace whose ``state`` is every rank's result.  ``drop``
    counts steps over both phases (0 .. 2N-3).
    """
    st = _init(xs, dtype)
    n = len(st)
    tr = RingTrace(state=st, sent=[0] * n, recv=[0] * n)
    _run_reduce_scatter(tr, dtype, op, rotation, record, drop, 0)
    _run_allgather(tr, dtype, rotation, record, drop, n - 1)
    return tr
