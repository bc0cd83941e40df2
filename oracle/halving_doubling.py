"""Message-passing simulation of recursive halving-doubling -- oracle (test infrastructure only).

"集合通信基础AllReduce、Ring算法与NCCL全解析", section 4.1, names the tree
AllReduce "Recursive Doubling / Halving" and describes pairwise merging in
log2 N steps.  The halving half is read here as the bandwidth-optimal
ReduceScatter by recursive halving followed by an AllGather by recursive
doubling (the textbook Rabenseifner scheme); the page gives only the name, so
every detail below is a reading:

* chunks as in ``oracle.layout`` (N chunks, ceil partition);
* ReduceScatter step s = 0..log2N-1, distance d = N / 2^(s+1): rank r and
  partner r XOR d each hold the same 2d-chunk segment; rank r keeps the half
  starting at chunk (r with its low log2(d) bits cleared) -- the lower half
  if bit d of r is clear, else the upper half -- and folds the partner's copy
  of that half into its own (own (+) received).  After log2 N steps rank r
  holds the finished chunk r; for AVG it divides it once by N;
* AllGather step t = 0..log2N-1, distance d = 2^t: rank r copies the d
  finished chunks its partner r XOR d holds.

For chunk c the result is the balanced fold that pairs ranks at distance N/2
first, then N/4, ..., 1: for N = 4, (x0 (+) x2) (+) (x1 (+) x3).  Every rank
sends (N-1)/N * K bytes in each phase, like the ring, in 2 log2 N steps.
"""

from __future__ import annotations

import numpy as np

from .elementops import avg_epilogue, hop, np_dtype_of
from .layout import chunk_layout
from .ring import BrokenRing, RingTrace


def _levels(n):
    if n < 1 or (n & (n - 1)):
        raise ValueError("halving-doubling needs a power-of-two rank count")
    return n.bit_length() - 1


def _span(layout, c0, m):
    """Element range of chunks c0 .. c0+m-1 (contiguous)."""
    lo = layout[c0][0]
    last = layout[c0 + m - 1]
    return lo, last[0] + last[1] - lo


def _init(xs, dtype):
    st = [np.array(x, dtype=np_dtype_of(dtype), copy=True).reshape(-1) for x in xs]
    return RingTrace(state=st, sent=[0] * len(st), recv=[0] * len(st))


def _rs(tr, dtype, op, record, drop, step0):
    n = len(tr.state)
    lay = chunk_layout(tr.state[0].size, n)
    isz = tr.state[0].dtype.itemsize
    levels = _levels(n)
    for s in range(levels):
        d = n >> (s + 1)
        msgs = []
        for r in range(n):
            p = r ^ d
            keep = r & ~(d - 1)                   # first chunk rank r keeps
            lo, ln = _span(lay, keep, d)
            # partner p sends its copy of the half that rank r keeps
            msgs.append((p, r, lo, ln, tr.state[p][lo:lo + ln].copy()))
        for src, dst, lo, ln, payload in msgs:
            if drop is not None and drop == (src, step0 + s):
                raise BrokenRing(f"message from rank {src} lost at step {step0 + s}")
            tr.state[dst][lo:lo + ln] = hop(tr.state[dst][lo:lo + ln], payload, dtype, op)
            tr.sent[src] += ln * isz
            tr.recv[dst] += ln * isz
        tr.steps += 1
        if op == "avg" and s == levels - 1:
            for r in range(n):
                lo, ln = lay[r]
                tr.state[r][lo:lo + ln] = avg_epilogue(tr.state[r][lo:lo + ln], n, dtype)
        if record:
            tr.snapshots.append([v.copy() for v in tr.state])
    if op == "avg" and levels == 0:
        tr.state = [avg_epilogue(v, n, dtype) for v in tr.state]


def _ag(tr, record, drop, step0):
    n = len(tr.state)
    lay = chunk_layout(tr.state[0].size, n)
    isz = tr.state[0].dtype.itemsize
    for t in range(_levels(n)):
        d = 1 << t
        msgs = []
        for r in range(n):
            p = r ^ d
            lo, ln = _span(lay, p & ~(d - 1), d)   # the partner's finished chunks
            msgs.append((p, r, lo, ln, tr.state[p][lo:lo + ln].copy()))
        for src, dst, lo, ln, payload in msgs:
            if drop is not None and drop == (src, step0 + t):
                raise BrokenRing(f"message from rank {src} lost at step {step0 + t}")
            tr.state[dst][lo:lo + ln] = payload
            tr.sent[src] += ln * isz
            tr.recv[dst] += ln * isz
        tr.steps += 1
        if record:
            tr.snapshots.append([v.copy() for v in tr.state])


def simulate_hd_reduce_scatter(xs, dtype, op, record=False, drop=None):
    """Recursive-halving ReduceScatter: rank r ends with the finished chunk r."""
    tr = _init(xs, dtype)
    _rs(tr, dtype, op, record, drop, 0)
    return tr


def simulate_hd_allgather(xs, dtype, record=False, drop=None):
    """Recursive-doubling AllGather of chunk r held by rank r."""
    tr = _init(xs, dtype)
    _ag(tr, record, drop, 0)
    return tr


def simulate_hd_allreduce(xs, dtype, op, record=False, drop=None):
    """Halving-doubling AllReduce = the two phases above (2 log2 N steps)."""
    tr = _init(xs, dtype)
    levels = _levels(len(xs))
    _rs(tr, dtype, op, record, drop, 0)
    _ag(tr, record, drop, levels)
    return tr


def hd_fold_at(values, dtype, op) -> np.ndarray:
    """Direct halving-doubling result for the N rows of ``values``, no messages.

    Ranks at distance N/2 are combined first, then the pair results at
    distance N/4, and so on: fold(ranks) = fold(even positions) (+) fold(odd
    positions).  For N = 4 this is (x0 (+) x2) (+) (x1 (+) x3).
    """
    v = np.asarray(values, dtype=np_dtype_of(dtype))
    n = v.shape[0]
    _levels(n)

    def fold(ranks):
        if len(ranks) == 1:
            return v[ranks[0]]
        # ranks at distance len/2 pair first: split by the lowest varying bit
        evens = ranks[0::2]
        odds = ranks[1::2]
        return hop(fold(evens), fold(odds), dtype, op)

    acc = fold(list(range(n)))
    if op == "avg":
        acc = avg_epilogue(acc, n, dtype)
    return acc
