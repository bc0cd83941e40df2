"""Message-passing simulation of the double binary tree -- oracle (test infrastructure only).

"AllReduce" (compassingai.com), section 3 技术原理, describes the tree
AllReduce as a reduction from the leaves up to the root followed by a
broadcast from the root back down, and the double binary tree as two
disjoint binary trees running at once, each carrying part of the data; the
pwwt.cn page ("Allreduce：大模型分布式训练的核心通信算法与优化实践"), section
2.3, and "AllReduce算法详解", section 4.3, describe the same reduce-then-
broadcast tree.  The pages give no tree shape, split or fold order; the
readings used here (N a power of two) are:

* Shape (the same for both trees), on positions 0..N-1: position 0 is the
  root and has one child, N/2.  A position v >= 1 whose lowest set bit is b
  has children v - b/2 and v + b/2 when b > 1 (an in-order binary tree: every
  subtree covers a contiguous run of positions).
* Tree A puts rank v at position v.  Tree B puts rank (v - 1) mod N at
  position v.  Leaves of A (odd ranks) are interior in B and vice versa, so
  the two trees are complementary.
* Tree A reduces and broadcasts elements [0, ceil(count/2)), tree B the rest.
* Reduce, level by level from the leaves: a node at position v replaces its
  partial by (left child (+) own) (+) right child; the last reduce step is the
  root: own (+) child N/2; AVG divides there once.  So each half ends as the
  in-order fold x_{p0} (+) ((((x_{p1} (+) x_{p2}) (+) x_{p3}) (+) ...)), with
  p_i the rank at position i.
* Broadcast, from the root down: position N/2 copies the root, then every
  node's children copy it, level by level.

2 log2 N steps in total.  Every non-root position sends its half-vector
partial once up and receives the result once down, per tree.
"""

from __future__ import annotations

import numpy as np

from .elementops import avg_epilogue, hop, np_dtype_of
from .ring import BrokenRing, RingTrace


def _levels(n):
    if n < 1 or (n & (n - 1)):
        raise ValueError("the double binary tree needs a power-of-two rank count")
    return n.bit_length() - 1


def rank_at(tree: int, v: int, n: int) -> int:
    """Rank placed at position v of tree 0 (A) or 1 (B)."""
    return v if tree == 0 else (v - 1) % n


def children(v: int, n: int) -> list:
    """Children positions of position v in the in-order tree shape."""
    if v == 0:
        return [n // 2] if n > 1 else []
    b = v & -v
    if b == 1:
        return []
    return [v - b // 2, v + b // 2]


def halves(count: int):
    """Element ranges carried by tree A and tree B."""
    h = -(-count // 2)
    return [(0, h), (h, count - h)]


def simulate_double_tree_allreduce(xs, dtype, op, record=False, drop=None):
    """Double binary tree AllReduce; returns a RingTrace (steps = 2 log2 N).

    ``drop=(rank, step)`` loses every message that rank sends at that step.
    """
    n = len(xs)
    levels = _levels(n)
    st = [np.array(x, dtype=np_dtype_of(dtype), copy=True).reshape(-1) for x in xs]
    isz = st[0].dtype.itemsize
    tr = RingTrace(state=st, sent=[0] * n, recv=[0] * n)
    spans = halves(st[0].size)
    step = 0

    def send(src, dst, nbytes):
        if drop is not None and drop == (src, step):
            raise BrokenRing(f"message from rank {src} lost at step {step}")
        tr.sent[src] += nbytes
        tr.recv[dst] += nbytes

    # reduce: interior levels 1 .. levels-1, then the root
    for lvl in range(1, levels + 1):
        for t, (lo, ln) in enumerate(spans):
            if lvl < levels:
                nodes = [v for v in range(1, n) if (v & -v) == (1 << lvl)]
            else:
                nodes = [0]
            for v in nodes:
                me = rank_at(t, v, n)
                kids = [rank_at(t, c, n) for c in children(v, n)]
                got = [tr.state[k][lo:lo + ln].copy() for k in kids]
                for k in kids:
                    send(k, me, ln * isz)
                own = tr.state[me][lo:lo + ln]
                if v == 0:
                    acc = hop(own, got[0], dtype, op)
                    if op == "avg":
                        acc = avg_epilogue(acc, n, dtype)
                else:
                    acc = hop(hop(got[0], own, dtype, op), got[1], dtype, op)
                tr.state[me][lo:lo + ln] = acc
        tr.steps += 1
        step += 1
        if record:
            tr.snapshots.append([s.copy() for s in tr.state])
    if n == 1 and op == "avg":
        tr.state = [avg_epilogue(s, 1, dtype) for s in tr.state]
    # broadcast: the root's child, then every interior level top-down
    for lvl in range(levels, 0, -1):
        for t, (lo, ln) in enumerate(spans):
            parents = [0] if lvl == levels else [v for v in range(1, n) if (v & -v) == (1 << lvl)]
            for v in parents:
                me = rank_at(t, v, n)
                for c in children(v, n):
                    k = rank_at(t, c, n)
                    send(me, k, ln * isz)
                    tr.state[k][lo:lo + ln] = tr.state[me][lo:lo + ln]
        tr.steps += 1
        step += 1
        if record:
            tr.snapshots.append([s.copy() for s in tr.state])
    return tr


def dtree_fold_at(values, tree: int, dtype, op) -> np.ndarray:
    """Direct in-order fold of tree ``tree`` over the N rows of ``values``."""
    v = np.asarray(values, dtype=np_dtype_of(dtype))
    n = v.shape[0]
    _levels(n)

    def sub(p):
        kids = children(p, n)
        own = v[rank_at(tree, p, n)]
        if not kids:
            return own
        return hop(hop(sub(kids[0]), own, dtype, op), sub(kids[1]), dtype, op)

    acc = v[rank_at(tree, 0, n)]
    if n > 1:
        acc = hop(acc, sub(n // 2), dtype, op)
    if op == "avg":
        acc = avg_epilogue(acc, n, dtype)
    return acc


def double_tree_fold(xs, dtype, op) -> np.ndarray:
    """Full-vector double-tree result with no messages."""
    a = np.stack([np.asarray(x, dtype=np_dtype_of(dtype)).reshape(-1) for x in xs])
    out = np.empty(a.shape[1], dtype=a.dtype)
    for t, (lo, ln) in enumerate(halves(a.shape[1])):
        if ln:
            out[lo:lo + ln] = dtree_fold_at(a[:, lo:lo + ln], t, dtype, op)
    return out
