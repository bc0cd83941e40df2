"""Message-passing simulation of the recursive-doubling tree -- oracle (test infrastructure only).

"集合通信基础AllReduce、Ring算法与NCCL全解析", section 4.1, describes the tree
AllReduce as pairwise merging: in the first step ranks 0 and 1 reduce
together, ranks 2 and 3 together, and so on; in the next step the pair
results are merged, and after log2 N steps every rank is done.  Reading used
here: in step s every rank r exchanges its whole current vector with partner
r XOR 2**s and both keep own (+) received.  Because every hop operator here
is commutative bit for bit, both partners hold the same bits after each step,
and the final result is the balanced pairwise fold
((x0 (+) x1) (+) (x2 (+) x3)) (+) ... .  N must be a power of two.  AVG
divides once, after the last step.
"""

from __future__ import annotations

import numpy as np

from .elementops import avg_epilogue, hop, np_dtype_of
from .ring import BrokenRing, RingTrace


def simulate_tree_allreduce(xs, dtype, op, record=False, drop=None):
    """Recursive doubling over power-of-two N; returns a RingTrace.

    ``drop=(rank, step)`` loses that rank's message at that step.
    """
    n = len(xs)
    if n < 1 or (n & (n - 1)) != 0:
        raise ValueError("the recursive-doubling tree needs a power-of-two rank count")
    st = [np.array(x, dtype=np_dtype_of(dtype), copy=True).reshape(-1) for x in xs]
    isz = st[0].dtype.itemsize
    nbytes = st[0].size * isz
    tr = RingTrace(state=st, sent=[0] * n, recv=[0] * n)
    levels = n.bit_length() - 1
    for s in range(levels):
        sent_msgs = [v.copy() for v in tr.state]          # every rank sends first
        for r in range(n):
            p = r ^ (1 << s)
            if drop is not None and drop == (p, s):
                raise BrokenRing(f"message from rank {p} lost at step {s}")
            tr.state[r] = hop(sent_msgs[r], sent_msgs[p], dtype, op)
            tr.sent[p] += nbytes
            tr.recv[r] += nbytes
        tr.steps += 1
        if op == "avg" and s == levels - 1:
            tr.state = [avg_epilogue(v, n, dtype) for v in tr.state]
        if record:
            tr.snapshots.append([v.copy() for v in tr.state])
    if op == "avg" and levels == 0:
        tr.state = [avg_epilogue(v, n, dtype) for v in tr.state]
    return tr
