"""Direct references, computed without any messages -- oracle (test infrastructure only).

* ``exact_int_sum`` / ``exact_max`` -- the plain AllReduce definition: every
  rank ends with the reduction of all ranks' data ("AllReduce",
  compassingai.com, section 3 技术原理; "AllReduce 集合通信", section 语义).  For
  int32 SUM (wrap-around) and for MAX this value does not depend on the
  order, so it is exact.
* ``fp64_sum`` -- the real sum, evaluated in binary64, for error bounds.
* ``ordered_ring_fold`` / ``ring_fold_at`` -- the value the ring produces for
  a floating-point SUM: chunk c folded left to right over ranks c+1, c+2, ...,
  c (the schedule reading described in ``oracle.ring``), each hop rounded.
* ``pairwise_tree_fold`` / ``tree_fold_at`` -- the value recursive doubling
  produces: the balanced pairwise fold over rank halves.
"""

from __future__ import annotations

import numpy as np

from .elementops import (
    avg_epilogue, bf16_to_f32, hop, ieee_maximum_f32, np_dtype_of,
)
from .layout import chunk_layout


def _stack(xs, dtype):
    return np.stack([np.asarray(x, dtype=np_dtype_of(dtype)).reshape(-1) for x in xs])


def exact_int_sum(xs) -> np.ndarray:
    """int32 SUM with two's-complement wrap-around: exact int64 sum, low 32 bits."""
    s = _stack(xs, "int32").astype(np.int64).sum(axis=0)
    return s.astype(np.uint64).astype(np.uint32).view(np.int32)


def exact_max(xs, dtype) -> np.ndarray:
    """Elementwise maximum over ranks (order-independent)."""
    a = _stack(xs, dtype)
    if dtype == "int32":
        return a.max(axis=0)
    f = a.astype(np.float32) if dtype == "float32" else bf16_to_f32(a)
    m = f[0]
    for row in f[1:]:
        m = ieee_maximum_f32(m, row)
    if dtype == "float32":
        return m
    return (m.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def fp64_sum(xs, dtype) -> np.ndarray:
    """Sum over ranks in binary64 (inputs widened exactly)."""
    a = _stack(xs, dtype)
    f = bf16_to_f32(a) if dtype == "bfloat16" else a
    return f.astype(np.float64).sum(axis=0)


def ring_fold_at(values, chunk_ids, nranks, dtype, op, rotation=0) -> np.ndarray:
    """Ring result at selected positions.

    ``values`` is (N, m): the N ranks' inputs at m positions; ``chunk_ids``
    the chunk each position lies in.  Position i in chunk c is folded over
    ranks c+1-rotation, c+2-rotation, ... (N terms, mod N), then divided by N
    for AVG.
    """
    v = np.asarray(values, dtype=np_dtype_of(dtype))
    n = nranks
    assert v.shape[0] == n
    c = np.asarray(chunk_ids, dtype=np.int64)
    cols = np.arange(v.shape[1])
    acc = v[(c + 1 - rotation) % n, cols]
    for j in range(2, n + 1):
        acc = hop(acc, v[(c + j - rotation) % n, cols], dtype, op)
    if op == "avg":
        acc = avg_epilogue(acc, n, dtype)
    return acc


def ordered_ring_fold(xs, dtype, op, rotation=0) -> np.ndarray:
    """Full-vector ring result, built chunk by chunk with no messages."""
    a = _stack(xs, dtype)
    n, count = a.shape
    out = np.empty(count, dtype=a.dtype)
    for c, (lo, ln) in enumerate(chunk_layout(count, n)):
        if ln:
            out[lo:lo + ln] = ring_fold_at(a[:, lo:lo + ln], np.full(ln, c), n,
                                           dtype, op, rotation)
    return out


def _pairwise(rows, dtype, op):
    if len(rows) == 1:
        return rows[0]
    half = len(rows) // 2
    return hop(_pairwise(rows[:half], dtype, op), _pairwise(rows[half:], dtype, op),
               dtype, op)


def tree_fold_at(values, dtype, op) -> np.ndarray:
    """Balanced pairwise fold of the N rows of ``values`` (power-of-two N)."""
    v = np.asarray(values, dtype=np_dtype_of(dtype))
    n = v.shape[0]
    if n & (n - 1):
        raise ValueError("pairwise tree fold needs a power-of-two rank count")
    acc = _pairwise([v[r] for r in range(n)], dtype, op)
    if op == "avg":
        acc = avg_epilogue(acc, n, dtype)
    return acc


def pairwise_tree_fold(xs, dtype, op) -> np.ndarray:
    """Full-vector tree result with no messages."""
    return tree_fold_at(_stack(xs, dtype), dtype, op)
