"""Chunk layout of one rank's vector -- oracle (test infrastructure only).

The ring splits every rank's vector into N chunks, one per rank
("AllReduce", compassingai.com, section 3 技术原理, Reduce-Scatter bullet;
"Allreduce：大模型分布式训练的核心通信算法与优化实践", section 2.2).  The
pages only show the case where N divides the element count.  Reading used
here for the remainder: every chunk has L = ceil(count / N) elements except
the trailing ones, which are shorter or empty.  Chunk c is the half-open
element range [min(c*L, count), min((c+1)*L, count)).
"""

from __future__ import annotations


def chunk_layout(count: int, nranks: int) -> list[tuple[int, int]]:
    """Return [(offset, length)] for chunks 0..nranks-1 (element units)."""
    if nranks < 1:
        raise ValueError("nranks must be >= 1")
    if count < 0:
        raise ValueError("count must be >= 0")
    per = -(-count // nranks)  # ceil(count / nranks)
    out = []
    for c in range(nranks):
        lo = min(c * per, count)
        hi = min((c + 1) * per, count)
        out.append((lo, hi - lo))
    return out


def chunk_of(index: int, count: int, nranks: int) -> int:
    """Chunk that element ``index`` belongs to, found by scanning the layout."""
    for c, (lo, ln) in enumerate(chunk_layout(count, nranks)):
        if lo <= index < lo + ln:
            return c
    raise IndexError(index)
