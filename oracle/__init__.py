"""CPU oracle for the ring AllReduce hot path -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, obviously-correct reference that the HIP
kernels are checked against.  Only the test suite, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
The product library (``ring_allreduce_rs_amd``) never imports, calls or links
anything here, and nothing here imports the product library: the two share no
kernels, headers, helpers, tables or constants.

What it computes, and where each part comes from (page titles as printed on
the pages; section numbers are each page's own):

* ``layout``     -- splitting a rank's vector into N chunks ("AllReduce",
                    compassingai.com, section 3 技术原理; "Allreduce：大模型分布式
                    训练的核心通信算法与优化实践", section 2.2).
* ``elementops`` -- the per-hop operator for int32, fp32 and bf16 (SUM, MAX)
                    and the AVG epilogue (divide by world size after the SUM,
                    same page, section 3.1).
* ``ring``       -- a message-passing simulation of Ring ReduceScatter then
                    Ring AllGather, with per-rank byte counters ("AllReduce
                    集合通信", zzmblog.top, sections 两阶段流程 and 通信量推导).
* ``tree``       -- a message-passing simulation of recursive doubling
                    ("集合通信基础AllReduce、Ring算法与NCCL全解析", section 4.1).
* ``halving_doubling`` -- recursive-halving ReduceScatter then
                    recursive-doubling AllGather (the same page's name for
                    the tree, read as the bandwidth-optimal variant).
* ``double_tree`` -- two complementary in-order binary trees, each reducing
                    half of the vector up to its root and broadcasting it
                    down ("AllReduce", compassingai.com, section 3).
* ``direct``     -- direct references with no messages: exact integer sums,
                    fp64 sums, the ordered fold the ring performs per chunk,
                    the pairwise fold the tree performs.

Pinning: every function here is checked, by ``tests/test_oracle_pins.py``,
against facts fixed outside this package (the pages' worked examples,
closed-form traffic and step counts, exact integer arithmetic, hand-derived
fp32/bf16 bit patterns).  Nothing is marked "parity unpinned".
"""

from .layout import chunk_layout, chunk_of
from .elementops import (
    DTYPES, OPS, bf16_to_f32, f32_to_bf16_rne, hop, avg_epilogue,
    np_dtype_of, ieee_maximum_f32,
)
from .ring import (
    BrokenRing, RingTrace, simulate_ring_allreduce,
    simulate_ring_reduce_scatter, simulate_ring_allgather,
)
from .tree import simulate_tree_allreduce
from .halving_doubling import (
    simulate_hd_reduce_scatter, simulate_hd_allgather, simulate_hd_allreduce, hd_fold_at,
)
from .double_tree import (
    simulate_double_tree_allreduce, dtree_fold_at, double_tree_fold,
)
from .direct import (
    exact_int_sum, exact_max, fp64_sum, ordered_ring_fold,
    ring_fold_at, pairwise_tree_fold, tree_fold_at,
)

__all__ = [
    "chunk_layout", "chunk_of", "DTYPES", "OPS", "bf16_to_f32",
    "f32_to_bf16_rne", "hop", "avg_epilogue", "np_dtype_of",
    "ieee_maximum_f32", "BrokenRing", "RingTrace",
    "simulate_ring_allreduce", "simulate_ring_reduce_scatter",
    "simulate_ring_allgather", "simulate_tree_allreduce", "exact_int_sum",
    "exact_max", "fp64_sum", "ordered_ring_fold", "ring_fold_at",
    "pairwise_tree_fold", "tree_fold_at", "simulate_hd_reduce_scatter",
    "simulate_hd_allgather", "simulate_hd_allreduce", "hd_fold_at",
    "simulate_double_tree_allreduce", "dtree_fold_at", "double_tree_fold",
]
