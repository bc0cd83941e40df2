"""Seeded synthetic workloads for the AllReduce hot path.

This module only draws inputs.  It holds none of the reduction's arithmetic,
so both the CPU oracle's tests and the GPU path's tests and benchmark can use
it without sharing method code.

The workloads stand in for the gradient buckets the pages talk about: DDP's
default 25 MB fp32 bucket ("Allreduce：大模型分布式训练的核心通信算法与优化实践",
section 4.1; "AllReduce 集合通信", section DDP 梯度同步中的地位), half-precision
gradients (same pwwt.cn page, section 4.2) and a message-size sweep from
latency-bound to bandwidth-bound sizes ("AllReduce", compassingai.com,
section 4 关键参数).  The pages measure on no dataset; every input here is
synthetic.

Recipe: one ``numpy.random.Generator(PCG64(seed))`` stream, ranks drawn in
order 0..N-1.  Normals are drawn in fp32 and scaled by sigma (a standard
deviation).  bf16 inputs are the fp32 draw cast by torch (round to nearest
even).  For inputs too large to draw on the host, ``device_inputs`` draws the
same distributions on the GPU with a seeded ``torch.Generator`` (a different
stream from the host one, recorded as such).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

MiB = 1 << 20


@dataclass(frozen=True)
class Workload:
    name: str
    nranks: int
    count: int          # elements per rank
    dtype: str          # "int32" | "float32" | "bfloat16"
    dist: tuple         # ("uniform_int", lo, hi) | ("normal", sigma) | ("uniform", lo, hi) | ...
    op: str             # "sum" | "max" | "avg"

    @property
    def itemsize(self) -> int:
        return {"int32": 4, "float32": 4, "bfloat16": 2}[self.dtype]

    @property
    def bytes_per_rank(self) -> int:
        return self.count * self.itemsize


# N=4 x 1024 int32 in [-1000, 1000], SUM, chunks of 256
SMALL_INT = Workload("n4_1024_int32_sum", 4, 1024, "int32", ("uniform_int", -1000, 1000), "sum")
# the 3-rank example: values 1, 2, 3 -> 6 on every rank
THREE_RANK = Workload("n3_scalar_123_sum", 3, 1, "int32", ("rank_plus_one",), "sum")
# N=8 x 25 MiB DDP fp32 bucket ~ N(0, 1e-3), AVG  (the headline workload)
DDP_BUCKET = Workload("n8_25MiB_fp32_avg", 8, 6_553_600, "float32", ("normal", 1e-3), "avg")
# N=8 x 2 GiB bf16 ~ N(0, 1e-2), SUM with a bf16 rounding per ring hop
BF16_2GIB = Workload("n8_2GiB_bf16_sum", 8, 1 << 30, "bfloat16", ("normal", 1e-2), "sum")
# N=64 fp32 U[-1, 1], SUM, message sizes per rank 4 KiB .. 64 MiB
SWEEP_BYTES = (4 << 10, 64 << 10, 1 << 20, 16 << 20, 64 << 20)
SWEEP = tuple(
    Workload(f"n64_{b >> 10}KiB_fp32_sum", 64, b // 4, "float32", ("uniform", -1.0, 1.0), "sum")
    for b in SWEEP_BYTES
)
# N=16 x 268,435,459 (ragged last chunk): fp32 N(0,1) MAX, int32 U[-2^20, 2^20] SUM
RAGGED_MAX = Workload("n16_ragged_fp32_max", 16, 268_435_459, "float32", ("normal", 1.0), "max")
RAGGED_INT = Workload("n16_ragged_int32_sum", 16, 268_435_459, "int32",
                      ("uniform_int", -(1 << 20), 1 << 20), "sum")

ALL = (SMALL_INT, THREE_RANK, DDP_BUCKET, BF16_2GIB) + SWEEP + (RAGGED_MAX, RAGGED_INT)


def scaled(w: Workload, count: int, nranks: int | None = None) -> Workload:
    """Same distribution and op at another size (for oracle-sized parity cases)."""
    n = w.nranks if nranks is None else nranks
    return Workload(f"{w.name}@{n}x{count}", n, count, w.dtype, w.dist, w.op)


def _draw_f32(rng, dist, count):
    kind = dist[0]
    if kind == "normal":
        return (rng.standard_normal(count, dtype=np.float32) * np.float32(dist[1])).astype(np.float32)
    if kind == "uniform":
        lo, hi = dist[1], dist[2]
        return rng.uniform(lo, hi, count).astype(np.float32)
    if kind == "uniform_int":
        return rng.integers(dist[1], dist[2], size=count, endpoint=True).astype(np.float32)
    raise ValueError(dist)


def host_inputs(w: Workload, seed: int = 0) -> list:
    """Per-rank numpy arrays (bf16 as uint16 bit patterns)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for r in range(w.nranks):
        kind = w.dist[0]
        if kind == "rank_plus_one":
            v = np.full(w.count, r + 1)
        elif kind == "rank":
            v = np.full(w.count, r)
        elif w.dtype == "int32" and kind == "uniform_int":
            v = rng.integers(w.dist[1], w.dist[2], size=w.count, endpoint=True)
        else:
            v = _draw_f32(rng, w.dist, w.count)
        if w.dtype == "int32":
            out.append(np.asarray(v, dtype=np.int32))
        elif w.dtype == "float32":
            out.append(np.asarray(v, dtype=np.float32))
        else:
            import torch
            t = torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16)
            out.append(t.view(torch.int16).numpy().view(np.uint16).copy())
    return out


def device_inputs(w: Workload, seed: int = 0, device: str = "cuda") -> list:
    """Per-rank torch tensors drawn on the device with one seeded generator."""
    import torch
    tdt = {"int32": torch.int32, "float32": torch.float32, "bfloat16": torch.bfloat16}[w.dtype]
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for r in range(w.nranks):
        kind = w.dist[0]
        if kind == "rank_plus_one":
            t = torch.full((w.count,), r + 1, dtype=tdt, device=device)
        elif kind == "rank":
            t = torch.full((w.count,), r, dtype=tdt, device=device)
        elif kind == "uniform_int":
            t = torch.randint(w.dist[1], w.dist[2] + 1, (w.count,), generator=g,
                              device=device, dtype=torch.int32).to(tdt)
        elif kind == "normal":
            t = (torch.randn(w.count, generator=g, device=device, dtype=torch.float32)
                 * w.dist[1]).to(tdt)
        elif kind == "uniform":
            lo, hi = w.dist[1], w.dist[2]
            t = (torch.rand(w.count, generator=g, device=device, dtype=torch.float32)
                 * (hi - lo) + lo).to(tdt)
        else:
            raise ValueError(w.dist)
        out.append(t.contiguous())
    return out
