"""Helpers shared by the GPU tests: moving seeded inputs between numpy (the
oracle's view) and torch device tensors (the library's view), and choosing
sample positions for full-size cases."""

from __future__ import annotations

import numpy as np
import torch

import oracle

TORCH_DT = {"int32": torch.int32, "float32": torch.float32, "bfloat16": torch.bfloat16}


def to_gpu(xs, dtype, device="cuda"):
    out = []
    for x in xs:
        if dtype == "bfloat16":
            t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(x))
        out.append(t.to(device))
    return out


def to_np(t):
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a


def assert_bits_equal(got, want, what=""):
    g, w = bits(got), bits(want)
    if g.shape != w.shape:
        raise AssertionError(f"{what}: shape {g.shape} != {w.shape}")
    bad = np.nonzero(g != w)[0]
    if bad.size:
        i = int(bad[0])
        raise AssertionError(f"{what}: {bad.size} elements differ; first at {i}: "
                             f"got {g[i]!r} want {w[i]!r}")


def sample_positions(count, nranks, k=4096, seed=0):
    """Random positions plus every chunk boundary's neighbourhood and both ends."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = set(rng.integers(0, count, size=min(k, count)).tolist()) if count else set()
    for lo, ln in oracle.chunk_layout(count, nranks):
        for d in range(-9, 18):
            if 0 <= lo + d < count:
                pos.add(lo + d)
        for d in range(-9, 1):
            if 0 <= lo + ln + d < count:
                pos.add(lo + ln + d)
    for i in list(range(20)) + list(range(count - 20, count)):
        if 0 <= i < count:
            pos.add(i)
    return np.array(sorted(pos), dtype=np.int64)


def gather(ts, idx):
    """(N, m) numpy array of the ranks' values at positions idx."""
    ti = torch.from_numpy(idx).to(ts[0].device)
    return np.stack([to_np(t.index_select(0, ti)) for t in ts])


def chunk_ids(idx, count, nranks):
    per = -(-count // nranks)
    return (idx // per).astype(np.int64)
