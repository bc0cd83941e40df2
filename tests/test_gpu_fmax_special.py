"""fp32 MAX over special values, every fused shape against the oracle.

The one-pass kernels (every fold order) take fp32 MAX in registers with the
hardware's IEEE-754-2019 maximum and make a NaN canonical once, at the end.
The rule given to the pages' max reduction here (NaN if any operand is NaN,
canonical 0x7FC00000; -0 below +0) is applied hop by hop by the per-step
kernels and by the oracle.
These inputs mix NaNs of every sign and payload (quiet and signalling),
signed zeros, infinities, subnormals and normal values, across the 8-rank
compiled loop, the run-time rank count, the DEEP and TINY shapes, the PACED
shapes above 128 MiB, line-aligned ragged chunks and the element-wise path
of misaligned buffers; every position of every rank must equal
oracle.exact_max bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_rs_amd as ar
from tests.gpu_helpers import assert_bits_equal

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MIB = 1 << 20


def special_bits(rng, count, n):
    """Bit patterns: mostly normal values, with zeros, infinities, subnormals
    and (about one position in 4n) a NaN of random sign and payload."""
    normal = rng.standard_normal(count, dtype=np.float32).view(np.uint32)
    kind = rng.integers(0, 64 * n, size=count)
    out = normal.copy()
    sign = rng.integers(0, 2, size=count).astype(np.uint32) << 31
    mant = rng.integers(1, 1 << 23, size=count).astype(np.uint32)
    out = np.where(kind < 16, sign | np.uint32(0x7F800000) | mant, out)       # NaN, any payload
    out = np.where((kind >= 16) & (kind < 24), sign, out)                     # +-0
    out = np.where((kind >= 24) & (kind < 28), sign | np.uint32(0x7F800000), out)   # +-inf
    out = np.where((kind >= 28) & (kind < 40), sign | mant, out)              # subnormal
    return out.astype(np.uint32)


def check(n, count, algo, seed, misalign=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    xs = [special_bits(rng, count, n) for _ in range(n)]
    want = oracle.exact_max([x.view(np.float32) for x in xs], "float32").view(np.uint32)
    if misalign:
        # rank r's data starts r mod 4 elements into its allocation: buffers
        # that disagree mod 16 bytes take the element-wise path
        bases = [torch.empty(count + 4, dtype=torch.float32, device="cuda") for _ in range(n)]
        ts = [b[r % 4:r % 4 + count] for r, b in enumerate(bases)]
        for t, x in zip(ts, xs):
            t.copy_(torch.from_numpy(x.view(np.float32)))
    else:
        ts = [torch.from_numpy(x.view(np.float32)).cuda() for x in xs]
    ar.allreduce(ts, op="max", algo=algo)
    torch.cuda.synchronize()
    for r, t in enumerate(ts):
        assert_bits_equal(t.cpu().numpy().view(np.uint32), want, f"n={n} count={count} {algo} rank {r}")


# (ranks, count): the shape each selects
SHAPES = [
    (2, 1000),              # two ranks, one hop (run-time rank count)
    (8, 4096 + 3),          # 8-rank WIDE, line-aligned ragged chunks
    (8, 1 << 16),           # 8-rank WIDE, aligned
    (12, 50005),            # run-time N WIDE
    (32, 33333),            # DEEP
    (64, 256),              # TINY (4-element chunks)
    (64, 1024 + 7),         # TINY, ragged
    (8, 4 * MIB + 8192),    # 8-rank PACED (over 128 MiB)
    (16, 2 * MIB + 3),      # run-time N PACED, line-aligned
]


@pytest.mark.parametrize("n,count", SHAPES, ids=[f"n{n}-{c}" for n, c in SHAPES])
def test_fp32_max_special_values_ring_fused(n, count):
    check(n, count, "ring_fused", seed=n * 1009 + count)


@pytest.mark.parametrize("n,count", [(8, 4096 + 3), (3, 777), (16, 20000)])
def test_fp32_max_special_values_misaligned(n, count):
    check(n, count, "ring_fused", seed=n + count, misalign=True)


@pytest.mark.parametrize("algo", ["ring_step", "tree_fused", "halving_doubling_fused",
                                  "double_tree_fused"])
def test_fp32_max_special_values_other_orders(algo):
    check(8, 4096 + 3, algo, seed=len(algo))
