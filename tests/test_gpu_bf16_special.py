"""bf16 SUM and AVG over special values, every fused shape and order against
the oracle.

Every hop widens both operands, adds in fp32 and rounds to nearest even,
and a NaN result becomes the canonical 0x7FC0.  These inputs mix
NaNs of every sign and payload (signalling ones included), infinities of both
signs (whose sums make NaNs), the largest finite values (whose sums overflow
by rounding), signed zeros, subnormals and normal values, across the DEEP,
TINY and PACED shapes, line-aligned ragged chunks, the element-wise path of
misaligned buffers and the pairwise and double-tree orders; every position of
every rank must equal the oracle's fold bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_rs_amd as ar
from tests.gpu_helpers import assert_bits_equal

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

MIB = 1 << 20


def special_bf16(rng, count, n):
    """bf16 bit patterns: mostly rounded normal values, with NaNs (about one
    position in 4n), infinities, the largest finite values, signed zeros and
    subnormals."""
    normal = torch.from_numpy(rng.standard_normal(count, dtype=np.float32)).to(torch.bfloat16)
    out = normal.view(torch.int16).numpy().view(np.uint16).astype(np.uint32)
    kind = rng.integers(0, 64 * n, size=count)
    sign = rng.integers(0, 2, size=count).astype(np.uint32) << 15
    mant = rng.integers(1, 1 << 7, size=count).astype(np.uint32)
    out = np.where(kind < 16, sign | 0x7F80 | mant, out)                   # NaN, any payload
    out = np.where((kind >= 16) & (kind < 22), sign | 0x7F80, out)         # +-inf
    out = np.where((kind >= 22) & (kind < 30), sign | 0x7F7F, out)         # largest finite
    out = np.where((kind >= 30) & (kind < 36), sign, out)                  # +-0
    out = np.where((kind >= 36) & (kind < 46), sign | mant, out)           # subnormal
    return out.astype(np.uint16)


def run(xs, algo, misalign=False):
    n, count = len(xs), xs[0].size
    if misalign:
        # rank r's data starts r mod 8 elements into its allocation: buffers
        # that disagree mod 16 bytes take the element-wise path
        bases = [torch.empty(count + 8, dtype=torch.bfloat16, device="cuda") for _ in range(n)]
        ts = [b[r % 8:r % 8 + count] for r, b in enumerate(bases)]
        for t, x in zip(ts, xs):
            t.copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
    else:
        ts = [torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda() for x in xs]
    return ts


def check(n, count, op, algo, seed, misalign=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    xs = [special_bf16(rng, count, n) for _ in range(n)]
    with np.errstate(over="ignore", invalid="ignore"):    # inf + -inf, overflow: intended
        if algo == "ring_fused":
            want = oracle.ordered_ring_fold(xs, "bfloat16", op)
        elif algo == "tree_fused":
            want = oracle.pairwise_tree_fold(xs, "bfloat16", op)
        elif algo == "halving_doubling_fused":
            want = oracle.simulate_hd_allreduce(xs, "bfloat16", op).state[0]
        else:
            want = oracle.double_tree_fold(xs, "bfloat16", op)
    ts = run(xs, algo, misalign)
    ar.allreduce(ts, op=op, algo=algo)
    torch.cuda.synchronize()
    for r, t in enumerate(ts):
        got = t.view(torch.int16).cpu().numpy().view(np.uint16)
        assert_bits_equal(got, np.asarray(want).view(np.uint16), f"n={n} {op} {algo} rank {r}")


SHAPES = [
    (2, 1000),              # two ranks, one hop
    (8, 4096 + 3),          # DEEP, line-aligned ragged chunks
    (12, 50005),            # DEEP, run-time rank count
    (32, 33333),            # DEEP beyond 16 ranks
    (64, 512),              # TINY (8-element chunks)
    (8, 8 * MIB + 1024),    # PACED, 8-rank loop (over 128 MiB)
]


@pytest.mark.parametrize("op", ["sum", "avg"])
@pytest.mark.parametrize("n,count", SHAPES, ids=[f"n{n}-{c}" for n, c in SHAPES])
def test_bf16_special_values_ring_fused(n, count, op):
    check(n, count, op, "ring_fused", seed=n * 7919 + count + len(op))


@pytest.mark.parametrize("n,count", [(8, 4096 + 3), (3, 777)])
def test_bf16_special_values_misaligned(n, count):
    check(n, count, "sum", "ring_fused", seed=n + count, misalign=True)


@pytest.mark.parametrize("algo", ["tree_fused", "halving_doubling_fused", "double_tree_fused"])
@pytest.mark.parametrize("op", ["sum", "avg"])
def test_bf16_special_values_tree_orders(algo, op):
    check(8, 4096 + 3, op, algo, seed=len(algo) * 31 + len(op))
