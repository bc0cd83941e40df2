"""The pages' worked examples and the hand-derived bit patterns, run through
the HIP path (every algorithm that applies)."""

import numpy as np
import pytest
import torch

import ring_allreduce_rs_amd as ar
from tests.gpu_helpers import assert_bits_equal, to_gpu, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

RING = ("ring_step", "ring_fused")
# the tree algorithms, per step and in one pass (power-of-two rank counts)
TREES = ("tree", "halving_doubling", "double_tree", "tree_fused", "halving_doubling_fused",
         "double_tree_fused")


def h(s):
    return int(s, 16)


@pytest.mark.parametrize("count", [1, 3])
@pytest.mark.parametrize("algo", RING)
def test_three_rank_example(golden, count, algo):
    g = golden("three_rank_sum.json")
    ts = [torch.full((count,), v, dtype=torch.int32, device="cuda")
          for v in g["inputs_per_rank_value"]]
    ar.allreduce(ts, op="sum", algo=algo)
    torch.cuda.synchronize()
    for t in ts:
        assert (t.cpu() == g["expected_value_every_rank"]).all()


@pytest.mark.parametrize("algo", RING + TREES)
def test_four_rank_example(golden, algo):
    g = golden("four_rank_ones_2x3.json")
    for op, key in (("sum", "expected_sum_every_element"), ("avg", "expected_avg_every_element")):
        ts = [torch.ones(2, 3, device="cuda") * v for v in g["inputs_per_rank_value"]]
        ar.allreduce(ts, op=op, algo=algo)
        torch.cuda.synchronize()
        for t in ts:
            assert (t.cpu() == g[key]).all()


@pytest.mark.parametrize("n", [1, 2, 3, 4, 8, 16, 64])
@pytest.mark.parametrize("algo", RING + TREES)
def test_rank_valued_closed_form(n, algo):
    if algo in TREES and n & (n - 1):
        pytest.skip("tree needs a power of two")
    for op, want in (("sum", n * (n - 1) / 2), ("avg", (n - 1) / 2)):
        ts = [torch.ones(4, device="cuda") * r for r in range(n)]
        ar.allreduce(ts, op=op, algo=algo)
        torch.cuda.synchronize()
        for t in ts:
            assert (t.cpu() == want).all()


@pytest.mark.parametrize("algo", RING)
def test_ring_fold_order_golden(golden, algo):
    g = golden("fold_order_n4_fp32.json")
    xs = [np.array(x, dtype=np.float32) for x in g["inputs"]]
    ts = to_gpu(xs, "float32")
    ar.allreduce(ts, op="sum", algo=algo)
    torch.cuda.synchronize()
    want = np.array(g["expected_every_rank"], dtype=np.float32)
    for r, t in enumerate(ts):
        assert_bits_equal(to_np(t), want, f"{algo} rank {r}")


@pytest.mark.parametrize("algo", ["tree", "tree_fused"])
def test_tree_order_golden(golden, algo):
    g = golden("tree_order_n4_fp32.json")
    xs = [np.array(x, dtype=np.float32) for x in g["inputs"]]
    ts = to_gpu(xs, "float32")
    ar.allreduce(ts, op="sum", algo=algo)
    torch.cuda.synchronize()
    want = np.array(g["expected_every_rank"], dtype=np.float32)
    for r, t in enumerate(ts):
        assert_bits_equal(to_np(t), want, f"{algo} rank {r}")


def _pair_cases(cases, key_a="a", key_b="b"):
    a = [h(c[key_a]) for c in cases]
    b = [h(c[key_b]) for c in cases]
    return a, b, [h(c["expect"]) for c in cases]


@pytest.mark.parametrize("algo", RING + TREES)
@pytest.mark.parametrize("width", [1, 37])
def test_bf16_bits_golden(golden, algo, width):
    """Two ranks: the one hop is exactly the golden case.  ``width`` repeats the
    cases so both the element-wise and the 16-byte paths see them."""
    g = golden("bf16_hop_bits.json")
    for op, cases in (("sum", g["cases_sum"]), ("max", g["cases_max"])):
        a, b, e = _pair_cases(cases)
        xa = np.array(a * width, np.uint16)
        xb = np.array(b * width, np.uint16)
        ts = to_gpu([xa, xb], "bfloat16")
        ar.allreduce(ts, op=op, algo=algo)
        torch.cuda.synchronize()
        for t in ts:
            assert_bits_equal(to_np(t), np.array(e * width, np.uint16), f"bf16 {op} {algo}")
    # AVG: rank values that sum exactly to the golden sum, then one division
    for c in g["cases_avg"]:
        n = c["nranks"]
        s = np.array([h(c["sum"])], np.uint16)
        zero = np.zeros(1, np.uint16)
        xs = [s] + [zero] * (n - 1)
        if algo in TREES and n & (n - 1):
            continue
        ts = to_gpu([np.repeat(x, width) for x in xs], "bfloat16")
        ar.allreduce(ts, op="avg", algo=algo)
        torch.cuda.synchronize()
        for t in ts:
            assert_bits_equal(to_np(t), np.full(width, h(c["expect"]), np.uint16), c["why"])


@pytest.mark.parametrize("algo", RING + TREES)
@pytest.mark.parametrize("width", [1, 37])
def test_fp32_bits_golden(golden, algo, width):
    g = golden("fp32_edge_bits.json")
    for op, cases in (("sum", g["cases_sum"]), ("max", g["cases_max"])):
        a, b, e = _pair_cases(cases)
        xa = np.array(a * width, np.uint32).view(np.float32)
        xb = np.array(b * width, np.uint32).view(np.float32)
        ts = to_gpu([xa, xb], "float32")
        ar.allreduce(ts, op=op, algo=algo)
        torch.cuda.synchronize()
        for t in ts:
            assert_bits_equal(to_np(t).view(np.uint32), np.array(e * width, np.uint32),
                              f"fp32 {op} {algo}")
    for c in g["cases_avg"]:
        n = c["nranks"]
        if algo in TREES and n & (n - 1):
            continue
        s = np.full(width, h(c["sum"]), np.uint32).view(np.float32)
        xs = [s] + [np.zeros(width, np.float32)] * (n - 1)
        ts = to_gpu(xs, "float32")
        ar.allreduce(ts, op="avg", algo=algo)
        torch.cuda.synchronize()
        for t in ts:
            assert_bits_equal(to_np(t).view(np.uint32), np.full(width, h(c["expect"]), np.uint32),
                              c["why"])


@pytest.mark.parametrize("algo", RING + TREES)
def test_int32_wraps(algo):
    xs = [np.array([2**31 - 1, -2**31] * 9, np.int32), np.array([1, -1] * 9, np.int32)]
    ts = to_gpu(xs, "int32")
    ar.allreduce(ts, op="sum", algo=algo)
    torch.cuda.synchronize()
    for t in ts:
        assert to_np(t).tolist() == [-2**31, 2**31 - 1] * 9


@pytest.mark.parametrize("algo", ["halving_doubling", "halving_doubling_fused"])
def test_hd_order_golden(golden, algo):
    g = golden("hd_order_n4_fp32.json")
    xs = [np.array(x, dtype=np.float32) for x in g["inputs"]]
    ts = to_gpu(xs, "float32")
    ar.allreduce(ts, op="sum", algo=algo)
    torch.cuda.synchronize()
    want = np.array(g["expected_every_rank"], dtype=np.float32)
    for r, t in enumerate(ts):
        assert_bits_equal(to_np(t), want, f"{algo} rank {r}")


@pytest.mark.parametrize("algo", ["double_tree", "double_tree_fused"])
def test_dtree_order_golden(golden, algo):
    g = golden("dtree_order_n4_fp32.json")
    xs = [np.array(x, dtype=np.float32) for x in g["inputs"]]
    ts = to_gpu(xs, "float32")
    ar.allreduce(ts, op="sum", algo=algo)
    torch.cuda.synchronize()
    want = np.array(g["expected_every_rank"], dtype=np.float32)
    for r, t in enumerate(ts):
        assert_bits_equal(to_np(t), want, f"{algo} rank {r}")
