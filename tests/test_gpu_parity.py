"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: bitwise equality for every dtype -- int32 and MAX are exact, and fp32 /
bf16 SUM follow the same ring order (or pairwise tree order) with the same
per-hop rounding as the oracle.  The fused ring must also stay within
N * 2^-24 * sum|x| of the binary64 sum (checked in test_gpu_configs.py).
Sizes here span several 2048-element tiles per chunk and ragged tails.
"""

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_rs_amd as ar
from tests.gpu_helpers import TORCH_DT, assert_bits_equal, to_gpu, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DT_OPS = [("int32", "sum"), ("int32", "max"), ("float32", "sum"), ("float32", "max"),
          ("float32", "avg"), ("bfloat16", "sum"), ("bfloat16", "max"), ("bfloat16", "avg")]


def rand_inputs(dtype, n, count, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    if dtype == "int32":
        return [rng.integers(-2**31, 2**31, size=count, dtype=np.int64).astype(np.int32)
                for _ in range(n)]
    f = [(rng.standard_normal(count) * rng.choice([1e-3, 1.0, 1e3])).astype(np.float32)
         for _ in range(n)]
    if dtype == "float32":
        return f
    import torch as _t
    return [_t.from_numpy(x).to(_t.bfloat16).view(_t.int16).numpy().view(np.uint16) for x in f]


SIZES = [(1, 5), (2, 1), (2, 4099), (3, 1), (3, 3), (3, 10007), (4, 6), (4, 24581),
         (5, 4), (5, 9), (7, 30011), (8, 1), (8, 65539), (16, 33), (16, 40003)]


@pytest.mark.parametrize("dtype,op", DT_OPS)
@pytest.mark.parametrize("n,count", SIZES)
def test_ring_allreduce_matches_oracle(dtype, op, n, count):
    xs = rand_inputs(dtype, n, count, seed=n * 7919 + count)
    want = oracle.simulate_ring_allreduce(xs, dtype, op).state
    for algo in ("ring_step", "ring_fused"):
        ts = to_gpu(xs, dtype)
        ar.allreduce(ts, op=op, algo=algo)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(ts[r]), want[r], f"{algo} {dtype} {op} n={n} count={count} rank {r}")


@pytest.mark.parametrize("dtype,op", DT_OPS)
@pytest.mark.parametrize("n,count", [(1, 7), (2, 4099), (4, 6), (4, 24581), (8, 65539),
                                     (16, 33), (16, 40003), (32, 2050)])
def test_tree_allreduce_matches_oracle(dtype, op, n, count):
    xs = rand_inputs(dtype, n, count, seed=n * 31 + count)
    want = oracle.simulate_tree_allreduce(xs, dtype, op).state
    ts = to_gpu(xs, dtype)
    ar.allreduce(ts, op=op, algo="tree")
    torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_np(ts[r]), want[r], f"tree {dtype} {op} n={n} rank {r}")


@pytest.mark.parametrize("dtype,op", [("float32", "avg"), ("bfloat16", "sum"), ("int32", "max")])
@pytest.mark.parametrize("n,count", [(3, 10007), (5, 9), (8, 65539), (4, 6)])
def test_every_ring_step_matches_oracle_snapshot(dtype, op, n, count):
    """After each of the 2(N-1) steps the whole state (written and untouched
    chunks alike) equals the oracle's state after the same step."""
    xs = rand_inputs(dtype, n, count, seed=count)
    snaps = oracle.simulate_ring_allreduce(xs, dtype, op, record=True).snapshots
    assert len(snaps) == 2 * (n - 1)
    ts = to_gpu(xs, dtype)
    for k in range(n - 1):
        ar.ring_rs_step(ts, op, k)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(ts[r]), snaps[k][r], f"RS step {k} rank {r}")
    for k in range(n - 1):
        ar.ring_ag_step(ts, k)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(ts[r]), snaps[n - 1 + k][r], f"AG step {k} rank {r}")


@pytest.mark.parametrize("dtype,op", [("float32", "avg"), ("bfloat16", "sum"), ("int32", "sum")])
@pytest.mark.parametrize("n,count", [(4, 24581), (8, 1000), (16, 40003)])
def test_every_tree_step_matches_oracle_snapshot(dtype, op, n, count):
    xs = rand_inputs(dtype, n, count, seed=count + 1)
    snaps = oracle.simulate_tree_allreduce(xs, dtype, op, record=True).snapshots
    ts = to_gpu(xs, dtype)
    for s in range(len(snaps)):
        ar.tree_step(ts, op, s)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(ts[r]), snaps[s][r], f"tree step {s} rank {r}")


@pytest.mark.parametrize("dtype,op", DT_OPS)
@pytest.mark.parametrize("n,count", [(1, 7), (2, 4099), (4, 6), (4, 24581), (8, 65539),
                                     (16, 33), (16, 40003), (32, 2050)])
def test_halving_doubling_allreduce_matches_oracle(dtype, op, n, count):
    xs = rand_inputs(dtype, n, count, seed=n * 17 + count)
    want = oracle.simulate_hd_allreduce(xs, dtype, op).state
    ts = to_gpu(xs, dtype)
    ar.allreduce(ts, op=op, algo="halving_doubling")
    torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_np(ts[r]), want[r], f"hd {dtype} {op} n={n} rank {r}")


@pytest.mark.parametrize("dtype,op", [("float32", "avg"), ("bfloat16", "sum"), ("int32", "max")])
@pytest.mark.parametrize("n,count", [(4, 24581), (8, 1000), (16, 40003), (8, 5)])
def test_every_hd_step_matches_oracle_snapshot(dtype, op, n, count):
    xs = rand_inputs(dtype, n, count, seed=count + 2)
    snaps = oracle.simulate_hd_allreduce(xs, dtype, op, record=True).snapshots
    levels = n.bit_length() - 1
    assert len(snaps) == 2 * levels
    ts = to_gpu(xs, dtype)
    for s in range(levels):
        ar.hd_rs_step(ts, op, s)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(ts[r]), snaps[s][r], f"hd RS step {s} rank {r}")
    for s in range(levels):
        ar.hd_ag_step(ts, s)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(ts[r]), snaps[levels + s][r], f"hd AG step {s} rank {r}")


@pytest.mark.parametrize("dtype,op", DT_OPS)
@pytest.mark.parametrize("algo", ["ring_step", "ring_fused", "halving_doubling"])
@pytest.mark.parametrize("n,count", [(3, 10007), (4, 6), (8, 65539), (16, 40003)])
def test_reduce_scatter_then_allgather(dtype, op, algo, n, count):
    if algo == "halving_doubling" and n & (n - 1):
        pytest.skip("halving-doubling needs a power of two")
    xs = rand_inputs(dtype, n, count, seed=count * 3 + n)
    direct = (oracle.hd_fold_at(np.stack(xs), dtype, op) if algo == "halving_doubling"
              else oracle.ordered_ring_fold(xs, dtype, op))
    ts = to_gpu(xs, dtype)
    ar.reduce_scatter(ts, op=op, algo=algo)
    torch.cuda.synchronize()
    lay = oracle.chunk_layout(count, n)
    for r in range(n):
        lo, ln = lay[r]
        assert ar.chunk_range(count, n, r) == (lo, ln)
        assert_bits_equal(to_np(ts[r])[lo:lo + ln], direct[lo:lo + ln], f"RS {algo} rank {r}")
    ar.allgather(ts, algo=algo)
    torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_np(ts[r]), direct, f"RS+AG {algo} rank {r}")


@pytest.mark.parametrize("dtype", ["int32", "float32", "bfloat16"])
@pytest.mark.parametrize("n,count", [(3, 10007), (8, 65539), (5, 9), (4, 3)])
def test_allgather_copies_owner_chunks(dtype, n, count):
    xs = rand_inputs(dtype, n, count, seed=n + count)
    want = oracle.simulate_ring_allgather(xs, dtype).state
    for algo in ("ring_step", "ring_fused", "halving_doubling"):
        if algo == "halving_doubling" and n & (n - 1):
            continue
        ts = to_gpu(xs, dtype)
        ar.allgather(ts, algo=algo)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(ts[r]), want[r], f"AG {algo} rank {r}")


@pytest.mark.parametrize("dtype,op", [("float32", "avg"), ("bfloat16", "sum"), ("int32", "sum")])
@pytest.mark.parametrize("shift", [0, 1, 2, 3, 5])
@pytest.mark.parametrize("same_alignment", [True, False])
def test_unaligned_buffers(dtype, op, shift, same_alignment):
    """Buffers that start off a 16-byte boundary: a common misalignment takes
    the vector path with element-wise heads and tails, mixed misalignments the
    element-wise path.  Both must equal the oracle bitwise."""
    n, count = 4, 12345
    xs = rand_inputs(dtype, n, count, seed=shift + 17)
    wants = {"ring": oracle.simulate_ring_allreduce(xs, dtype, op).state,
             "tree": oracle.simulate_tree_allreduce(xs, dtype, op).state,
             "halving_doubling": oracle.simulate_hd_allreduce(xs, dtype, op).state,
             "double_tree": oracle.simulate_double_tree_allreduce(xs, dtype, op).state}
    stride = ((count + 64 + 7) // 8) * 8          # a multiple of 16 bytes per row
    for algo in ("ring_step", "ring_fused", "tree", "halving_doubling", "double_tree",
                 "tree_fused", "halving_doubling_fused", "double_tree_fused"):
        want = wants["ring" if algo.startswith("ring") else algo.replace("_fused", "")]
        store = torch.zeros(n * stride, dtype=to_gpu(xs[:1], dtype)[0].dtype, device="cuda")
        views = []
        for r in range(n):
            off = r * stride + (shift if same_alignment else (shift + r) % 8)
            v = store[off:off + count]
            v.copy_(to_gpu([xs[r]], dtype)[0])
            views.append(v)
        guard = store.clone()
        ar.allreduce(views, op=op, algo=algo)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(views[r]), want[r], f"{algo} shift {shift} rank {r}")
        # nothing outside the rank views was touched
        mask = torch.ones_like(store, dtype=torch.bool)
        for r in range(n):
            off = r * stride + (shift if same_alignment else (shift + r) % 8)
            mask[off:off + count] = False
        assert torch.equal(store[mask], guard[mask])


def test_sides_are_not_shared_state():
    """Two contexts on different streams give the same bits."""
    xs = rand_inputs("float32", 4, 5000, seed=1)
    want = oracle.simulate_ring_allreduce(xs, "float32", "avg").state
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ts = to_gpu(xs, "float32")
        ar.allreduce(ts, op="avg", algo="ring_fused")
    s.synchronize()
    for r in range(4):
        assert_bits_equal(to_np(ts[r]), want[r], "side stream")


@pytest.mark.parametrize("dtype,op", [("float32", "avg"), ("bfloat16", "sum"), ("int32", "max")])
@pytest.mark.parametrize("n,count", [(3, 10007), (8, 65539), (16, 33)])
def test_auto_runs_the_model_choice(dtype, op, n, count):
    """AUTO gives exactly the bits of the algorithm the model picks."""
    xs = rand_inputs(dtype, n, count, seed=count + 5)
    pick = ar.auto_algo(n, count, dtype)
    sim = {"ring_fused": oracle.simulate_ring_allreduce, "ring_step": oracle.simulate_ring_allreduce,
           "tree": oracle.simulate_tree_allreduce,
           "halving_doubling": oracle.simulate_hd_allreduce,
           "double_tree": oracle.simulate_double_tree_allreduce,
           "tree_fused": oracle.simulate_tree_allreduce,
           "halving_doubling_fused": oracle.simulate_hd_allreduce,
           "double_tree_fused": oracle.simulate_double_tree_allreduce}[pick]
    want = sim(xs, dtype, op).state
    ts = to_gpu(xs, dtype)
    ar.allreduce(ts, op=op, algo="auto")
    torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_np(ts[r]), want[r], f"auto ({pick}) rank {r}")
    rs = to_gpu(xs, dtype)
    ar.reduce_scatter(rs, op=op, algo="auto")
    ar.allgather(rs, algo="auto")
    torch.cuda.synchronize()
    if pick not in ("tree", "double_tree", "tree_fused", "double_tree_fused"):
        for r in range(n):
            assert_bits_equal(to_np(rs[r]), want[r], f"auto RS+AG rank {r}")


@pytest.mark.parametrize("dtype,op", DT_OPS)
@pytest.mark.parametrize("n,count", [(1, 7), (2, 4099), (4, 6), (4, 24581), (8, 65539),
                                     (16, 33), (16, 40003), (32, 2050), (2, 1)])
def test_double_tree_allreduce_matches_oracle(dtype, op, n, count):
    xs = rand_inputs(dtype, n, count, seed=n * 19 + count)
    want = oracle.simulate_double_tree_allreduce(xs, dtype, op).state
    ts = to_gpu(xs, dtype)
    ar.allreduce(ts, op=op, algo="double_tree")
    torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_np(ts[r]), want[r], f"dtree {dtype} {op} n={n} rank {r}")


@pytest.mark.parametrize("dtype,op", [("float32", "avg"), ("bfloat16", "sum"), ("int32", "max")])
@pytest.mark.parametrize("n,count", [(2, 1001), (4, 24581), (8, 1000), (16, 40003), (8, 3)])
def test_every_double_tree_step_matches_oracle_snapshot(dtype, op, n, count):
    xs = rand_inputs(dtype, n, count, seed=count + 4)
    snaps = oracle.simulate_double_tree_allreduce(xs, dtype, op, record=True).snapshots
    assert len(snaps) == 2 * (n.bit_length() - 1)
    ts = to_gpu(xs, dtype)
    for s in range(len(snaps)):
        ar.dtree_step(ts, op, s)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(ts[r]), snaps[s][r], f"dtree step {s} rank {r}")


# 33..64 ranks with chunks of at most 4 KiB take the fused kernel's
# element-wise all-loads-in-flight shape; 4100-byte chunks take the 16-byte
# one.  Both sides of that boundary, ragged counts and counts below N.
MANY_RANKS = [(33, 1), (33, 500), (40, 2050), (48, 3001), (64, 1), (64, 63), (64, 4101),
              (64, 65536), (64, 65600)]


@pytest.mark.parametrize("dtype,op", DT_OPS)
@pytest.mark.parametrize("n,count", MANY_RANKS)
def test_fused_many_ranks_small_chunks(dtype, op, n, count):
    xs = rand_inputs(dtype, n, count, seed=n * 104729 + count)
    want = oracle.simulate_ring_allreduce(xs, dtype, op).state
    ts = to_gpu(xs, dtype)
    ar.allreduce(ts, op=op, algo="ring_fused")
    torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_np(ts[r]), want[r], f"fused {dtype} {op} n={n} count={count} rank {r}")
    ts = to_gpu(xs, dtype)
    ar.reduce_scatter(ts, op=op, algo="ring_fused")
    torch.cuda.synchronize()
    for r, (lo, ln) in enumerate(oracle.chunk_layout(count, n)):
        assert_bits_equal(to_np(ts[r])[lo:lo + ln], want[r][lo:lo + ln],
                          f"fused RS {dtype} {op} n={n} count={count} rank {r}")


# The one-pass forms of recursive doubling and halving-doubling: same bits as
# the per-step algorithms (the oracle's message-passing simulations), over
# every fused shape -- WIDE (8 ranks, 16-byte path), DEEP, TINY (33-64 ranks,
# small chunks) and the element-wise path (counts below N, bf16 heads).
POW2 = [(2, 1), (2, 4099), (4, 6), (4, 24581), (8, 1), (8, 1000), (8, 65539), (16, 33),
        (16, 40003), (32, 2050), (64, 63), (64, 4101), (64, 70_001)]
FUSED_TREES = [("tree_fused", oracle.simulate_tree_allreduce),
               ("halving_doubling_fused", oracle.simulate_hd_allreduce),
               ("double_tree_fused", oracle.simulate_double_tree_allreduce)]


@pytest.mark.parametrize("algo,sim", FUSED_TREES, ids=[a for a, _ in FUSED_TREES])
@pytest.mark.parametrize("dtype,op", DT_OPS)
@pytest.mark.parametrize("n,count", POW2)
def test_fused_tree_orders_match_oracle(algo, sim, dtype, op, n, count):
    xs = rand_inputs(dtype, n, count, seed=n * 7207 + count)
    want = sim(xs, dtype, op).state
    ts = to_gpu(xs, dtype)
    ar.allreduce(ts, op=op, algo=algo)
    torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_np(ts[r]), want[r], f"{algo} {dtype} {op} n={n} count={count} rank {r}")


@pytest.mark.parametrize("dtype,op", DT_OPS)
@pytest.mark.parametrize("n,count", POW2)
def test_fused_halving_doubling_reduce_scatter_then_allgather(dtype, op, n, count):
    xs = rand_inputs(dtype, n, count, seed=n * 131 + count)
    rs = oracle.simulate_hd_reduce_scatter(xs, dtype, op).state
    full = oracle.simulate_hd_allreduce(xs, dtype, op).state
    ts = to_gpu(xs, dtype)
    ar.reduce_scatter(ts, op=op, algo="halving_doubling_fused")
    torch.cuda.synchronize()
    for r, (lo, ln) in enumerate(oracle.chunk_layout(count, n)):
        assert_bits_equal(to_np(ts[r])[lo:lo + ln], rs[r][lo:lo + ln], f"RS rank {r}")
    ar.allgather(ts, algo="halving_doubling_fused")
    torch.cuda.synchronize()
    for r in range(n):
        assert_bits_equal(to_np(ts[r]), full[r], f"RS+AG rank {r}")


def test_fused_tree_orders_refuse_what_they_do_not_define():
    ts = to_gpu(rand_inputs("float32", 6, 100, seed=1), "float32")
    for algo in ("tree_fused", "halving_doubling_fused", "double_tree_fused"):
        with pytest.raises(ar.ArError):
            ar.allreduce(ts, op="sum", algo=algo)           # 6 ranks: not a power of two
    ts = to_gpu(rand_inputs("float32", 8, 100, seed=1), "float32")
    for algo in ("tree_fused", "double_tree_fused"):
        with pytest.raises(ar.ArError):
            ar.reduce_scatter(ts, op="sum", algo=algo)      # AllReduce only
        with pytest.raises(ar.ArError):
            ar.allgather(ts, algo=algo)


# Chunk bodies that start off a 128-byte line take the line-aligned kernels
# (tiles shifted back by 0-7 idle 16-byte units).  Rank 0's view walks
# through one line in 16-byte steps (every shift value); the counts make the
# chunk starts themselves drift across lines and span several tiles per chunk
# (WIDE tile: 4 KiB per rank; DEEP: 1 KiB).
LINE_CASES = [(3, 3 * 4099 + 1), (8, 8 * 2051 + 5), (16, 16 * 3001 + 7)]


@pytest.mark.parametrize("dtype,op", [("float32", "avg"), ("int32", "sum"), ("bfloat16", "sum"),
                                      ("float32", "max")])
@pytest.mark.parametrize("n,count", LINE_CASES)
@pytest.mark.parametrize("line_shift", [0, 16, 48, 112])
def test_line_aligned_tiles_match_oracle(dtype, op, n, count, line_shift):
    xs = rand_inputs(dtype, n, count, seed=n * 977 + line_shift)
    eb = 2 if dtype == "bfloat16" else 4
    shift = line_shift // eb                      # elements; a multiple of 16 bytes
    stride = ((count + 256) // 64 + 1) * 64       # rows of whole 128-byte lines (fp32)
    tdt = to_gpu(xs[:1], dtype)[0].dtype
    want_ring = oracle.simulate_ring_allreduce(xs, dtype, op).state
    rs_want = oracle.simulate_ring_reduce_scatter(xs, dtype, op).state
    algos = [("ring_fused", want_ring)]
    if n & (n - 1) == 0:
        algos += [("tree_fused", oracle.simulate_tree_allreduce(xs, dtype, op).state),
                  ("halving_doubling_fused", oracle.simulate_hd_allreduce(xs, dtype, op).state),
                  ("double_tree_fused",
                   oracle.simulate_double_tree_allreduce(xs, dtype, op).state)]
    for algo, want in algos + [("rs+ag", want_ring)]:
        store = torch.zeros(n * stride + 64, dtype=tdt, device="cuda")
        assert store.data_ptr() % 128 == 0
        views = []
        for r in range(n):
            v = store[r * stride + shift:r * stride + shift + count]
            v.copy_(to_gpu([xs[r]], dtype)[0])
            views.append(v)
        guard = store.clone()
        if algo == "rs+ag":
            ar.reduce_scatter(views, op=op, algo="ring_fused")
            torch.cuda.synchronize()
            for r, (lo, ln) in enumerate(oracle.chunk_layout(count, n)):
                assert_bits_equal(to_np(views[r])[lo:lo + ln], rs_want[r][lo:lo + ln],
                                  f"RS shift {line_shift} rank {r}")
            ar.allgather(views, algo="ring_fused")
        else:
            ar.allreduce(views, op=op, algo=algo)
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(views[r]), want[r], f"{algo} shift {line_shift} rank {r}")
        mask = torch.ones_like(store, dtype=torch.bool)
        for r in range(n):
            mask[r * stride + shift:r * stride + shift + count] = False
        assert torch.equal(store[mask], guard[mask]), f"{algo}: wrote outside the rank views"


# Seeded random layouts: rank counts 1-64, counts from 0 up to a few tiles per
# chunk, every dtype/op, a common shift of rank 0's row within a 128-byte line
# (16-byte path, with or without line-aligned tiles) or mixed per-rank shifts
# (element-wise path).  One-pass AllReduce, and ReduceScatter then AllGather,
# bitwise against the oracle, with nothing written outside the views.
def _random_layout_cases(k=40, seed=20261203):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(k):
        n = int(rng.choice([1, 2, 3, 5, 8, 12, 16, 31, 64]))
        dtype, op = DT_OPS[int(rng.integers(len(DT_OPS)))]
        count = int(rng.choice([0, 1, n - 1, n * 1000 + 3, int(rng.integers(1, 40000))]))
        mixed = bool(rng.integers(4) == 0)
        shift_bytes = int(rng.integers(0, 128))
        out.append((i, n, max(count, 0), dtype, op, mixed, shift_bytes))
    return out


@pytest.mark.parametrize("case", _random_layout_cases(), ids=lambda c: f"case{c[0]}")
def test_random_layouts_match_oracle(case):
    _, n, count, dtype, op, mixed, shift_bytes = case
    eb = 2 if dtype == "bfloat16" else 4
    xs = rand_inputs(dtype, n, count, seed=case[0] + 5000)
    want = oracle.simulate_ring_allreduce(xs, dtype, op).state
    rs_want = oracle.simulate_ring_reduce_scatter(xs, dtype, op).state
    stride = ((count + 512) // 64 + 1) * 64           # whole 128-byte lines per row
    base_shift = shift_bytes // eb
    shifts = [(base_shift + (r % 3 if mixed else 0)) for r in range(n)]
    tdt = TORCH_DT[dtype]
    for kind in ("allreduce", "rs+ag"):
        store = torch.zeros(n * stride + 64, dtype=tdt, device="cuda")
        views = []
        for r in range(n):
            v = store[r * stride + shifts[r]:r * stride + shifts[r] + count]
            if count:
                v.copy_(to_gpu([xs[r]], dtype)[0])
            views.append(v)
        guard = store.clone()
        if kind == "allreduce":
            ar.allreduce(views, op=op, algo="ring_fused")
        else:
            ar.reduce_scatter(views, op=op, algo="ring_fused")
            torch.cuda.synchronize()
            for r, (lo, ln) in enumerate(oracle.chunk_layout(count, n)):
                assert_bits_equal(to_np(views[r])[lo:lo + ln], rs_want[r][lo:lo + ln],
                                  f"RS {case} rank {r}")
            ar.allgather(views, algo="ring_fused")
        torch.cuda.synchronize()
        for r in range(n):
            assert_bits_equal(to_np(views[r]), want[r], f"{kind} {case} rank {r}")
        mask = torch.ones_like(store, dtype=torch.bool)
        for r in range(n):
            mask[r * stride + shifts[r]:r * stride + shifts[r] + count] = False
        assert torch.equal(store[mask], guard[mask]), f"{kind} {case}: wrote outside the views"
