"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times.

Where the oracle finishes in seconds it runs on the whole input (4-rank
int32, the 25 MiB DDP bucket, the two small sweep points).  The two
multi-GiB workloads (8 x 2^30 bf16, 16 x 268,435,459) are checked against the
oracle over the whole array too, streamed through the host in slices (each
slice's inputs and results downloaded, the oracle's per-position fold run on
it, several slices at a time on the host's cores), besides sampled positions
(random positions plus the neighbourhood of every chunk boundary, where
heads, tails and straddling 16-byte units live).  Whole-array properties are
also checked on the GPU: all ranks identical, fused == per-step bitwise.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import ring_allreduce_rs_amd as ar
import workloads as W
from tests.gpu_helpers import (assert_bits_equal, bits, chunk_ids, gather, sample_positions,
                               to_gpu, to_np)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def run(ts, op, algo):
    ar.allreduce(ts, op=op, algo=algo)
    torch.cuda.synchronize()


def clone_all(ts):
    return [t.clone() for t in ts]


def ranks_identical(ts):
    return all(torch.equal(t, ts[0]) for t in ts[1:])


SLICE = 1 << 23          # elements per slice of the streamed whole-array checks


def whole_array_vs_oracle(inputs, result, want_at, what, workers=12):
    """Compare ``result`` (one rank's output, on the GPU) with the oracle over
    every position.  ``inputs`` are the untouched input tensors; for each
    slice [lo, hi) the (N, hi - lo) input block and the result slice are
    downloaded and ``want_at(values, lo)`` (an oracle function of the block)
    must equal the result bit for bit.  Slices run ``workers`` at a time
    (numpy releases the interpreter lock in its kernels)."""
    from concurrent.futures import ThreadPoolExecutor
    count = result.numel()

    def one(lo):
        hi = min(lo + SLICE, count)
        vals = np.stack([to_np(t[lo:hi]) for t in inputs])
        got = to_np(result[lo:hi])
        want = want_at(vals, lo)
        g = np.ascontiguousarray(got).view(np.uint8)
        w_ = np.ascontiguousarray(want).view(np.uint8)
        if not np.array_equal(g, w_):
            bad = np.nonzero(bits(got) != bits(want))[0]
            return f"{what}: slice at {lo}: {bad.size} elements differ, first at {lo + int(bad[0])}"
        return None

    starts = range(0, count, SLICE)
    with ThreadPoolExecutor(max_workers=workers) as pool:
        res = list(pool.map(one, starts))
    assert len(res) == -(-count // SLICE)          # every slice was compared
    errs = [e for e in res if e]
    assert not errs, errs[:3]


def test_small_int32_config():
    w = W.SMALL_INT
    xs = W.host_inputs(w, seed=0)
    assert [ln for _, ln in oracle.chunk_layout(w.count, w.nranks)] == [256] * 4
    want = oracle.simulate_ring_allreduce(xs, "int32", "sum").state
    exact = oracle.exact_int_sum(xs)
    for algo in ("ring_step", "ring_fused", "tree"):
        ts = to_gpu(xs, "int32")
        run(ts, "sum", algo)
        for r in range(w.nranks):
            assert_bits_equal(to_np(ts[r]), want[r], f"{algo} rank {r}")
            assert_bits_equal(to_np(ts[r]), exact, f"{algo} exact rank {r}")


def test_three_rank_scalar_config():
    w = W.THREE_RANK
    xs = W.host_inputs(w, seed=0)
    for algo in ("ring_step", "ring_fused"):
        ts = to_gpu(xs, "int32")
        run(ts, "sum", algo)
        for t in ts:
            assert to_np(t).tolist() == [6]


def test_ddp_bucket_config_full_oracle():
    """8 ranks x 6,553,600 fp32 ~ N(0, 1e-3), AVG: whole-vector bitwise parity."""
    w = W.DDP_BUCKET
    xs = W.host_inputs(w, seed=0)
    say("ddp bucket: oracle")
    want = oracle.simulate_ring_allreduce(xs, "float32", "avg").state[0]
    f64 = oracle.fp64_sum(xs, "float32") / w.nranks
    bound = w.nranks * 2.0 ** -24 * np.abs(np.stack(xs).astype(np.float64)).sum(axis=0) / w.nranks
    for algo in ("ring_fused", "ring_step"):
        say(f"ddp bucket: {algo}")
        ts = to_gpu(xs, "float32")
        run(ts, "avg", algo)
        assert ranks_identical(ts)
        got = to_np(ts[0])
        assert_bits_equal(got, want, algo)
        assert (np.abs(got.astype(np.float64) - f64) <= bound + 2.0 ** -149).all()
        # the same two facts from the on-device checker
        r = ar.check(ts, ref=torch.from_numpy(f64).cuda(),
                     bound=torch.from_numpy(bound + 2.0 ** -149).cuda())
        assert r["mismatched"] == 0 and r["over_bound"] == 0, r
        assert r["max_abs_err"] == float(np.abs(got.astype(np.float64) - f64).max())
    tw = oracle.simulate_tree_allreduce(xs, "float32", "avg").state[0]
    hw = oracle.simulate_hd_allreduce(xs, "float32", "avg").state[0]
    for algo, want in (("tree", tw), ("tree_fused", tw), ("halving_doubling", hw),
                       ("halving_doubling_fused", hw)):
        ts = to_gpu(xs, "float32")
        run(ts, "avg", algo)
        assert ranks_identical(ts)
        assert_bits_equal(to_np(ts[0]), want, algo)
    dw = oracle.simulate_double_tree_allreduce(xs, "float32", "avg").state[0]
    for algo in ("double_tree", "double_tree_fused"):
        ts = to_gpu(xs, "float32")
        run(ts, "avg", algo)
        assert ranks_identical(ts)
        assert_bits_equal(to_np(ts[0]), dw, algo)


@pytest.mark.slow
def test_bf16_2gib_config():
    """8 ranks x 2^30 bf16 ~ N(0, 1e-2), SUM with a bf16 rounding per hop."""
    w = W.BF16_2GIB
    say("bf16 2GiB: generate")
    a = W.device_inputs(w, seed=0)
    idx = sample_positions(w.count, w.nranks, k=8192, seed=1)
    vals = gather(a, idx)
    pristine = clone_all(a)
    b = clone_all(a)
    say("bf16 2GiB: ring_step")
    run(a, "sum", "ring_step")
    say("bf16 2GiB: ring_fused")
    run(b, "sum", "ring_fused")
    for r in range(w.nranks):
        assert torch.equal(a[r], b[r]), f"fused != step on rank {r}"
    assert ranks_identical(a)
    assert ar.check(b)["mismatched"] == 0
    want = oracle.ring_fold_at(vals, chunk_ids(idx, w.count, w.nranks), w.nranks, "bfloat16", "sum")
    assert_bits_equal(gather(a[:1], idx)[0], want, "sampled positions")
    # bf16 bound: (N-1) hops of an fp32 add then a bf16 rounding
    f = oracle.bf16_to_f32(vals).astype(np.float64)
    up = 2.0 ** -8 + 2.0 ** -24 + 2.0 ** -32
    gamma = (w.nranks - 1) * up / (1 - (w.nranks - 1) * up)
    err = np.abs(oracle.bf16_to_f32(want).astype(np.float64) - f.sum(axis=0))
    assert (err <= gamma * np.abs(f).sum(axis=0)).all()
    say("bf16 2GiB: whole array against the oracle")
    per = -(-w.count // w.nranks)
    whole_array_vs_oracle(
        pristine, b[0],
        lambda v, lo: oracle.ring_fold_at(v, (np.arange(lo, lo + v.shape[1]) // per), w.nranks,
                                          "bfloat16", "sum"),
        "bf16 2GiB fused")
    del a, b, pristine
    torch.cuda.empty_cache()


@pytest.mark.parametrize("w", W.SWEEP, ids=[w.name for w in W.SWEEP])
def test_sweep_config(w):
    """64 ranks, fp32 U[-1,1], SUM: ring (per step and fused) and tree."""
    say(f"sweep {w.name}")
    full = w.count <= 16384
    if full:
        xs = W.host_inputs(w, seed=0)
        a = to_gpu(xs, "float32")
    else:
        a = W.device_inputs(w, seed=0)
        idx = sample_positions(w.count, w.nranks, k=4096, seed=2)
        vals = gather(a, idx)
    b, c, h, d = clone_all(a), clone_all(a), clone_all(a), clone_all(a)
    cf, hf, df = clone_all(a), clone_all(a), clone_all(a)
    run(a, "sum", "ring_step")
    run(b, "sum", "ring_fused")
    run(c, "sum", "tree")
    run(h, "sum", "halving_doubling")
    run(d, "sum", "double_tree")
    run(cf, "sum", "tree_fused")
    run(hf, "sum", "halving_doubling_fused")
    run(df, "sum", "double_tree_fused")
    assert ranks_identical(d)
    for r in range(w.nranks):
        assert torch.equal(a[r], b[r]), f"fused != step on rank {r}"
        assert torch.equal(c[r], cf[r]), f"tree_fused != tree on rank {r}"
        assert torch.equal(h[r], hf[r]), f"halving_doubling_fused != halving_doubling on rank {r}"
        assert torch.equal(d[r], df[r]), f"double_tree_fused != double_tree on rank {r}"
    del cf, hf, df
    assert ranks_identical(a) and ranks_identical(c) and ranks_identical(h)
    if full:
        assert_bits_equal(to_np(a[0]), oracle.simulate_ring_allreduce(xs, "float32", "sum").state[0],
                          "ring")
        assert_bits_equal(to_np(c[0]), oracle.simulate_tree_allreduce(xs, "float32", "sum").state[0],
                          "tree")
        assert_bits_equal(to_np(h[0]), oracle.simulate_hd_allreduce(xs, "float32", "sum").state[0],
                          "halving_doubling")
        assert_bits_equal(to_np(d[0]),
                          oracle.simulate_double_tree_allreduce(xs, "float32", "sum").state[0],
                          "double_tree")
    else:
        ring_want = oracle.ring_fold_at(vals, chunk_ids(idx, w.count, w.nranks), w.nranks,
                                        "float32", "sum")
        tree_want = oracle.tree_fold_at(vals, "float32", "sum")
        hd_want = oracle.hd_fold_at(vals, "float32", "sum")
        assert_bits_equal(gather(a[:1], idx)[0], ring_want, "ring sampled")
        assert_bits_equal(gather(c[:1], idx)[0], tree_want, "tree sampled")
        assert_bits_equal(gather(h[:1], idx)[0], hd_want, "hd sampled")
        half = (w.count + 1) // 2
        dt_want = np.where(idx < half, oracle.dtree_fold_at(vals, 0, "float32", "sum"),
                           oracle.dtree_fold_at(vals, 1, "float32", "sum"))
        assert_bits_equal(gather(d[:1], idx)[0], dt_want, "double tree sampled")
    del a, b, c, h, d
    torch.cuda.empty_cache()


@pytest.mark.slow
@pytest.mark.parametrize("w", [W.RAGGED_MAX, W.RAGGED_INT], ids=lambda w: w.name)
def test_ragged_config(w):
    """16 ranks x 268,435,459 elements (ragged last chunk; chunk starts cycle
    through 16-byte misalignments 0, 4, 8, 12)."""
    say(f"ragged {w.name}: generate")
    lay = oracle.chunk_layout(w.count, w.nranks)
    assert [ln for _, ln in lay] == [16_777_217] * 15 + [16_777_204]
    a = W.device_inputs(w, seed=0)
    idx = sample_positions(w.count, w.nranks, k=8192, seed=3)
    vals = gather(a, idx)
    pristine = clone_all(a)
    # independent whole-array reference computed by torch before the call
    if w.op == "max":
        ref = a[0].clone()
        for t in a[1:]:
            ref = torch.maximum(ref, t)
    else:
        acc = torch.zeros(w.count, dtype=torch.int64, device="cuda")
        for t in a:
            acc += t.to(torch.int64)
        ref = acc.to(torch.int32)
        del acc
    b = clone_all(a)
    say(f"ragged {w.name}: ring_fused")
    run(a, w.op, "ring_fused")
    say(f"ragged {w.name}: ring_step")
    run(b, w.op, "ring_step")
    for r in range(w.nranks):
        assert torch.equal(a[r], ref), f"rank {r} differs from the whole-array reference"
        assert torch.equal(b[r], ref), f"ring_step rank {r} differs"
    assert ar.check(a)["mismatched"] == 0
    want = (oracle.exact_max(vals, w.dtype) if w.op == "max" else oracle.exact_int_sum(vals))
    assert_bits_equal(gather(a[:1], idx)[0], want, "sampled positions")
    del b, ref
    say(f"ragged {w.name}: whole array against the oracle")
    whole_array_vs_oracle(
        pristine, a[0],
        (lambda v, lo: oracle.exact_max(list(v), w.dtype)) if w.op == "max"
        else (lambda v, lo: oracle.exact_int_sum(list(v))),
        f"{w.name} fused")
    del a, pristine
    torch.cuda.empty_cache()
