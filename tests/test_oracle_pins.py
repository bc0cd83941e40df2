"""Pins for the CPU oracle: facts fixed outside the oracle itself.

Each test checks the oracle against something it cannot produce by
construction: the pages' worked examples (``tests/golden``), closed-form
traffic and step counts, exact integer arithmetic, hand-derived fp32/bf16 bit
patterns, rounding-error bounds against binary64, and invariants of the
algorithm (AllReduce = ReduceScatter + AllGather, one finished chunk per rank
after ReduceScatter, AllGather copies without changing bits).  The last group
plants mistakes in the oracle and shows that a pin fails for each.
"""

import numpy as np
import pytest

import oracle
from oracle import elementops, ring as oring
from workloads import Workload, host_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def h(s):
    return int(s, 16)


def _rand(dtype, n, count, seed, kind="normal"):
    rng = np.random.Generator(np.random.PCG64(seed))
    if dtype == "int32":
        return [rng.integers(-2**31, 2**31, size=count, dtype=np.int64).astype(np.int32)
                for _ in range(n)]
    f = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
    if dtype == "float32":
        return f
    # bf16 by truncating random fp32 bit patterns (any bf16 value is fine here)
    return [(x.view(np.uint32) >> np.uint32(16)).astype(np.uint16) for x in f]


def _bits(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    return a


# ---------------------------------------------------------------- layout

def test_layout_closed_forms():
    assert oracle.chunk_layout(1024, 4) == [(0, 256), (256, 256), (512, 256), (768, 256)]
    assert oracle.chunk_layout(1, 3) == [(0, 1), (1, 0), (1, 0)]
    assert [ln for _, ln in oracle.chunk_layout(6, 4)] == [2, 2, 2, 0]
    big = oracle.chunk_layout(268_435_459, 16)
    assert [ln for _, ln in big] == [16_777_217] * 15 + [16_777_204]
    assert [ln for _, ln in oracle.chunk_layout(6_553_600, 8)] == [819_200] * 8
    assert oracle.chunk_layout(0, 5) == [(0, 0)] * 5


@pytest.mark.parametrize("n", range(1, 10))
def test_layout_partitions_every_count(n):
    for count in (0, 1, 2, n - 1, n, 2 * n + 1, 37, 100):
        if count < 0:
            continue
        lay = oracle.chunk_layout(count, n)
        assert len(lay) == n
        pos = 0
        for lo, ln in lay:
            assert lo == pos and ln >= 0
            pos += ln
        assert pos == count
        per = -(-count // n)
        assert all(ln <= per for _, ln in lay)
        # only trailing chunks may be short
        lens = [ln for _, ln in lay]
        assert lens == sorted(lens, reverse=True)
        for i in range(count):
            c = oracle.chunk_of(i, count, n)
            assert lay[c][0] <= i < lay[c][0] + lay[c][1]


# ---------------------------------------------------------------- worked examples

@pytest.mark.parametrize("count", [1, 3])
def test_three_rank_example(golden, count):
    g = golden("three_rank_sum.json")
    xs = [np.full(count, v, dtype=np.int32) for v in g["inputs_per_rank_value"]]
    tr = oracle.simulate_ring_allreduce(xs, "int32", "sum")
    for r in range(g["nranks"]):
        assert (tr.state[r] == g["expected_value_every_rank"]).all()
    with pytest.raises(ValueError):
        oracle.simulate_tree_allreduce(xs, "int32", "sum")   # 3 is not a power of two


def test_four_rank_example(golden):
    g = golden("four_rank_ones_2x3.json")
    xs = [np.ones((2, 3), dtype=np.float32) * v for v in g["inputs_per_rank_value"]]
    assert [ln for _, ln in oracle.chunk_layout(g["count"], g["nranks"])] == [2, 2, 2, 0]
    for algo in (oracle.simulate_ring_allreduce, oracle.simulate_tree_allreduce):
        s = algo(xs, "float32", "sum")
        a = algo(xs, "float32", "avg")
        for r in range(4):
            assert (s.state[r] == g["expected_sum_every_element"]).all()
            assert (a.state[r] == g["expected_avg_every_element"]).all()


@pytest.mark.parametrize("n", range(1, 10))
def test_rank_valued_closed_form(n):
    # each rank holds ones(4) * rank; SUM is n(n-1)/2 everywhere, AVG (n-1)/2
    xs = [np.ones(4, dtype=np.float32) * r for r in range(n)]
    s = oracle.simulate_ring_allreduce(xs, "float32", "sum")
    a = oracle.simulate_ring_allreduce(xs, "float32", "avg")
    for r in range(n):
        assert (s.state[r] == n * (n - 1) / 2).all()
        assert (a.state[r] == (n - 1) / 2).all()
    if n & (n - 1) == 0:
        t = oracle.simulate_tree_allreduce(xs, "float32", "avg")
        for r in range(n):
            assert (t.state[r] == (n - 1) / 2).all()


# ---------------------------------------------------------------- exact integer results

@pytest.mark.parametrize("n", range(1, 10))
def test_int32_bruteforce(n):
    for count in sorted({0, 1, 2, max(n - 1, 0), n, 2 * n + 1, 37}):
        xs = _rand("int32", n, count, seed=100 * n + count)
        ref_sum = np.zeros(count, dtype=np.int64)
        for x in xs:                       # brute force, element by element
            ref_sum += x.astype(np.int64)
        ref_sum = ((ref_sum + 2**31) % 2**32 - 2**31).astype(np.int32)
        ref_max = np.array([max(int(x[i]) for x in xs) for i in range(count)], dtype=np.int32)
        assert (oracle.exact_int_sum(xs) == ref_sum).all()
        assert (oracle.exact_max(xs, "int32") == ref_max).all()
        rs = oracle.simulate_ring_allreduce(xs, "int32", "sum")
        rm = oracle.simulate_ring_allreduce(xs, "int32", "max")
        for r in range(n):
            assert (rs.state[r] == ref_sum).all()
            assert (rm.state[r] == ref_max).all()
        if n & (n - 1) == 0:
            ts = oracle.simulate_tree_allreduce(xs, "int32", "sum")
            for r in range(n):
                assert (ts.state[r] == ref_sum).all()


def test_int32_wraps():
    xs = [np.array([2**31 - 1, -2**31], dtype=np.int32), np.array([1, -1], dtype=np.int32)]
    tr = oracle.simulate_ring_allreduce(xs, "int32", "sum")
    assert tr.state[0].tolist() == [-2**31, 2**31 - 1]
    assert tr.state[1].tolist() == [-2**31, 2**31 - 1]


def test_int32_avg_undefined():
    with pytest.raises(ValueError):
        oracle.simulate_ring_allreduce([np.ones(4, np.int32)] * 2, "int32", "avg")


@pytest.mark.parametrize("n", [2, 3, 5, 8, 16])
def test_fp32_integer_valued_is_exact(n):
    # integer-valued fp32 with every partial sum below 2^24 adds without rounding
    rng = np.random.Generator(np.random.PCG64(n))
    ints = [rng.integers(-1000, 1001, size=301).astype(np.int32) for _ in range(n)]
    xs = [x.astype(np.float32) for x in ints]
    exact = oracle.exact_int_sum(ints).astype(np.float32)
    tr = oracle.simulate_ring_allreduce(xs, "float32", "sum")
    for r in range(n):
        assert (tr.state[r] == exact).all()
    mx = oracle.simulate_ring_allreduce(xs, "float32", "max")
    assert (mx.state[0] == oracle.exact_max(ints, "int32").astype(np.float32)).all()


# ---------------------------------------------------------------- error bounds vs binary64

@pytest.mark.parametrize("n", [2, 3, 5, 8, 16])
@pytest.mark.parametrize("count", [37, 1000])
def test_fp32_ring_within_bound(n, count):
    xs = _rand("float32", n, count, seed=7 * n + count)
    tr = oracle.simulate_ring_allreduce(xs, "float32", "sum")
    ref = np.stack(xs).astype(np.float64).sum(axis=0)            # binary64 reference
    absum = np.abs(np.stack(xs).astype(np.float64)).sum(axis=0)
    u = 2.0 ** -24
    gamma = (n - 1) * u / (1 - (n - 1) * u)                       # left-to-right sum bound
    err = np.abs(tr.state[0].astype(np.float64) - ref)
    assert (err <= gamma * absum).all()
    # not trivially exact: some element must actually round
    if n > 2:
        assert (err > 0).any()


@pytest.mark.parametrize("n", [2, 4, 8])
def test_bf16_ring_within_bound(n):
    w = Workload("b", n, 999, "bfloat16", ("normal", 1e-2), "sum")
    xs = host_inputs(w, seed=n)
    tr = oracle.simulate_ring_allreduce(xs, "bfloat16", "sum")
    f = np.stack([oracle.bf16_to_f32(x) for x in xs]).astype(np.float64)
    ref = f.sum(axis=0)
    up = 2.0 ** -8 + 2.0 ** -24 + 2.0 ** -32          # one fp32 add then one bf16 rounding
    gamma = (n - 1) * up / (1 - (n - 1) * up)
    err = np.abs(oracle.bf16_to_f32(tr.state[0]).astype(np.float64) - ref)
    assert (err <= gamma * np.abs(f).sum(axis=0)).all()


def test_fp64_sum_matches_fsum():
    import math
    xs = _rand("float32", 5, 50, seed=3)
    ref = [math.fsum(float(x[i]) for x in xs) for i in range(50)]
    assert np.allclose(oracle.fp64_sum(xs, "float32"), ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- fold order and bit patterns

def test_ring_fold_order_golden(golden):
    g = golden("fold_order_n4_fp32.json")
    xs = [np.array(x, dtype=np.float32) for x in g["inputs"]]
    expect = np.array(g["expected_every_rank"], dtype=np.float32)
    other = np.array(g["expected_other_reading"], dtype=np.float32)
    tr = oracle.simulate_ring_allreduce(xs, "float32", "sum")
    for r in range(g["nranks"]):
        assert (_bits(tr.state[r]) == _bits(expect)).all()
    assert (_bits(oracle.ordered_ring_fold(xs, "float32", "sum")) == _bits(expect)).all()
    alt = oracle.simulate_ring_allreduce(xs, "float32", "sum", rotation=1)
    assert (_bits(alt.state[0]) == _bits(other)).all()


def test_tree_order_golden(golden):
    g = golden("tree_order_n4_fp32.json")
    xs = [np.array(x, dtype=np.float32) for x in g["inputs"]]
    expect = np.array(g["expected_every_rank"], dtype=np.float32)
    tr = oracle.simulate_tree_allreduce(xs, "float32", "sum")
    for r in range(4):
        assert (_bits(tr.state[r]) == _bits(expect)).all()
    assert (_bits(oracle.pairwise_tree_fold(xs, "float32", "sum")) == _bits(expect)).all()


def test_bf16_bits_golden(golden):
    g = golden("bf16_hop_bits.json")
    for c in g["cases_sum"]:
        a = np.array([h(c["a"])], np.uint16)
        b = np.array([h(c["b"])], np.uint16)
        assert int(oracle.hop(a, b, "bfloat16", "sum")[0]) == h(c["expect"]), c["why"]
        assert int(oracle.hop(b, a, "bfloat16", "sum")[0]) == h(c["expect"]), c["why"]
    for c in g["cases_max"]:
        a = np.array([h(c["a"])], np.uint16)
        b = np.array([h(c["b"])], np.uint16)
        assert int(oracle.hop(a, b, "bfloat16", "max")[0]) == h(c["expect"]), c["why"]
        assert int(oracle.hop(b, a, "bfloat16", "max")[0]) == h(c["expect"]), c["why"]
    for c in g["cases_avg"]:
        s = np.array([h(c["sum"])], np.uint16)
        assert int(oracle.avg_epilogue(s, c["nranks"], "bfloat16")[0]) == h(c["expect"]), c["why"]


def test_fp32_bits_golden(golden):
    g = golden("fp32_edge_bits.json")

    def f(s):
        return np.array([h(s)], np.uint32).view(np.float32)
    for c in g["cases_max"]:
        for a, b in ((c["a"], c["b"]), (c["b"], c["a"])):
            got = oracle.hop(f(a), f(b), "float32", "max")
            assert int(got.view(np.uint32)[0]) == h(c["expect"]), c["why"]
    for c in g["cases_sum"]:
        got = oracle.hop(f(c["a"]), f(c["b"]), "float32", "sum")
        assert int(got.view(np.uint32)[0]) == h(c["expect"]), c["why"]
    for c in g["cases_avg"]:
        got = oracle.avg_epilogue(f(c["sum"]), c["nranks"], "float32")
        assert int(got.view(np.uint32)[0]) == h(c["expect"]), c["why"]


def test_bf16_rounding_matches_exact_rational():
    # round-to-nearest-even checked against exact rational arithmetic
    from fractions import Fraction
    rng = np.random.Generator(np.random.PCG64(11))
    u = rng.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) < 3e38)
    f = f[keep]
    got = oracle.f32_to_bf16_rne(f)
    for x, b in zip(f[:1500], got[:1500]):
        xv = Fraction(float(x))
        lo = int((np.array([x]).view(np.uint32)[0] >> 16))
        cands = [lo, lo + 1]
        vals = [Fraction(float(oracle.bf16_to_f32(np.array([c], np.uint16))[0])) for c in cands]
        d = [abs(v - xv) for v in vals]
        if d[0] < d[1]:
            want = cands[0]
        elif d[1] < d[0]:
            want = cands[1]
        else:
            want = cands[0] if cands[0] % 2 == 0 else cands[1]
        assert int(b) == want


# ---------------------------------------------------------------- invariants

CASES = [(n, c) for n in (1, 2, 3, 4, 5, 8, 9) for c in (0, 1, 2, n + 1, 37, 64)]


@pytest.mark.parametrize("dtype", ["int32", "float32", "bfloat16"])
@pytest.mark.parametrize("n,count", CASES)
def test_allreduce_is_reduce_scatter_then_allgather(dtype, n, count):
    xs = _rand(dtype, n, count, seed=n * 1000 + count)
    ops = ["sum", "max"] + (["avg"] if dtype != "int32" else [])
    for op in ops:
        ar = oracle.simulate_ring_allreduce(xs, dtype, op)
        rs = oracle.simulate_ring_reduce_scatter(xs, dtype, op)
        ag = oracle.simulate_ring_allgather(rs.state, dtype)
        direct = oracle.ordered_ring_fold(xs, dtype, op)
        lay = oracle.chunk_layout(count, n)
        for r in range(n):
            assert (_bits(ar.state[r]) == _bits(ag.state[r])).all()
            assert (_bits(ar.state[r]) == _bits(ar.state[0])).all()   # all ranks identical
            lo, ln = lay[r]
            # after ReduceScatter rank r holds the finished chunk r
            assert (_bits(rs.state[r][lo:lo + ln]) == _bits(direct[lo:lo + ln])).all()
        assert (_bits(ar.state[0]) == _bits(direct)).all()


@pytest.mark.parametrize("n,count", [(4, 17), (5, 5), (8, 64), (3, 1)])
def test_allgather_copies_owner_chunks_unchanged(n, count):
    xs = _rand("float32", n, count, seed=count)
    ag = oracle.simulate_ring_allgather(xs, "float32")
    lay = oracle.chunk_layout(count, n)
    for r in range(n):
        for c, (lo, ln) in enumerate(lay):
            assert (_bits(ag.state[r][lo:lo + ln]) == _bits(xs[c][lo:lo + ln])).all()


@pytest.mark.parametrize("n", [2, 4, 8, 16])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "int32"])
def test_tree_matches_pairwise_fold(n, dtype):
    xs = _rand(dtype, n, 53, seed=n)
    ops = ["sum", "max"] + (["avg"] if dtype != "int32" else [])
    for op in ops:
        tr = oracle.simulate_tree_allreduce(xs, dtype, op)
        ref = oracle.pairwise_tree_fold(xs, dtype, op)
        for r in range(n):
            assert (_bits(tr.state[r]) == _bits(ref)).all()


def test_ring_fold_at_matches_full_fold():
    n, count = 7, 1000
    xs = _rand("float32", n, count, seed=5)
    full = oracle.ordered_ring_fold(xs, "float32", "avg")
    idx = np.array([0, 1, 142, 143, 144, 500, 857, 858, 999])
    chunks = [oracle.chunk_of(int(i), count, n) for i in idx]
    vals = np.stack([x[idx] for x in xs])
    at = oracle.ring_fold_at(vals, chunks, n, "float32", "avg")
    assert (_bits(at) == _bits(full[idx])).all()


# ---------------------------------------------------------------- traffic and steps

@pytest.mark.parametrize("n", range(1, 10))
@pytest.mark.parametrize("dtype", ["int32", "bfloat16"])
def test_ring_traffic_closed_form(n, dtype):
    isz = 4 if dtype == "int32" else 2
    for count in (0, 1, n, 3 * n, 3 * n + 1, 37):
        xs = _rand(dtype, n, count, seed=count)
        tr = oracle.simulate_ring_allreduce(xs, dtype, "sum")
        k_bytes = count * isz
        lay = oracle.chunk_layout(count, n)
        assert tr.steps == 2 * (n - 1)
        if count % n == 0:
            assert tr.sent == tr.recv          # equal send and receive per rank
        for r in range(n):
            expect = 2 * k_bytes - lay[r][1] * isz - lay[(r + 1) % n][1] * isz
            if n == 1:
                expect = 0
            assert tr.sent[r] == expect
            # rank r receives what its predecessor sends
            assert tr.recv[r] == tr.sent[(r - 1) % n]
            if count % n == 0:
                assert tr.sent[r] * n == 2 * (n - 1) * k_bytes     # 2(N-1)/N * K
        assert sum(tr.sent) == sum(tr.recv)
        if count % n == 0:
            assert sum(tr.sent) == 2 * (n - 1) * k_bytes


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64])
def test_tree_steps_and_traffic(n):
    xs = _rand("float32", n, 10, seed=n)
    tr = oracle.simulate_tree_allreduce(xs, "float32", "sum")
    logn = n.bit_length() - 1
    assert tr.steps == logn
    assert tr.sent == [40 * logn] * n and tr.recv == [40 * logn] * n


def test_broken_ring_raises():
    xs = _rand("float32", 4, 16, seed=1)
    for step in range(6):
        with pytest.raises(oracle.BrokenRing):
            oracle.simulate_ring_allreduce(xs, "float32", "sum", drop=(2, step))
    with pytest.raises(oracle.BrokenRing):
        oracle.simulate_tree_allreduce(xs, "float32", "sum", drop=(1, 1))


def test_record_snapshots_count():
    xs = _rand("float32", 5, 23, seed=2)
    tr = oracle.simulate_ring_allreduce(xs, "float32", "avg", record=True)
    assert len(tr.snapshots) == 8
    # the last snapshot is the result; the snapshot after ReduceScatter holds
    # the finished (and averaged) chunk r on rank r
    direct = oracle.ordered_ring_fold(xs, "float32", "avg")
    lay = oracle.chunk_layout(23, 5)
    for r in range(5):
        lo, ln = lay[r]
        assert (_bits(tr.snapshots[3][r][lo:lo + ln]) == _bits(direct[lo:lo + ln])).all()
        assert (_bits(tr.snapshots[-1][r]) == _bits(direct)).all()


# ---------------------------------------------------------------- planted mistakes

def test_planted_mistakes_are_caught(golden, monkeypatch):
    """Each plausible oracle bug makes at least one pin above fail."""
    g = golden("fold_order_n4_fp32.json")
    xs4 = [np.array(x, dtype=np.float32) for x in g["inputs"]]
    expect4 = np.array(g["expected_every_rank"], dtype=np.float32)
    g2 = golden("four_rank_ones_2x3.json")
    ones = [np.ones(6, np.float32) * v for v in g2["inputs_per_rank_value"]]

    def fold_pin_holds():
        return (_bits(oracle.simulate_ring_allreduce(xs4, "float32", "sum").state[0])
                == _bits(expect4)).all()

    def avg_pin_holds():
        return (oracle.simulate_ring_allreduce(ones, "float32", "avg").state[1] == 2.5).all()

    def int_pin_holds():
        xs = _rand("int32", 5, 37, seed=9)
        return (oracle.simulate_ring_allreduce(xs, "int32", "sum").state[3]
                == oracle.exact_int_sum(xs)).all()

    assert fold_pin_holds() and avg_pin_holds() and int_pin_holds()

    real_hop = elementops.hop
    # 1. a dropped term: the receiver ignores what it was sent
    monkeypatch.setattr(oring, "hop", lambda a, b, d, o: b)
    assert not int_pin_holds()
    monkeypatch.setattr(oring, "hop", real_hop)
    # 2. a wrong divisor in the AVG epilogue
    real_avg = elementops.avg_epilogue
    monkeypatch.setattr(oring, "avg_epilogue", lambda a, n, d: real_avg(a, n - 1, d))
    assert not avg_pin_holds()
    monkeypatch.setattr(oring, "avg_epilogue", real_avg)
    # 3. a wrong chunk index in the schedule (off by one)
    real_run = oring._run_reduce_scatter
    monkeypatch.setattr(oring, "_run_reduce_scatter",
                        lambda tr, d, o, rot, rec, drop, s0: real_run(tr, d, o, rot + 1, rec, drop, s0))
    assert not fold_pin_holds()
    monkeypatch.setattr(oring, "_run_reduce_scatter", real_run)
    # 4. truncation instead of round-to-nearest-even in bf16
    real_rne = elementops.f32_to_bf16_rne
    monkeypatch.setattr(elementops, "f32_to_bf16_rne",
                        lambda x: (np.ascontiguousarray(x, np.float32).view(np.uint32)
                                   >> np.uint32(16)).astype(np.uint16))
    a = np.array([0x3F81], np.uint16)
    b = np.array([0x3B80], np.uint16)
    assert int(elementops.hop(a, b, "bfloat16", "sum")[0]) != 0x3F82
    monkeypatch.setattr(elementops, "f32_to_bf16_rne", real_rne)
    # 5. a sign error in one operand
    monkeypatch.setattr(oring, "hop", lambda a, b, d, o: real_hop(a, -b, d, o))
    assert not int_pin_holds()
    monkeypatch.setattr(oring, "hop", real_hop)
    assert fold_pin_holds() and avg_pin_holds() and int_pin_holds()


# ---------------------------------------------------------------- halving-doubling

def test_hd_order_golden(golden):
    g = golden("hd_order_n4_fp32.json")
    xs = [np.array(x, dtype=np.float32) for x in g["inputs"]]
    expect = np.array(g["expected_every_rank"], dtype=np.float32)
    tr = oracle.simulate_hd_allreduce(xs, "float32", "sum")
    for r in range(4):
        assert (_bits(tr.state[r]) == _bits(expect)).all()
    assert (_bits(oracle.hd_fold_at(np.stack(xs), "float32", "sum")) == _bits(expect)).all()
    # recursive doubling pairs differently
    rd = oracle.simulate_tree_allreduce(xs, "float32", "sum").state[0]
    assert not (_bits(rd) == _bits(expect)).all()


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16])
def test_hd_int32_exact_and_invariants(n):
    for count in (0, 1, n - 1, n, 3 * n + 1, 37, 200):
        xs = _rand("int32", n, count, seed=n * 13 + count)
        exact = oracle.exact_int_sum(xs)
        ar_ = oracle.simulate_hd_allreduce(xs, "int32", "sum")
        mx = oracle.simulate_hd_allreduce(xs, "int32", "max")
        for r in range(n):
            assert (ar_.state[r] == exact).all()
            assert (mx.state[r] == oracle.exact_max(xs, "int32")).all()
        assert ar_.steps == 2 * (n.bit_length() - 1)


@pytest.mark.parametrize("n", [2, 4, 8, 16])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_hd_rs_ag_and_direct_fold(n, dtype):
    for count in (n, 5 * n + 3, 97):
        xs = _rand(dtype, n, count, seed=count + n)
        for op in ("sum", "max", "avg"):
            ar_ = oracle.simulate_hd_allreduce(xs, dtype, op)
            rs = oracle.simulate_hd_reduce_scatter(xs, dtype, op)
            ag = oracle.simulate_hd_allgather(rs.state, dtype)
            direct = oracle.hd_fold_at(np.stack(xs), dtype, op)
            lay = oracle.chunk_layout(count, n)
            for r in range(n):
                lo, ln = lay[r]
                assert (_bits(rs.state[r][lo:lo + ln]) == _bits(direct[lo:lo + ln])).all()
                assert (_bits(ag.state[r]) == _bits(ar_.state[r])).all()
                assert (_bits(ar_.state[r]) == _bits(direct)).all()


@pytest.mark.parametrize("n", [2, 4, 8, 16, 64])
def test_hd_traffic_closed_form(n):
    count = 3 * n
    xs = _rand("float32", n, count, seed=1)
    tr = oracle.simulate_hd_allreduce(xs, "float32", "sum")
    k_bytes = count * 4
    for r in range(n):
        assert tr.sent[r] * n == 2 * (n - 1) * k_bytes      # 2(N-1)/N * K, like the ring
        assert tr.recv[r] == tr.sent[r]
    for count in (1, n + 1, 7 * n - 3):                      # ragged: the total is still 2(N-1)K
        xs = _rand("float32", n, count, seed=2)
        tr = oracle.simulate_hd_allreduce(xs, "float32", "sum")
        assert sum(tr.sent) == 2 * (n - 1) * count * 4 == sum(tr.recv)


def test_hd_fp32_bound_and_broken():
    xs = _rand("float32", 8, 500, seed=4)
    tr = oracle.simulate_hd_allreduce(xs, "float32", "sum")
    ref = np.stack(xs).astype(np.float64).sum(axis=0)
    absum = np.abs(np.stack(xs).astype(np.float64)).sum(axis=0)
    u = 2.0 ** -24
    assert (np.abs(tr.state[0] - ref) <= 3 * u / (1 - 3 * u) * absum).all()   # depth log2 8 = 3
    with pytest.raises(oracle.BrokenRing):
        oracle.simulate_hd_allreduce(xs, "float32", "sum", drop=(3, 4))
    with pytest.raises(ValueError):
        oracle.simulate_hd_allreduce(xs[:3], "float32", "sum")


# ---------------------------------------------------------------- double binary tree

def test_dtree_shape_is_complementary():
    from oracle.double_tree import children, rank_at
    for n in (2, 4, 8, 16, 64):
        for t in (0, 1):
            seen = [rank_at(t, 0, n)]
            stack = [0]
            while stack:                                   # every position reached once
                v = stack.pop()
                for c in children(v, n):
                    seen.append(rank_at(t, c, n))
                    stack.append(c)
            assert sorted(seen) == list(range(n))
        if n >= 4:
            leaves = [{rank_at(t, v, n) for v in range(1, n) if not children(v, n)} for t in (0, 1)]
            interior = [set(range(n)) - lv for lv in leaves]
            assert leaves[0] <= interior[1] and leaves[1] <= interior[0]


def test_dtree_order_golden(golden):
    g = golden("dtree_order_n4_fp32.json")
    xs = [np.array(x, dtype=np.float32) for x in g["inputs"]]
    expect = np.array(g["expected_every_rank"], dtype=np.float32)
    tr = oracle.simulate_double_tree_allreduce(xs, "float32", "sum")
    for r in range(4):
        assert (_bits(tr.state[r]) == _bits(expect)).all()
    assert (_bits(oracle.double_tree_fold(xs, "float32", "sum")) == _bits(expect)).all()
    rd = oracle.simulate_tree_allreduce(xs, "float32", "sum").state[0]
    assert not (_bits(rd) == _bits(expect)).all()


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16])
def test_dtree_int32_exact_and_steps(n):
    for count in (0, 1, 2, n, 3 * n + 1, 37, 200):
        xs = _rand("int32", n, count, seed=n * 7 + count)
        tr = oracle.simulate_double_tree_allreduce(xs, "int32", "sum")
        mx = oracle.simulate_double_tree_allreduce(xs, "int32", "max")
        for r in range(n):
            assert (tr.state[r] == oracle.exact_int_sum(xs)).all()
            assert (mx.state[r] == oracle.exact_max(xs, "int32")).all()
        assert tr.steps == 2 * (n.bit_length() - 1)


@pytest.mark.parametrize("n", [2, 4, 8, 16])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_dtree_matches_direct_fold(n, dtype):
    for count in (1, n + 3, 101):
        xs = _rand(dtype, n, count, seed=count * n)
        for op in ("sum", "max", "avg"):
            tr = oracle.simulate_double_tree_allreduce(xs, dtype, op)
            ref = oracle.double_tree_fold(xs, dtype, op)
            for r in range(n):
                assert (_bits(tr.state[r]) == _bits(ref)).all()


@pytest.mark.parametrize("n", [2, 4, 8, 16, 64])
def test_dtree_traffic_closed_form(n):
    from oracle.double_tree import children, rank_at
    count = 2 * n + 1                                   # halves of n+1 and n elements
    xs = _rand("float32", n, count, seed=3)
    tr = oracle.simulate_double_tree_allreduce(xs, "float32", "sum")
    halves = [(n + 1) * 4, n * 4]
    # per tree: N-1 partials go up and N-1 results come down
    assert sum(tr.sent) == sum(tr.recv) == 2 * (n - 1) * sum(halves)
    for r in range(n):
        want = 0
        for t in (0, 1):
            v = [p for p in range(n) if rank_at(t, p, n) == r][0]
            # up: a non-root sends its partial once; down: one copy per child
            want += ((v != 0) + len(children(v, n))) * halves[t]
        assert tr.sent[r] == want == tr.recv[r]
    with pytest.raises(oracle.BrokenRing):
        oracle.simulate_double_tree_allreduce(xs, "float32", "sum", drop=(1, 0))


def test_sampled_tree_folds_equal_the_whole_vector_folds():
    """The per-position forms that the full-size GPU tests call on sampled
    columns (tree_fold_at, dtree_fold_at, ring_fold_at) give, column by
    column, the whole-vector folds that the goldens above pin."""
    rng = np.random.Generator(np.random.PCG64(404))
    for n in (2, 4, 8, 16):
        count = 6 * n + 5
        xs = [rng.standard_normal(count).astype(np.float32) for _ in range(n)]
        vals = np.stack(xs)
        cols = np.array([0, 1, count // 2, count - 1])
        for op in ("sum", "max", "avg"):
            tree = oracle.pairwise_tree_fold(xs, "float32", op)
            assert (_bits(oracle.tree_fold_at(vals[:, cols], "float32", op)) == _bits(tree[cols])).all()
            dt = oracle.double_tree_fold(xs, "float32", op)
            ring = oracle.ordered_ring_fold(xs, "float32", op)
            chunk = np.array([oracle.chunk_of(int(i), count, n) for i in cols])
            assert (_bits(oracle.ring_fold_at(vals[:, cols], chunk, n, "float32", op))
                    == _bits(ring[cols])).all()
            first = (count + 1) // 2
            for tree_id, sel in ((0, cols[cols < first]), (1, cols[cols >= first])):
                got = oracle.dtree_fold_at(vals[:, sel], tree_id, "float32", op)
                assert (_bits(got) == _bits(dt[sel])).all(), (n, op, tree_id)
