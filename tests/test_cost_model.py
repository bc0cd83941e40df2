"""Host-only checks of the alpha-beta cost model behind AR_ALGO_AUTO (no GPU).

The model follows the pages' latency/bandwidth form ("AllReduce",
compassingai.com, section 4: per-step latency alpha times the step count plus
bytes over bandwidth) with launches and HBM bytes of this library's kernels.
Its constants were fitted to the 64-rank sweep measured on MI355X (bench.py
--sweep), where ring-per-step and tree crossed at about 4 MiB per rank.
"""

import itertools

import pytest

ar = pytest.importorskip("ring_allreduce_rs_amd")

ALGOS = ("ring_fused", "ring_step", "tree", "halving_doubling")


def test_prediction_grows_with_size_and_steps():
    for algo, n in itertools.product(ALGOS, (2, 8, 64)):
        prev = 0.0
        for count in (0, 1, 1 << 10, 1 << 16, 1 << 20, 1 << 24):
            t = ar.predict_us(algo, n, count, "float32")
            assert t >= prev
            prev = t
    # per-step latency: more ranks, more launches
    small = 1024
    assert ar.predict_us("ring_step", 64, small, "float32") > ar.predict_us("ring_step", 8, small, "float32")


def test_ring_tree_crossover_matches_the_measured_sweep():
    # measured on MI355X: 64 ranks fp32, ring per step vs tree crossed at ~4 MiB / rank
    def diff(mib):
        c = int(mib * (1 << 20)) // 4
        return ar.predict_us("ring_step", 64, c, "float32") - ar.predict_us("tree", 64, c, "float32")
    assert diff(1) > 0          # small messages: the tree's 6 launches beat 126
    assert diff(16) < 0         # large messages: the ring's bytes win
    lo, hi = 1.0, 16.0
    for _ in range(40):
        mid = (lo + hi) / 2
        lo, hi = (mid, hi) if diff(mid) > 0 else (lo, mid)
    assert 2.0 < lo < 8.0


def test_auto_is_the_argmin():
    for n, count, dt in itertools.product((1, 2, 3, 8, 16, 64), (0, 7, 4096, 1 << 22),
                                          ("float32", "bfloat16", "int32")):
        pick = ar.auto_algo(n, count, dt)
        cands = [a for a in ALGOS if a in ("ring_fused", "ring_step") or n & (n - 1) == 0]
        best = min(cands, key=lambda a: ar.predict_us(a, n, count, dt))
        assert ar.predict_us(pick, n, count, dt) == ar.predict_us(best, n, count, dt)


def test_model_rejects_bad_arguments():
    with pytest.raises(ar.ArError) as e:
        ar.predict_us("tree", 3, 10, "float32")
    assert e.value.status == 2
    with pytest.raises(ar.ArError):
        ar.predict_us("auto", 8, 10, "float32")
    with pytest.raises(ar.ArError):
        ar.predict_us("ring_fused", 0, 10, "float32")
    with pytest.raises(ar.ArError):
        ar.auto_algo(65, 10, "float32")
