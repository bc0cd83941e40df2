"""Pins for the oracle's direct references ``exact_max`` and ``fp64_sum`` on
the floating-point types.

MAX is one of the reduction operators an AllReduce applies ("AllReduce",
compassingai.com, section 3 技术原理).  For it the oracle's reference is the
plain definition -- the elementwise maximum over all ranks -- under the
IEEE-754-2019 ``maximum`` rule this library reads into the pages (a NaN
operand makes the result NaN, returned as the canonical quiet NaN; +0 ranks
above -0).  The pins below recompute that maximum element by element in plain
Python from the numbers' values (``math``/``struct``, no numpy arithmetic and
none of the oracle's helpers), on random values mixed with NaN, signed zeros,
infinities, subnormals and the largest finite values, for 1 to 9 ranks.

``fp64_sum`` is the binary64 sum used for error bounds.  On inputs whose exact
sum fits in 53 bits it must equal ``math.fsum`` (the correctly rounded sum)
exactly; the bf16 branch decodes bf16 with ``struct`` here, independently of
the oracle's widening.

The last tests plant plausible mistakes in the oracle (NaN dropped, signed
zeros compared as equal, a rank left out, bf16 widened by value instead of by
bit pattern, a binary32 accumulator) and show that a pin fails for each.
"""

import math
import struct

import numpy as np
import pytest

import oracle
from oracle import direct

F32_QNAN = 0x7FC00000
BF16_QNAN = 0x7FC0

# bit patterns worth having in every column mix
F32_SPECIAL = [
    0x00000000, 0x80000000,                  # +0, -0
    0x7F800000, 0xFF800000,                  # +inf, -inf
    0x7FC00000, 0xFFC00000, 0x7F800001,      # quiet NaN, negative NaN, signalling NaN
    0x7FFFFFFF,                              # NaN with a full payload
    0x00000001, 0x80000001,                  # smallest subnormals
    0x007FFFFF, 0x807FFFFF,                  # largest subnormals
    0x00800000, 0x80800000,                  # smallest normals
    0x7F7FFFFF, 0xFF7FFFFF,                  # largest finite
    0x3F800000, 0xBF800000,                  # +1, -1
]
BF16_SPECIAL = [
    0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC0, 0x7F81, 0x7FFF,
    0x0001, 0x8001, 0x007F, 0x807F, 0x0080, 0x8080, 0x7F7F, 0xFF7F, 0x3F80, 0xBF80,
]


def f32_of(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def bf16_of(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits << 16))[0]


def py_maximum_index(values):
    """Index of the IEEE-754-2019 maximum of a list of Python floats, or None
    when one of them is a NaN (then the result is NaN).  Among equal values
    +0 beats -0; any other tie picks an equal value, so the bits agree."""
    if any(math.isnan(v) for v in values):
        return None
    best = 0
    for i in range(1, len(values)):
        a, b = values[best], values[i]
        if b > a or (b == a and math.copysign(1.0, b) > math.copysign(1.0, a)):
            best = i
    return best


def brute_max_bits(cols_bits, decode, qnan):
    """Per position: the bits of the maximum of that position's rank values.
    With one rank nothing is combined (an AllReduce over one rank leaves the
    data as it is), so the bits pass through, a NaN payload included."""
    out = []
    for col in cols_bits:
        if len(col) == 1:
            out.append(col[0])
            continue
        i = py_maximum_index([decode(b) for b in col])
        out.append(qnan if i is None else col[i])
    return out


def mixed_bits(rng, n, count, special, width):
    """n ranks x count bit patterns: random finite values (of several
    magnitudes) with a fraction of special patterns mixed in."""
    if width == 32:
        vals = (rng.standard_normal((n, count)) *
                rng.choice([1e-40, 1e-3, 1.0, 1e30], size=(n, count))).astype(np.float32)
        bits = vals.view(np.uint32).astype(np.int64)
    else:
        vals = (rng.standard_normal((n, count)) *
                rng.choice([1e-40, 1e-3, 1.0, 1e30], size=(n, count))).astype(np.float32)
        bits = (vals.view(np.uint32) >> np.uint32(16)).astype(np.int64)
    mask = rng.random((n, count)) < 0.3
    bits[mask] = rng.choice(np.array(special, dtype=np.int64), size=int(mask.sum()))
    return bits


def as_rank_arrays(bits, width):
    if width == 32:
        return [b.astype(np.uint32).view(np.float32) for b in bits]
    return [b.astype(np.uint16) for b in bits]


def got_bits(res, width):
    res = np.ascontiguousarray(res)
    return (res.view(np.uint32) if width == 32 else res.astype(np.uint16)).astype(np.int64).tolist()


@pytest.mark.parametrize("n", range(1, 10))
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_exact_max_float_bruteforce(n, dtype):
    width = 32 if dtype == "float32" else 16
    special = F32_SPECIAL if width == 32 else BF16_SPECIAL
    decode = f32_of if width == 32 else bf16_of
    qnan = F32_QNAN if width == 32 else BF16_QNAN
    rng = np.random.Generator(np.random.PCG64(1000 + n + width))
    bits = mixed_bits(rng, n, 300, special, width)
    want = brute_max_bits(bits.T.tolist(), decode, qnan)
    got = got_bits(oracle.exact_max(as_rank_arrays(bits, width), dtype), width)
    assert got == want


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_exact_max_float_edge_cases(dtype):
    """Hand-listed columns: the answer of each is written out."""
    if dtype == "float32":
        P0, N0, PINF, NINF, QNAN, SUB, NSUB, ONE, MAXF = (
            0x00000000, 0x80000000, 0x7F800000, 0xFF800000, F32_QNAN, 0x00000001, 0x80000001,
            0x3F800000, 0x7F7FFFFF)
        nan_payload, neg_nan = 0x7F800001, 0xFFC00000
        width, qnan = 32, F32_QNAN
    else:
        P0, N0, PINF, NINF, QNAN, SUB, NSUB, ONE, MAXF = (
            0x0000, 0x8000, 0x7F80, 0xFF80, BF16_QNAN, 0x0001, 0x8001, 0x3F80, 0x7F7F)
        nan_payload, neg_nan = 0x7F81, 0xFFC0
        width, qnan = 16, BF16_QNAN
    cases = [
        ([N0, P0], P0), ([P0, N0], P0), ([N0, N0], N0), ([N0, N0, N0], N0),
        ([NSUB, N0], N0), ([N0, NSUB], N0), ([SUB, P0], SUB), ([NSUB, SUB], SUB),
        ([NINF, NSUB], NSUB), ([NINF, NINF], NINF), ([MAXF, PINF], PINF),
        ([ONE, MAXF, NINF], MAXF), ([QNAN, ONE], qnan), ([ONE, nan_payload], qnan),
        ([neg_nan, PINF], qnan), ([PINF, ONE, N0, neg_nan], qnan),
    ]
    for col, expect in cases:
        n = len(col)
        bits = np.array(col, dtype=np.int64).reshape(n, 1)
        got = got_bits(oracle.exact_max(as_rank_arrays(bits, width), dtype), width)
        assert got == [expect], (dtype, [hex(c) for c in col])


def bounded_values(rng, n, count):
    """fp32 values with exponents in [-12, 4): any sum of up to 9 of them is
    exact in binary64 (24 + 16 + 4 bits < 53)."""
    m = rng.integers(-(1 << 23), 1 << 23, size=(n, count)).astype(np.float64)
    e = rng.integers(-12 - 23, 4 - 23, size=(n, count))
    return (m * np.exp2(e)).astype(np.float32)


@pytest.mark.parametrize("n", [1, 2, 5, 9])
def test_fp64_sum_is_exact_sum_float32(n):
    rng = np.random.Generator(np.random.PCG64(77 + n))
    xs = list(bounded_values(rng, n, 200))
    want = [math.fsum(f32_of(int(x[i].view(np.uint32))) for x in xs) for i in range(200)]
    assert oracle.fp64_sum(xs, "float32").tolist() == want


@pytest.mark.parametrize("n", [1, 2, 5, 9])
def test_fp64_sum_is_exact_sum_bfloat16(n):
    rng = np.random.Generator(np.random.PCG64(88 + n))
    f = bounded_values(rng, n, 200)
    xs = [(x.view(np.uint32) >> np.uint32(16)).astype(np.uint16) for x in f]
    want = [math.fsum(bf16_of(int(x[i])) for x in xs) for i in range(200)]
    assert oracle.fp64_sum(xs, "bfloat16").tolist() == want
    # a column binary32 cannot hold: 1 + 2^-30 + 2^-30 (bf16 0x3F80, 0x3080)
    col = [np.array([0x3F80], np.uint16), np.array([0x3080], np.uint16),
           np.array([0x3080], np.uint16)]
    assert oracle.fp64_sum(col, "bfloat16").tolist() == [1.0 + 2.0 ** -29]


# ---------------------------------------------------------------- planted mistakes

def _max_pins_hold():
    try:
        for dtype in ("float32", "bfloat16"):
            test_exact_max_float_edge_cases(dtype)
            for n in (2, 5):
                test_exact_max_float_bruteforce(n, dtype)
    except AssertionError:
        return False
    return True


def _sum_pins_hold():
    try:
        for n in (2, 5):
            test_fp64_sum_is_exact_sum_float32(n)
            test_fp64_sum_is_exact_sum_bfloat16(n)
    except AssertionError:
        return False
    return True


def test_planted_max_mistakes_are_caught(monkeypatch):
    assert _max_pins_hold()
    real_max, real_stack, real_widen = direct.ieee_maximum_f32, direct._stack, direct.bf16_to_f32
    # 1. NaN ignored instead of propagated
    monkeypatch.setattr(direct, "ieee_maximum_f32", np.fmax)
    assert not _max_pins_hold()
    # 2. numpy's maximum: NaN payloads kept, -0 and +0 treated as equal
    monkeypatch.setattr(direct, "ieee_maximum_f32", np.maximum)
    assert not _max_pins_hold()
    monkeypatch.setattr(direct, "ieee_maximum_f32", real_max)
    # 3. one rank left out of the reduction
    monkeypatch.setattr(direct, "_stack", lambda xs, d: real_stack(xs, d)[:-1]
                        if len(xs) > 1 else real_stack(xs, d))
    assert not _max_pins_hold()
    monkeypatch.setattr(direct, "_stack", real_stack)
    # 4. bf16 widened by value (the integer pattern as a number), not by bits
    monkeypatch.setattr(direct, "bf16_to_f32", lambda a: np.asarray(a).astype(np.float32))
    assert not _max_pins_hold()
    monkeypatch.setattr(direct, "bf16_to_f32", real_widen)
    assert _max_pins_hold()


def test_planted_sum_mistakes_are_caught(monkeypatch):
    assert _sum_pins_hold()
    real_stack, real_widen = direct._stack, direct.bf16_to_f32
    # 1. a rank left out
    monkeypatch.setattr(direct, "_stack", lambda xs, d: real_stack(xs, d)[1:])
    assert not _sum_pins_hold()
    monkeypatch.setattr(direct, "_stack", real_stack)
    # 2. bf16 widened by value
    monkeypatch.setattr(direct, "bf16_to_f32", lambda a: np.asarray(a).astype(np.float32))
    assert not _sum_pins_hold()
    # 3. a binary32 accumulator
    monkeypatch.setattr(direct, "bf16_to_f32", real_widen)
    real_fp64 = direct.fp64_sum
    monkeypatch.setattr(oracle, "fp64_sum",
                        lambda xs, d: real_fp64(xs, d).astype(np.float32).astype(np.float64))
    assert not _sum_pins_hold()
    monkeypatch.setattr(oracle, "fp64_sum", real_fp64)
    assert _sum_pins_hold()
