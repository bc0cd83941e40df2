"""Per-hop reduction operator and AVG epilogue -- oracle (test infrastructure only).

The pages define AllReduce over an elementwise operator such as sum or max
("AllReduce", compassingai.com, section 3 技术原理; "AllReduce 集合通信",
zzmblog.top, section 语义) and average as the sum divided by the world size
("Allreduce：大模型分布式训练的核心通信算法与优化实践", section 3.1 and the
code in section 3.2; "AllReduce 集合通信", section DDP 梯度同步中的地位).
They leave the arithmetic of one hop open.  Readings used here:

* int32 SUM: two's-complement wrap-around add.
* fp32 SUM: one IEEE-754 binary32 add, round-to-nearest-even, per hop; no
  wider accumulator; subnormals kept.
* bf16 SUM: widen both operands to fp32, add in fp32 (RNE), round the fp32
  sum to bf16 (RNE) -- every hop rounds.
* MAX: IEEE-754-2019 ``maximum``: a NaN operand gives NaN (this oracle returns
  the canonical quiet NaN), +0 is larger than -0.
* AVG: done once, after the full SUM: fp32 correctly rounded division by
  float(N); bf16 round_bf16(fp32(acc) / N).  int32 AVG is not defined.

bf16 values are carried as ``numpy.uint16`` bit patterns.  The fp32 -> bf16
rounding is the integer round-half-to-even rule on the fp32 bit pattern; a NaN
becomes 0x7FC0.
"""

from __future__ import annotations

import numpy as np

DTYPES = ("int32", "float32", "bfloat16")
OPS = ("sum", "max", "avg")

_BF16_QNAN = np.uint16(0x7FC0)
_F32_QNAN_BITS = np.uint32(0x7FC00000)


def np_dtype_of(dtype: str):
    """numpy storage type for one of DTYPES (bf16 is stored as uint16 bits)."""
    return {"int32": np.int32, "float32": np.float32, "bfloat16": np.uint16}[dtype]


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32 (append 16 zero bits)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(x) -> np.ndarray:
    """Round fp32 to bf16, nearest with ties to even; NaN -> 0x7FC0.

    Adding 0x7FFF plus the lowest kept bit, then dropping 16 bits, rounds up
    exactly when the dropped half is above one half, or equal to one half with
    an odd kept part.  A carry out of the mantissa bumps the exponent, so the
    largest finite values round to infinity as IEEE rounding requires.
    """
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) & np.uint64(0xFFFF)
    out = r.astype(np.uint16)
    isnan = (u & np.uint64(0x7FFFFFFF)) > np.uint64(0x7F800000)
    out[isnan] = _BF16_QNAN
    return out


def ieee_maximum_f32(a, b) -> np.ndarray:
    """IEEE-754-2019 maximum on fp32 arrays (NaN wins; +0 > -0).

    When a == b the two bit patterns are equal except possibly for the sign
    of a zero; AND-ing the bit patterns then gives -0 only if both are -0.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    ua = a.view(np.uint32)
    ub = b.view(np.uint32)
    bigger = np.where(a > b, ua, ub)
    same = np.where(a == b, ua & ub, bigger)
    nan = np.isnan(a) | np.isnan(b)
    res = np.where(nan, _F32_QNAN_BITS, same).astype(np.uint32)
    return res.view(np.float32)


def hop(acc, incoming, dtype: str, op: str) -> np.ndarray:
    """One ring hop: combine a received chunk with the local one.

    ``op`` is the reduction (``avg`` hops are ``sum`` hops; the division
    happens once at the end).  Arrays keep their storage dtype.
    """
    if op not in OPS:
        raise ValueError(op)
    red = "sum" if op == "avg" else op
    if dtype == "int32":
        if op == "avg":
            raise ValueError("int32 AVG is not defined")
        a = np.asarray(acc, dtype=np.int32)
        b = np.asarray(incoming, dtype=np.int32)
        if red == "sum":
            # wrap-around: do the add in int64, keep the low 32 bits
            s = a.astype(np.int64) + b.astype(np.int64)
            return s.astype(np.uint64).astype(np.uint32).view(np.int32)
        return np.maximum(a, b)
    if dtype == "float32":
        a = np.asarray(acc, dtype=np.float32)
        b = np.asarray(incoming, dtype=np.float32)
        if red == "sum":
            return np.add(a, b, dtype=np.float32)
        return ieee_maximum_f32(a, b)
    if dtype == "bfloat16":
        fa = bf16_to_f32(acc)
        fb = bf16_to_f32(incoming)
        if red == "sum":
            return f32_to_bf16_rne(np.add(fa, fb, dtype=np.float32))
        # the maximum of two bf16 values is one of them: exact
        return f32_to_bf16_rne(ieee_maximum_f32(fa, fb))
    raise ValueError(dtype)


def avg_epilogue(acc, nranks: int, dtype: str) -> np.ndarray:
    """Divide a finished SUM by the number of ranks (AVG)."""
    if dtype == "float32":
        return np.divide(np.asarray(acc, dtype=np.float32), np.float32(nranks),
                         dtype=np.float32)
    if dtype == "bfloat16":
        q = np.divide(bf16_to_f32(acc), np.float32(nranks), dtype=np.float32)
        return f32_to_bf16_rne(q)
    raise ValueError("AVG is defined for float32 and bfloat16 only")
