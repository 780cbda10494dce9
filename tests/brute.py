"""Independent brute-force reduction for tiny inputs, in pure Python.

Used only to pin the C oracle.  It shares no code with the oracle: values are
decoded through numpy / plain bit reinterpretation, 16-bit float results are
rounded by searching the sorted list of every representable value (nearest
wins, ties go to the even bit pattern), f32 steps use numpy's binary32
arithmetic, and i32 steps use Python integers reduced modulo 2^32.

The reduction order is the one in "CANN PTO-ISA TREDUCE instruction
explained" §4.3: start from the root's value, then fold in every other rank
in ascending rank order.
"""

from __future__ import annotations

import bisect
import math
from fractions import Fraction

import numpy as np

INF = float("inf")


class SmallFloat:
    """A 16-bit binary float format, enumerated."""

    def __init__(self, name: str, inf_bits: int, decode):
        self.name = name
        self.inf_bits = inf_bits
        self.decode = decode  # bits -> Python float (exact), or nan / inf
        # Positive finite patterns 0 .. inf_bits-1 are ordered by value; the
        # pattern inf_bits stands for the first value past the largest finite
        # one, 2^(emax+1), whose mantissa bits are zero (even) and which
        # encodes +Inf.
        self.values = [Fraction(decode(b)) for b in range(inf_bits)]
        top = self.values[-1]
        ulp = top - self.values[-2]
        self.values.append(top + ulp)

    def exact(self, bits: int):
        v = self.decode(bits)
        if math.isnan(v) or math.isinf(v):
            return v
        return Fraction(v)

    def is_nan(self, bits: int) -> bool:
        return math.isnan(self.decode(bits))

    def round(self, v, negative_zero: bool = False) -> int:
        """Bits of the nearest representable value to the exact value v."""
        if isinstance(v, float):
            if math.isnan(v):
                return self.inf_bits | 0x0200 if self.name == "f16" else self.inf_bits | 0x40
            return self.inf_bits | (0x8000 if v < 0 else 0)
        sign = 0x8000 if (v < 0 or (v == 0 and negative_zero)) else 0
        a = abs(v)
        if a >= self.values[-1]:
            return self.inf_bits | sign
        i = bisect.bisect_right(self.values, a) - 1
        lo, hi = self.values[i], self.values[i + 1]
        if a == lo:
            return i | sign
        dlo, dhi = a - lo, hi - a
        if dlo < dhi:
            pick = i
        elif dhi < dlo:
            pick = i + 1
        else:
            pick = i if i % 2 == 0 else i + 1
        return pick | sign


def _dec_f16(b: int) -> float:
    return float(np.array([b], dtype=np.uint16).view(np.float16)[0])


def _dec_bf16(b: int) -> float:
    return float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])


_FORMATS = {}


def fmt(name: str) -> SmallFloat:
    if name not in _FORMATS:
        if name == "f16":
            _FORMATS[name] = SmallFloat("f16", 0x7C00, _dec_f16)
        else:
            _FORMATS[name] = SmallFloat("bf16", 0x7F80, _dec_bf16)
    return _FORMATS[name]


def _value(dtype: str, bits: int) -> float:
    if dtype == "f32":
        return float(np.array([bits], dtype=np.uint32).view(np.float32)[0])
    return fmt(dtype).decode(bits)


def _extremum(dtype: str, op: str, a: int, b: int) -> int:
    """Max / Min: any NaN gives NaN; otherwise totalOrder with -0 below +0."""
    x, y = _value(dtype, a), _value(dtype, b)
    if math.isnan(x) or math.isnan(y):
        return -1  # marker: NaN (compared by NaN-ness only)
    if x == y:
        # equal values differ only as -0 / +0
        xneg = math.copysign(1.0, x) < 0
        yneg = math.copysign(1.0, y) < 0
        if op == "max":
            return b if (xneg and not yneg) else a
        return b if (yneg and not xneg) else a
    if op == "max":
        return a if x > y else b
    return a if x < y else b


def _arith_small(dtype: str, op: str, a: int, b: int) -> int:
    f = fmt(dtype)
    x, y = f.exact(a), f.exact(b)
    xf, yf = f.decode(a), f.decode(b)  # floats keep the sign of zero
    if math.isnan(xf) or math.isnan(yf):
        return -1
    if op == "sum":
        if math.isinf(xf) or math.isinf(yf):
            s = xf + yf
            return -1 if math.isnan(s) else f.round(s)
        exact = x + y
        # exact zero: -0 only when both addends are -0 (round to nearest)
        both_neg_zero = (xf == 0 and yf == 0 and math.copysign(1, xf) < 0
                         and math.copysign(1, yf) < 0)
        return f.round(exact, negative_zero=both_neg_zero)
    # prod
    if math.isinf(xf) or math.isinf(yf):
        p = xf * yf
        return -1 if math.isnan(p) else f.round(p)
    neg = (math.copysign(1, xf) < 0) != (math.copysign(1, yf) < 0)
    return f.round(x * y, negative_zero=neg)


def _arith_f32(op: str, a: int, b: int) -> int:
    x = np.array([a], dtype=np.uint32).view(np.float32)
    y = np.array([b], dtype=np.uint32).view(np.float32)
    with np.errstate(all="ignore"):
        r = x + y if op == "sum" else x * y
    if np.isnan(r[0]):
        return -1
    return int(r.view(np.uint32)[0])


def _i32(op: str, a: int, b: int) -> int:
    if op == "sum":
        v = (a + b) & 0xFFFFFFFF
    elif op == "prod":
        v = (a * b) & 0xFFFFFFFF
    elif op == "max":
        return max(a, b)
    else:
        return min(a, b)
    return v - (1 << 32) if v >= (1 << 31) else v


def combine(dtype: str, op: str, a: int, b: int) -> int:
    """One step on element bits (i32: Python int value).  -1 marks a NaN result
    for float types (all-ones is never produced otherwise: it is a NaN pattern)."""
    if a == -1 and dtype != "i32":
        a = 0x7FC00000 if dtype == "f32" else fmt(dtype).inf_bits | 0x40
    if b == -1 and dtype != "i32":
        b = 0x7FC00000 if dtype == "f32" else fmt(dtype).inf_bits | 0x40
    if dtype == "i32":
        return _i32(op, a, b)
    if op in ("max", "min"):
        return _extremum(dtype, op, a, b)
    if dtype == "f32":
        return _arith_f32(op, a, b)
    return _arith_small(dtype, op, a, b)


def treduce(srcs, root, dtype, op, ld, valid_rows, valid_cols):
    """dict (i, j) -> result bits (-1 = NaN for float types) over the valid region.

    ``srcs`` are lists of element bits (unsigned for float types, signed
    values for i32) indexed by i*ld + j.
    """
    out = {}
    n = len(srcs)
    for i in range(valid_rows):
        for j in range(valid_cols):
            k = i * ld + j
            acc = srcs[root][k]
            for r in range(n):
                if r != root:
                    acc = combine(dtype, op, acc, srcs[r][k])
            out[(i, j)] = acc
    return out
