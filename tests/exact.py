"""Exact-arithmetic helpers for pinning the oracle (independent of its code).

Rounding to fp32 is done here on ``fractions.Fraction`` with integer arithmetic,
never through a double, so it cannot share a double-rounding mistake with the
oracle's ``(float)(double)`` conversion.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name: str) -> list[list[str]]:
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def f32_from_bits(bits: int) -> float:
    return float(np.array([bits], np.uint32).view(np.float32)[0])


def bits_of_f32(v) -> int:
    return int(np.array([v], np.float32).view(np.uint32)[0])


def round_f32(q: Fraction, negative_zero: bool = False) -> float:
    """Round an exact rational to the nearest fp32 (ties to even) -> float.
    Overflow gives +-inf.  A zero result keeps the sign given."""
    if q == 0:
        return -0.0 if negative_zero else 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                       # subnormal range shares quantum 2^-149
    quantum = Fraction(2) ** (e - 23)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(r)   # r is an fp32 value, so the float conversion is exact


def e2m1_exact(code: int) -> Fraction:
    """From the golden OCP value list."""
    for c, v in read_golden("e2m1_ocp_values.txt"):
        if int(c, 16) == code:
            return Fraction(v.replace("-", "")) * (-1 if v.startswith("-") else 1)
    raise KeyError(code)
