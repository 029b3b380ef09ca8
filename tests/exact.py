"""Exact-rational IEEE 754 binary32 arithmetic for pinning the oracle on tiny inputs.

Each fused multiply-add and each add is evaluated exactly with ``fractions.Fraction`` and rounded once to binary32
with round-to-nearest-ties-to-even, keeping subnormals and overflowing to infinity, with IEEE 754's rules for signed
zeros, infinities and NaN. Nothing here calls the C library's fmaf or the oracle: it is an independent
implementation of the standard, slow and only for small inputs.
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction

EMIN = -126            # smallest normal exponent
MANT = 23              # fraction bits
MIN_SUB_EXP = EMIN - MANT   # 2**-149, the subnormal quantum
OVERFLOW = Fraction(2) ** 128


def bits(f: float) -> int:
    """binary32 bit pattern of a Python float that is exactly representable in binary32."""
    return struct.unpack("<I", struct.pack("<f", f))[0]


def from_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def _neg_zero(f: float) -> bool:
    return f == 0.0 and math.copysign(1.0, f) < 0


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2**e may be off by one either way: adjust.
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_rational(q: Fraction) -> float:
    """Round a nonzero exact rational to binary32, ties to even, subnormals kept, overflow to +-inf."""
    if q == 0:
        raise ValueError("zero has a sign decided by the operation, not by rounding")
    sign = -1.0 if q < 0 else 1.0
    a = -q if q < 0 else q
    e = _floor_log2(a)
    qexp = MIN_SUB_EXP if e < EMIN else e - MANT      # exponent of the last significand bit
    quantum = Fraction(2) ** qexp
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= OVERFLOW:
        return sign * math.inf
    if r == 0:                        # a tiny value rounded to zero keeps its sign
        return math.copysign(0.0, sign)
    return sign * float(r)            # exactly representable in binary32, hence in binary64


def fma(a: float, b: float, c: float) -> float:
    """binary32 fused multiply-add a*b + c with one rounding (IEEE 754-2019, 5.4.1 and 6)."""
    if math.isnan(a) or math.isnan(b) or math.isnan(c):
        return math.nan
    a_inf, b_inf, c_inf = math.isinf(a), math.isinf(b), math.isinf(c)
    if (a_inf and b == 0) or (b_inf and a == 0):
        return math.nan                                   # invalid: 0 * inf
    if a_inf or b_inf:
        psign = math.copysign(1.0, a) * math.copysign(1.0, b)
        if c_inf and math.copysign(1.0, c) != psign:
            return math.nan                               # inf - inf
        return psign * math.inf
    if c_inf:
        return c
    exact = Fraction(a) * Fraction(b) + Fraction(c)
    if exact == 0:
        prod_zero = (a == 0 or b == 0)
        if prod_zero and c == 0:
            prod_neg = (math.copysign(1.0, a) * math.copysign(1.0, b)) < 0
            return -0.0 if (prod_neg and _neg_zero(c)) else 0.0
        return 0.0                                        # exact cancellation: +0 under round-to-nearest
    return round_rational(exact)


def add(a: float, b: float) -> float:
    """binary32 addition with one rounding."""
    if math.isnan(a) or math.isnan(b):
        return math.nan
    if math.isinf(a) and math.isinf(b):
        return a if math.copysign(1.0, a) == math.copysign(1.0, b) else math.nan
    if math.isinf(a):
        return a
    if math.isinf(b):
        return b
    exact = Fraction(a) + Fraction(b)
    if exact == 0:
        if a == 0 and b == 0:
            return -0.0 if (_neg_zero(a) and _neg_zero(b)) else 0.0
        return 0.0
    return round_rational(exact)


def step(d_u, x, d_dv, ti: int, P: int, hd: int):
    """The chained update of step ti on nested Python lists of floats (d_u and d_dv indexed [n][row][col], x
    [n][j][i]); returns a new d_u."""
    out = [[list(row) for row in chunk] for chunk in d_u]
    C = len(x[0])
    for p in range(P):
        n = ti * P + p
        for i in range(C):
            for c in range(hd):
                acc = 0.0
                for j in range(C):
                    acc = fma(x[n][j][i], d_dv[n][j][c], acc)
                out[n][i][c] = add(d_u[n][i][c], acc)
    return out


def mul(a: float, b: float) -> float:
    """binary32 multiplication with one rounding: a*b + (-0) is a*b exactly for every a, b (a +0 product stays +0, a
    -0 product stays -0), so one fused rounding of it is the rounded product."""
    return fma(a, b, -0.0)
