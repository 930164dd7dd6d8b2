"""Exact-rational model of IEEE binary32 arithmetic, for brute-force pins.

Every value is a ``fractions.Fraction``; ``rn32`` rounds an exact rational to
the nearest binary32 value with ties to even, straight from the format's
definition (24-bit significand, exponent range [-126, 127], subnormal step
2^-149).  Nothing here calls the C oracle or uses hardware float arithmetic,
so agreement with the oracle checks the oracle's operations, their order and
their rounding independently of the machine that runs it.
"""
from __future__ import annotations

from fractions import Fraction
import math

import numpy as np

_EMIN = -126
_P = 24


def _floor_log2(q: Fraction) -> int:
    """floor(log2(q)) for q > 0, exactly."""
    n, d = q.numerator, q.denominator
    e = n.bit_length() - d.bit_length()
    # now 2^(e-1) < n/d < 2^(e+1); fix up
    if Fraction(n, d) < Fraction(2) ** e:
        e -= 1
    return e


def round_half_even(q: Fraction) -> int:
    f = math.floor(q)
    r = q - f
    if r > Fraction(1, 2):
        return f + 1
    if r < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def rn32(q: Fraction) -> Fraction:
    if q == 0:
        return Fraction(0)
    s = -1 if q < 0 else 1
    a = -q if q < 0 else q
    e = max(_floor_log2(a), _EMIN)
    ulp = Fraction(2) ** (e - (_P - 1))
    n = round_half_even(a / ulp)
    v = n * ulp
    if v >= Fraction(2) ** 128:
        raise OverflowError("binary32 overflow")
    return s * v


def f32(v) -> Fraction:
    """Exact value of a float32 (or of the float32 nearest to a Python float literal)."""
    return Fraction(float(np.float32(v)))


def to_np32(q: Fraction) -> np.float32:
    return np.float32(float(q))  # exact: q is a binary32 value


F1 = f32(7.49)
F2 = f32(14.98)


def decompose_group(a_vals, ):
    """Steps 1-8 of the MSD expansion for one group, exact-rational model.
    a_vals: iterable of exact values (fp16 inputs).  Returns (A1, A2, A3, amax)."""
    a_vals = [Fraction(v) for v in a_vals]
    amax = max(abs(v) for v in a_vals)
    A1, A2, A3 = [], [], []
    for a in a_vals:
        if amax == 0:
            A1.append(0); A2.append(0); A3.append(0)
            continue
        t1 = rn32(rn32(F1 * a) / amax)
        l1 = round_half_even(t1)
        t2 = rn32(rn32(t1 - l1) * F2)
        l2 = round_half_even(t2)
        t3 = rn32(rn32(t2 - l2) * F2)
        l3 = round_half_even(t3)
        A1.append(l1); A2.append(l2); A3.append(l3)
    return A1, A2, A3, amax


def tie_levels(a: Fraction, amax: Fraction):
    """The three pre-rounding values (t1, t2, t3) of one element."""
    t1 = rn32(rn32(F1 * a) / amax)
    t2 = rn32(rn32(t1 - round_half_even(t1)) * F2)
    t3 = rn32(rn32(t2 - round_half_even(t2)) * F2)
    return t1, t2, t3
