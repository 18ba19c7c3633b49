"""Exact rational re-derivations used to pin the oracle (pure Python, tiny inputs).

These are written from the definitions with fractions.Fraction, never with
floating point, so a mistake in the oracle's fp64 implementation (a wrong
tie rule, a dropped term, a transposed operand) shows up as a mismatch.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def f32_exact(x) -> Fraction:
    return Fraction(float(np.float32(x)))


def round_to_f32(fr: Fraction) -> Fraction:
    """Nearest fp32 value to an exact rational (ties to even), with subnormals."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e_ulp = max(e, -126) - 23
    ulp = Fraction(2) ** e_ulp
    q = round(a / ulp)          # Fraction.__round__ is round-half-even
    return sign * q * ulp


def quant_group_int4_exact(v):
    """(codes, scale) of one symmetric INT4 group, exactly."""
    vals = [f32_exact(x) for x in v]
    a = max(abs(x) for x in vals)
    if a == 0:
        return [0] * len(vals), Fraction(0)
    scale = round_to_f32(a / 7)
    if scale < Fraction(2) ** -126 and scale * 7 < a:
        scale += Fraction(2) ** -149          # subnormal range rounds upward
    codes = []
    for x in vals:
        q = round(x / scale)     # half-even on the exact quotient
        codes.append(max(-7, min(7, q)))
    return codes, scale


E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def quant_block_mxfp4_exact(v):
    """(codes, e8m0) of one MXFP4 block, exactly (OCP MX v1.0 conversion)."""
    vals = [f32_exact(x) for x in v]
    a = max(abs(x) for x in vals)
    if a == 0:
        X = -127
    else:
        X = a.numerator.bit_length() - a.denominator.bit_length()
        if Fraction(2) ** X > a:
            X -= 1
        while Fraction(2) ** (X + 1) <= a:
            X += 1
        X -= 2
    X = max(-127, min(127, X))
    codes = []
    for x, raw in zip(vals, v):
        t = abs(x) / Fraction(2) ** X
        if t >= 6:
            idx = 7
        else:
            best = None
            for i, g in enumerate(E2M1):
                d = abs(t - g)
                if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
                    best = (d, i)
            idx = best[1]
        sign = 1 if np.signbit(np.float32(raw)) else 0
        codes.append((sign << 3) | idx)
    return codes, X + 127


def int4_code(nib: int) -> int:
    """Sign-magnitude nibble -> integer."""
    return -(nib & 7) if nib & 8 else nib & 7
