"""Exact rational-arithmetic mini-oracle for tiny cases -- TEST INFRASTRUCTURE ONLY.

Independent of ``vbq_oracle.c``: it decodes IEEE binary16 / bfloat16 bit
patterns into ``fractions.Fraction`` from the format definition and forms the
dequantised product exactly, so the C oracle's fp64 results can be checked
against the exact value. Follows the same passages as ``vbq_oracle.c``
(VBQ abstract: the fused kernel must match the plain dequantised product; CellFill
abstract: dequantised weight plus an in-cell residual).
"""
from __future__ import annotations

from fractions import Fraction


def f16_value(h: int) -> Fraction:
    """Exact value of an IEEE binary16 bit pattern (finite values only)."""
    h = int(h) & 0xFFFF
    sign = -1 if h >> 15 else 1
    e = (h >> 10) & 0x1F
    m = h & 0x3FF
    if e == 0x1F:
        raise ValueError("inf/nan")
    if e == 0:
        v = Fraction(m, 1 << 24)
    else:
        v = Fraction(1024 + m) * (Fraction(2) ** (e - 25))
    return sign * v


def bf16_value(h: int) -> Fraction:
    """Exact value of a bfloat16 bit pattern (finite values only):
    1 sign bit, 8 exponent bits (bias 127), 7 fraction bits."""
    h = int(h) & 0xFFFF
    sign = -1 if h >> 15 else 1
    e = (h >> 7) & 0xFF
    m = h & 0x7F
    if e == 0xFF:
        raise ValueError("inf/nan")
    if e == 0:
        v = Fraction(m) * (Fraction(2) ** -133)
    else:
        v = Fraction(128 + m) * (Fraction(2) ** (e - 134))
    return sign * v


def dequant_exact(q, s16, o16, resid16=None):
    """Wdq[n][k] = s*q + o (+ r), exact. q: [N][K] ints, s16/o16: [N][G]."""
    N, K = len(q), len(q[0])
    out = []
    for n in range(N):
        row = []
        for k in range(K):
            g = k // 64
            w = f16_value(s16[n][g]) * int(q[n][k]) + f16_value(o16[n][g])
            if resid16 is not None:
                w += f16_value(resid16[n][k])
            row.append(w)
        out.append(row)
    return out


def gemv_exact(q, s16, o16, x, resid16=None, bf16=False):
    """y[b][n] = sum_k x[b][k] * Wdq[n][k], exact rationals."""
    dec = bf16_value if bf16 else f16_value
    W = dequant_exact(q, s16, o16, resid16)
    xs = [[dec(v) for v in row] for row in x]
    return [[sum((xb[k] * W[n][k] for k in range(len(xb))), Fraction(0)) for n in range(len(W))]
            for xb in xs]


def nearest_levels(w: Fraction, s: Fraction, o: Fraction, L: int):
    """All q in [0, L] minimising |w - (s*q + o)| (brute force; >1 entry = tie)."""
    best, arg = None, []
    for q in range(L + 1):
        d = abs(w - (s * q + o))
        if best is None or d < best:
            best, arg = d, [q]
        elif d == best:
            arg.append(q)
    return arg
