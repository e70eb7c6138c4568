"""Exact rational arithmetic on float inputs (oracle helper).

Every bf16 or fp32 value is a dyadic rational, so dot products of such
vectors are exact in Python's unbounded integers.  The oracle uses these only
where a float64 evaluation cannot certify a decision.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np


def _mant_exp(a):
    a = np.asarray(a, dtype=np.float64).ravel()
    m, e = np.frexp(a)                      # a = m * 2**e, 0.5 <= |m| < 1
    mi = (m * 2.0 ** 53).astype(np.int64)   # exact: 53-bit integer mantissa
    return mi, e.astype(np.int64) - 53


def exact_dot(x, y) -> Fraction:
    """Exact value of sum_i x_i * y_i for finite float inputs."""
    mx, ex = _mant_exp(x)
    my, ey = _mant_exp(y)
    e = ex + ey
    if e.size == 0:
        return Fraction(0)
    emin = int(e.min())
    total = 0
    for a, b, s in zip(mx.tolist(), my.tolist(), (e - emin).tolist()):
        if a and b:
            total += (a * b) << s
    return Fraction(total) * (Fraction(2) ** emin)


def exact_sqnorm(x) -> Fraction:
    return exact_dot(x, x)


def _sign(v) -> int:
    return (v > 0) - (v < 0)


def cos_compare(d1: Fraction, nn1: Fraction, d2: Fraction, nn2: Fraction) -> int:
    """Sign of cos1 - cos2 where cos = d / sqrt(nn) and cos = 0 when nn == 0.

    d is an exact dot product a.b and nn the exact product |a|^2 |b|^2.
    """
    if nn1 == 0:
        d1 = Fraction(0)
    if nn2 == 0:
        d2 = Fraction(0)
    s1, s2 = _sign(d1), _sign(d2)
    if s1 != s2:
        return _sign(s1 - s2)
    if s1 == 0:
        return 0
    c = _sign(d1 * d1 * nn2 - d2 * d2 * nn1)
    return c if s1 > 0 else -c


def cos_at_least(d: Fraction, nn: Fraction, tau: Fraction) -> bool:
    """Exact test of d / sqrt(nn) >= tau (cos taken as 0 when nn == 0)."""
    if nn == 0:
        return tau <= 0
    if d >= 0 and tau <= 0:
        return True
    if d < 0 and tau >= 0:
        return False
    if d >= 0:                       # tau > 0
        return d * d >= tau * tau * nn
    return d * d <= tau * tau * nn   # d < 0, tau < 0: |cos| <= |tau|
