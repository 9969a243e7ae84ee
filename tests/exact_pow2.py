"""The exact power of two 2^x, for a double x, rounded once to binary32, from
a 60-digit decimal power and exact rational comparisons: an arbiter that
shares nothing with the oracle's or the GPU path's own evaluation (both
check their 1Q grid levels against it)."""
import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np

RN32_OVERFLOW = Fraction(2) ** 128 - Fraction(2) ** 103   # RN32 of this and above is +inf


def pow2_fraction(x):
    """2^x as an exact fraction of a 60-digit decimal power (relative error
    below 1e-58)."""
    with localcontext() as c:
        c.prec = 60
        return Fraction(Decimal(2) ** Decimal(x))


def rn32_pow2(x):
    """(RN32(2^x), the power's relative distance to the nearest binary32
    midpoint); raises if 60 digits cannot decide."""
    if math.isnan(x):
        return np.float32(np.nan), 1.0
    if x >= 128:   # 2^x >= 2^128, beyond the threshold
        return np.float32(np.inf), 1.0
    if x <= -150:  # 2^x <= 2^-150, the midpoint between 0 and 2^-149: even 0
        return np.float32(0.0), 1.0
    if x == math.floor(x):
        return np.float32(2.0 ** x), 1.0
    d = pow2_fraction(x)
    err = d / 10 ** 58
    if abs(d - RN32_OVERFLOW) <= err:
        raise AssertionError(f"2^{x!r} undecided at 60 digits")
    if d > RN32_OVERFLOW:
        return np.float32(np.inf), float(abs(d - RN32_OVERFLOW) / d)
    f = np.float32(float(d))
    with np.errstate(over="ignore"):
        cand = [np.nextafter(f, np.float32(0)), f, np.nextafter(f, np.float32(np.inf))]
    cand = [c for c in cand if np.isfinite(c)]
    dist = sorted((abs(Fraction(float(c)) - d), i) for i, c in enumerate(cand))
    assert dist[1][0] - dist[0][0] > 2 * err, f"2^{x!r} undecided at 60 digits"
    best = cand[dist[0][1]]
    mids = [(Fraction(float(best)) + Fraction(float(c))) / 2 for c in cand if c != best]
    if best == np.finfo(np.float32).max:
        mids.append(RN32_OVERFLOW)
    return best, float(min(abs(d - m) for m in mids) / d)


def grid_x(lo, hi, k, L):
    """The exponent of 1Q level k >= 1 between fp16 log2 endpoints lo and hi."""
    return lo + ((hi - lo) * (k - 1)) / (L - 2)
