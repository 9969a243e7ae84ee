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


def near_midpoint_exponents(seed, n_near_one=6000, n_wide=2000):
    """Doubles x whose power 2^x lies very close to a binary32 midpoint:
    x = log2(m), rounded to double, for seeded random midpoints m between
    adjacent binary32 values.  Most m have exponents in [-6, 5], where |x|
    is small and its double is fine enough that 2^x often falls within
    2^-56 of m; the rest span every binade, the subnormal ones included.
    Input construction only (numpy's long-double log2 picks x)."""
    r = np.random.default_rng(seed)
    e = r.integers(-6, 6, n_near_one)
    mant = r.integers(0, 1 << 23, n_near_one)
    near = ((e + 127).astype(np.uint32) << 23) | mant.astype(np.uint32)
    wide = r.integers(1, 0x7F7FFFFF, n_wide, dtype=np.int64).astype(np.uint32)
    a = np.concatenate([near, wide]).view(np.float32)
    b = np.nextafter(a, np.float32(np.inf))
    m = (a.astype(np.longdouble) + b.astype(np.longdouble)) / 2
    return np.log2(m).astype(np.float64)
