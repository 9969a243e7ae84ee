"""Input sets for pinning codecs: every rounding boundary of a lane and its
neighbourhood, plus seeded random FP32 bit patterns and special values.

Pure input construction (no codec arithmetic): boundaries are taken from a
table of lane values handed in by the caller.
"""
import numpy as np


def f32_neighbours(x64, k=2):
    """float32 values within k steps of each float64 value (rounded to f32 first)."""
    x = np.asarray(x64, np.float64).astype(np.float32)
    out = [x]
    lo, hi = x.copy(), x.copy()
    for _ in range(k):
        lo = np.nextafter(lo, np.float32(-np.inf))
        hi = np.nextafter(hi, np.float32(np.inf))
        out += [lo, hi]
    return np.concatenate(out)


def boundary_set(values):
    """Ascending non-negative lane values -> float32 inputs at and around every
    value and every midpoint between neighbours, both signs."""
    v = np.asarray(values, np.float64)
    mids = 0.5 * (v[:-1] + v[1:])
    pos = np.concatenate([f32_neighbours(v), f32_neighbours(mids)])
    return np.concatenate([pos, -pos])


def random_patterns(n, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    return r.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32).view(np.float32)


def specials():
    f = np.float32
    vals = [0.0, -0.0, np.inf, -np.inf, np.nan, -np.nan,
            np.finfo(np.float32).max, -np.finfo(np.float32).max,
            np.finfo(np.float32).tiny, -np.finfo(np.float32).tiny,
            1.0, -1.0, 2.0, -2.0, 65504.0, 65520.0, 65519.996, 1e30, -1e30]
    den = np.array([1, 2, 3, 0x7FFFFF, 0x400000], np.uint32).view(np.float32)
    return np.concatenate([np.array(vals, f), den, -den])
