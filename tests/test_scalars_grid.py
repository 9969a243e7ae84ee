"""The library's per-call scalars against the oracle's, over the
hyperparameter grid the GPU grid test runs (host only: pa_debug_scalars
does no device work, so this runs without a GPU).

The eight binary32 scalars must match the oracle's bit for bit (both form
them in double and round each once; KBench quantized-optimizer-state
reference, `quantized_adamw_step`, where the bias corrections are Python
floats).  The two extra values the kernels take are checked against what
they stand for: beta1 * 2^112 must be exact, and the double reciprocal of
bc2 must turn v'/bc2 into the correctly rounded quotient, which is checked
against exact rational arithmetic on sampled v'.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle

BETA1 = [0.0, 1e-30, 0.5, 0.9, 0.999999]
BETA2 = [0.0, 0.5, 0.999, 0.99999]
LR = [0.0, 1e-3, 3.0]
WD = [0.0, 0.01, 0.3]
EPS = [0.0, 1e-8, 1e-2]
STEPS = [1, 2, 1000, 10 ** 7, 2 ** 40]


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    if not __import__("os").path.exists(pa_mod.LIB_PATH):
        pytest.skip("libpa.so is not built")
    pa_mod.lib()
    return pa_mod


def _rn32(fr):
    """Round an exact rational to binary32, to nearest even (normal range)."""
    x = float(fr)                       # correctly rounded to double
    f = np.float32(x)                   # double -> float32, to nearest even
    # double rounding is harmless unless the double lands on a binary32
    # midpoint; settle that case exactly
    lo, hi = np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))
    for cand in (lo, hi):
        mid = (Fraction(float(f)) + Fraction(float(cand))) / 2
        if fr == mid:
            even = f if (int(np.float32(f).view(np.uint32)) & 1) == 0 else cand
            return np.float32(even)
    if abs(Fraction(float(lo)) - fr) < abs(Fraction(float(f)) - fr):
        return lo
    if abs(Fraction(float(hi)) - fr) < abs(Fraction(float(f)) - fr):
        return hi
    return f


def test_scalars_match_oracle_on_grid(pa):
    n = 0
    for b1, b2, lr, wd, eps, t in itertools.product(BETA1, BETA2, LR, WD, EPS, STEPS):
        h = dict(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
        got, inv = pa.pa_debug_scalars(h, t)
        want = oracle.scalars(lr, b1, b2, eps, wd, t)
        assert np.array_equal(got[:8].view(np.uint32), want.view(np.uint32)), (h, t, got[:8], want)
        assert float(got[8]) == float(np.ldexp(np.float64(got[0]), 112)), (h, t)
        assert inv == 1.0 / float(got[4]), (h, t)
        n += 1
    assert n == 5 * 4 * 3 * 3 * 3 * 5


def test_quotient_by_bc2_is_correctly_rounded(pa):
    """v'/bc2 through the double reciprocal equals the exact quotient rounded
    once to binary32, for every bc2 of the grid and v' spread over the
    normal range (wide exponents, all mantissa patterns sampled)."""
    r = np.random.Generator(np.random.PCG64(2024))
    v = np.concatenate([
        (r.random(4000) * 2.0 ** r.integers(-120, 120, 4000)).astype(np.float32),
        np.float32(1.0) + np.arange(64, dtype=np.float32) * np.float32(2.0 ** -23),
    ])
    v = v[(v > 0) & np.isfinite(v)]
    for b2, t in itertools.product(BETA2, STEPS):
        _, inv = pa.pa_debug_scalars(dict(lr=1e-3, beta1=0.9, beta2=b2, eps=1e-8, weight_decay=0.0), t)
        bc2 = oracle.scalars(1e-3, 0.9, b2, 1e-8, 0.0, t)[4]
        with np.errstate(over="ignore"):
            fast = (v.astype(np.float64) * inv).astype(np.float32)
        for x, y in zip(v[:600], fast[:600]):
            q = Fraction(float(x)) / Fraction(float(bc2))
            if q > Fraction(2.0 ** 127) or q < Fraction(2.0 ** -126):
                continue
            assert y == _rn32(q), (b2, t, x, bc2, y)


def test_debug_scalars_rejects_what_the_step_rejects(pa):
    bad = [dict(lr=1e-3, beta1=1.0, beta2=0.999, eps=1e-8, weight_decay=0.0),
           dict(lr=1e-3, beta1=0.9, beta2=-0.1, eps=1e-8, weight_decay=0.0),
           dict(lr=float("nan"), beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0),
           dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=-1e-8, weight_decay=0.0)]
    for h in bad:
        with pytest.raises(pa.PAError):
            pa.pa_debug_scalars(h, 1)
    with pytest.raises(pa.PAError):
        pa.pa_debug_scalars(dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0), 0)
