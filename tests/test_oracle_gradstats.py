"""Pins of the oracle's gradient pre-pass (sum of squares, non-finite count,
clip coefficient, gradient scaling) against what mathematics fixes: Python's
correctly rounded math.fsum, closed forms, exact ties, the extremes of
binary32, and numpy's own binary32 arithmetic and 16-bit widening."""
import math

import numpy as np
import pytest

import oracle


def _fsum_sq(x):
    # binary32 squares are exact in double (48-bit significands); fsum rounds
    # the exact sum once.
    return math.fsum(float(v) * float(v) for v in np.asarray(x, np.float32))


def _mixed(rng, n):
    mag = 10.0 ** rng.uniform(-44, 38, n)
    x = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    x[rng.random(n) < 0.05] = 0.0
    return x


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sumsq_equals_fsum(oracle_mod, seed):
    rng = np.random.default_rng(seed)
    g = _mixed(rng, 5000)
    s, bad, _ = oracle.grad_stats(oracle.DT_F32, [g])
    assert bad == 0
    assert s == _fsum_sq(g)


def test_sumsq_ordinary_gradients_and_lists(oracle_mod):
    rng = np.random.default_rng(7)
    parts = [(rng.standard_normal(n) * 10.0 ** rng.uniform(-6, -1)).astype(np.float32) for n in (1, 17, 4096, 9999)]
    s, bad, _ = oracle.grad_stats(oracle.DT_F32, parts)
    assert bad == 0
    assert s == _fsum_sq(np.concatenate(parts))


def test_sumsq_closed_form(oracle_mod):
    n = 100000
    g = np.arange(1, n + 1, dtype=np.float32)          # exact integers below 2^24
    s, _, _ = oracle.grad_stats(oracle.DT_F32, [g])
    assert s == n * (n + 1) * (2 * n + 1) // 6        # below 2^53: exact in double


def test_sumsq_round_to_nearest_even(oracle_mod):
    big = np.float32(2.0 ** 26)                         # square 2^52
    one = np.float32(1.0)
    cases = [([big, big, one], 2.0 ** 53),              # 2^53 + 1: tie, even is 2^53
             ([big, big, one, one], 2.0 ** 53 + 2),     # exact
             ([big, big, one, one, one], 2.0 ** 53 + 4)]  # 2^53 + 3: tie, even is 2^53 + 4
    for vals, want in cases:
        s, _, _ = oracle.grad_stats(oracle.DT_F32, [np.array(vals, np.float32)])
        assert s == want
        assert s == _fsum_sq(vals)


def test_sumsq_binary32_extremes(oracle_mod):
    tiny = np.array([2.0 ** -149] * 6, np.float32)
    assert oracle.grad_stats(oracle.DT_F32, [tiny])[0] == 6 * 2.0 ** -298
    huge = np.array([np.finfo(np.float32).max] * 3, np.float32)
    assert oracle.grad_stats(oracle.DT_F32, [huge])[0] == _fsum_sq(huge)
    both = np.concatenate([tiny, huge, np.float32([1.0])])
    assert oracle.grad_stats(oracle.DT_F32, [both])[0] == _fsum_sq(both)
    assert oracle.grad_stats(oracle.DT_F32, [np.zeros(5, np.float32)])[0] == 0.0
    assert oracle.grad_stats(oracle.DT_F32, [np.zeros(0, np.float32)])[:2] == (0.0, 0)


def test_sumsq_order_free(oracle_mod):
    rng = np.random.default_rng(3)
    g = _mixed(rng, 20000)
    a = oracle.grad_stats(oracle.DT_F32, [g])[0]
    b = oracle.grad_stats(oracle.DT_F32, [g[rng.permutation(g.size)]])[0]
    c = oracle.grad_stats(oracle.DT_F32, [g[:7], g[7:12345], g[12345:]])[0]
    assert a == b == c


def test_nonfinite_count_and_value(oracle_mod):
    g = np.array([1.0, np.inf, 2.0, -np.inf], np.float32)
    s, bad, _ = oracle.grad_stats(oracle.DT_F32, [g])
    assert math.isinf(s) and s > 0 and bad == 2
    g2 = np.array([np.nan, 1.0, np.inf, 3.0, np.nan], np.float32)
    s, bad, _ = oracle.grad_stats(oracle.DT_F32, [g2])
    assert math.isnan(s) and bad == 3


def test_16bit_gradients_widen_exactly(oracle_mod):
    rng = np.random.default_rng(11)
    f32 = (rng.standard_normal(3000) * 1e-2).astype(np.float32)
    bf_bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    bf_wide = (bf_bits.astype(np.uint32) << 16).view(np.float32)
    assert oracle.grad_stats(oracle.DT_BF16, [bf_bits])[0] == _fsum_sq(bf_wide)
    h = f32.astype(np.float16)
    h[:3] = [np.inf, np.nan, 6e-8]
    s, bad, _ = oracle.grad_stats(oracle.DT_F16, [h.view(np.uint16)])
    assert math.isnan(s) and bad == 2
    s, bad, _ = oracle.grad_stats(oracle.DT_F16, [h[2:].view(np.uint16).copy()])
    assert bad == 0 and s == _fsum_sq(h[2:].astype(np.float32))


def test_clip_coefficient(oracle_mod):
    assert oracle.clip_scale(4.0, 1.0) == np.float32(1.0 / (2.0 + 1e-6))
    assert oracle.clip_scale(4.0, 10.0) == np.float32(1.0)
    assert oracle.clip_scale(0.0, 1.0) == np.float32(1.0)
    assert oracle.clip_scale(math.inf, 1.0) == np.float32(0.0)
    assert math.isnan(oracle.clip_scale(math.nan, 1.0))
    g = np.full(100, 0.5, np.float32)                  # norm 5
    s, _, clip = oracle.grad_stats(oracle.DT_F32, [g], max_norm=1.0)
    assert s == 25.0 and clip == float(np.float32(1.0 / (5.0 + 1e-6)))


def test_scale_grads_is_one_binary32_product(oracle_mod):
    rng = np.random.default_rng(5)
    g = _mixed(rng, 4000)
    for s in (np.float32(0.3), np.float32(1.0), np.float32(2.0 ** -20), np.float32(7.5e-3)):
        out = oracle.scale_grads(oracle.DT_F32, g, s)
        want = g * s                                     # numpy: binary32 product, rounded to nearest
        assert np.array_equal(out.view(np.uint32), want.view(np.uint32))
    bf_bits = (g.view(np.uint32) >> 16).astype(np.uint16)
    out = oracle.scale_grads(oracle.DT_BF16, bf_bits, np.float32(0.25))
    assert np.array_equal(out, (bf_bits.astype(np.uint32) << 16).view(np.float32) * np.float32(0.25))
