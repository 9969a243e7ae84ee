"""Pins of the oracle's lane codecs against things other than the oracle.

Format (Packed AdamW Reference README, introduction; project page, Release
scope): low half of the word a signed finite E4M11 first moment, high half
an unsigned finite E4M12 RMS.  Readings where the pages are silent: bias 15
for both lanes (parity unpinned: the pages never print it), gradual
underflow, no Inf/NaN codes, round to nearest even, finite saturation.

Pins used here:
  * numpy's IEEE binary16: with bias 15, every E4M11 code whose mantissa is
    even, and every E4M12 code whose mantissa is a multiple of four, is a
    binary16 value with the same exponent field;
  * closed forms for the largest finite, smallest normal and smallest
    subnormal values;
  * invariants over all 65,536 codes of each lane: decode->encode identity,
    strict monotonicity, RMS >= 0, sign symmetry, signed zero;
  * an independent rounding rule (scale into the lane's integer grid with
    numpy.rint, ties to even) on every rounding boundary of the lane and its
    neighbours, on whole FP32 binades and on seeded random bit patterns;
  * numpy's float32->float16 cast (binary16 lanes) and torch's
    float32->bfloat16 cast (blockwise parameter output).
"""
import numpy as np
import pytest

from pins import boundary_set, random_patterns, specials

M_MAX = 2.0 - 2.0 ** -11
R_MAX = 2.0 - 2.0 ** -12


def _f16_value(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def test_bias_reading_is_15(oracle_mod):
    assert oracle_mod.e4_bias() == 15


def test_m_lane_closed_forms(oracle_mod):
    d = oracle_mod.decode(0, np.array([0x7FFF, 0x0800, 0x07FF, 0x0001, 0x0000, 0x8000, 0xFFFF],
                                      np.uint16)).astype(np.float64)
    assert d[0] == M_MAX == 1.99951171875
    assert d[1] == 2.0 ** -14
    assert d[2] == 2047 * 2.0 ** -25
    assert d[3] == 2.0 ** -25
    assert d[4] == 0.0 and not np.signbit(d[4])
    assert d[5] == 0.0 and np.signbit(d[5])
    assert d[6] == -M_MAX


def test_r_lane_closed_forms(oracle_mod):
    d = oracle_mod.decode(1, np.array([0xFFFF, 0x1000, 0x0001, 0x0000], np.uint16)).astype(np.float64)
    assert d[0] == R_MAX == 1.999755859375
    assert d[1] == 2.0 ** -14
    assert d[2] == 2.0 ** -26
    assert d[3] == 0.0 and not np.signbit(d[3])


def test_m_lane_decode_against_binary16(oracle_mod):
    codes = np.arange(1 << 16, dtype=np.uint32)
    val = oracle_mod.decode(0, codes.astype(np.uint16)).astype(np.float64)
    sign, e, f = codes >> 15, (codes >> 11) & 0xF, codes & 0x7FF
    even = (f % 2) == 0
    want = _f16_value(((sign << 15) | (e << 10) | (f >> 1))[even])
    np.testing.assert_array_equal(val[even], want)
    # odd mantissas sit exactly halfway between their neighbours
    mag = val[:0x8000]
    odd = np.arange(1, 0x7FFF, 2)
    np.testing.assert_array_equal(mag[odd], 0.5 * (mag[odd - 1] + mag[odd + 1]))
    assert mag[0x7FFF] == M_MAX
    # sign symmetry and strict monotonicity of the magnitudes
    np.testing.assert_array_equal(val[0x8000:], -mag)
    assert np.all(np.diff(mag) > 0)


def test_r_lane_decode_against_binary16(oracle_mod):
    codes = np.arange(1 << 16, dtype=np.uint32)
    val = oracle_mod.decode(1, codes.astype(np.uint16)).astype(np.float64)
    e, f = codes >> 12, codes & 0xFFF
    q = (f % 4) == 0
    np.testing.assert_array_equal(val[q], _f16_value(((e << 10) | (f >> 2))[q]))
    # codes between multiples of four interpolate linearly within the binade
    ext = np.append(val, 2.0)                      # the next power of two closes the top run
    c0 = codes - (f % 4)
    frac = (f % 4) / 4.0
    np.testing.assert_array_equal(val, ext[c0] + frac * (ext[c0 + 4] - ext[c0]))
    assert np.all(val >= 0) and np.all(np.diff(val) > 0)


@pytest.mark.parametrize("lane", [0, 1])
def test_decode_encode_identity_all_codes(oracle_mod, lane):
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    back = oracle_mod.encode(lane, oracle_mod.decode(lane, codes))
    np.testing.assert_array_equal(back, codes)


def _rint_round(a, mbits, max_val):
    """Round non-negative finite float64 a onto a lane with mbits mantissa bits,
    smallest normal 2^-14, to nearest with ties to even, saturating at max_val."""
    a = np.asarray(a, np.float64)
    out = np.empty_like(a)
    sub = a < 2.0 ** -14
    step = 2.0 ** (-14 - mbits)
    out[sub] = np.rint(a[sub] / step) * step
    _, ex = np.frexp(a[~sub])
    e = ex - 1                                     # a in [2^e, 2^(e+1))
    out[~sub] = np.ldexp(np.rint(np.ldexp(a[~sub], mbits - e)), e - mbits)
    return np.minimum(out, max_val)


def _whole_binade(lo_exp):
    """Every float32 in [2^lo_exp, 2^(lo_exp+1))."""
    base = np.uint32((lo_exp + 127) << 23)
    return (base + np.arange(1 << 23, dtype=np.uint32)).view(np.float32)


def _m_inputs(oracle_mod):
    mags = oracle_mod.decode(0, np.arange(0x8000, dtype=np.uint16)).astype(np.float64)
    return np.concatenate([boundary_set(mags), boundary_set([M_MAX, 2.0]), random_patterns(1 << 22, 11),
                           specials(), _whole_binade(-15), -_whole_binade(0), _whole_binade(-26)])


def _r_inputs(oracle_mod):
    vals = oracle_mod.decode(1, np.arange(0x10000, dtype=np.uint16)).astype(np.float64)
    return np.concatenate([boundary_set(vals), boundary_set([R_MAX, 2.0]), random_patterns(1 << 22, 12),
                           specials(), _whole_binade(-15), _whole_binade(0), _whole_binade(-27)])


def test_m_lane_encoder_against_rint(oracle_mod):
    x = _m_inputs(oracle_mod)
    code = oracle_mod.encode(0, x)
    nan = np.isnan(x)
    assert np.all(code[nan] == 0)
    x, code = x[~nan], code[~nan]
    # the sign bit follows the input's sign, zero included
    np.testing.assert_array_equal((code >> 15).astype(bool), np.signbit(x))
    got = oracle_mod.decode(0, code).astype(np.float64)
    a = np.abs(x.astype(np.float64))
    fin = np.isfinite(a)
    want = np.full(a.shape, M_MAX)
    want[fin] = _rint_round(a[fin], 11, M_MAX)
    np.testing.assert_array_equal(np.abs(got), want)


def test_r_lane_encoder_against_rint(oracle_mod):
    x = _r_inputs(oracle_mod)
    code = oracle_mod.encode(1, x)
    zero_class = np.isnan(x) | np.signbit(x)
    assert np.all(code[zero_class] == 0)
    x, code = x[~zero_class], code[~zero_class]
    got = oracle_mod.decode(1, code).astype(np.float64)
    a = x.astype(np.float64)
    fin = np.isfinite(a)
    want = np.full(a.shape, R_MAX)
    want[fin] = _rint_round(a[fin], 12, R_MAX)
    np.testing.assert_array_equal(got, want)


def test_saturation(oracle_mod):
    above_m = np.nextafter(np.float32(M_MAX), np.float32(3))
    above_r = np.nextafter(np.float32(R_MAX), np.float32(3))
    x = np.array([2.0, 1e30, np.inf, -2.0, -np.inf, above_m, above_r], np.float32)
    np.testing.assert_array_equal(oracle_mod.encode(0, x),
                                  np.array([0x7FFF, 0x7FFF, 0x7FFF, 0xFFFF, 0xFFFF, 0x7FFF, 0x7FFF],
                                           np.uint16))
    np.testing.assert_array_equal(oracle_mod.encode(1, x),
                                  np.array([0xFFFF, 0xFFFF, 0xFFFF, 0, 0, 0xFFFE, 0xFFFF], np.uint16))


def _f16_inputs(oracle_mod):
    vals = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    return np.concatenate([boundary_set(np.append(vals, 65536.0)), random_patterns(1 << 22, 13),
                           specials(), _whole_binade(-25), _whole_binade(15)])


def test_binary16_lanes_against_numpy(oracle_mod):
    x = _f16_inputs(oracle_mod)
    code = oracle_mod.encode(2, x)
    want = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    np.testing.assert_array_equal(code[~nan], want[~nan])
    assert np.all(np.isnan(code[nan].view(np.float16)))
    # decode: every binary16 code, against numpy
    allc = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    d = oracle_mod.decode(2, allc)
    ref = allc.view(np.float16).astype(np.float32)
    finite = ~np.isnan(ref)
    np.testing.assert_array_equal(d[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.all(np.isnan(d[~finite]))


def test_bfloat16_against_torch(oracle_mod):
    torch = pytest.importorskip("torch")
    vals = np.arange(0x7F80, dtype=np.uint32)
    bf_vals = (vals << 16).view(np.float32).astype(np.float64)
    x = np.concatenate([boundary_set(np.append(bf_vals[::7], [bf_vals[-1], 2.0 ** 128])),
                        random_patterns(1 << 22, 14), specials()])
    x = x[np.isfinite(x.astype(np.float64)) | np.isinf(x)]
    code = oracle_mod.encode(3, x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    np.testing.assert_array_equal(code[~nan], want[~nan])
    assert np.all((code[nan] & 0x7F80) == 0x7F80) and np.all((code[nan] & 0x7F) != 0)
