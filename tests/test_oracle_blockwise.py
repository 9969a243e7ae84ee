"""Pins of the oracle's blockwise 8-bit mode against things other than the oracle.

Source: KBench quantized-optimizer-state reference (`quantized_adamw_step`
and `_requantise`): 2048-element blocks, one FP32 absmax per block per
moment, nearest entry of an ascending 256-point map through the 255 FP32
midpoints with ties to the lower entry, BF16 parameter output.

Pins:
  * torch.bucketize on the same FP32 normalised values and midpoints;
  * a float64 nearest-entry brute force (ties low), with the places where
    the FP32 midpoint differs from the exact one counted;
  * the blockwise step equals the (separately pinned) FP32 step on the
    dequantised moments, followed by numpy's absmax, torch's FP32 division,
    torch.bucketize and torch's bfloat16 cast;
  * zero blocks, NaN blocks, map endpoints and the block-length rule.
"""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
B = 2048
H = workloads.HYPER


def sc(step, **kw):
    import oracle
    h = dict(H)
    h.update(kw)
    return oracle.scalars(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], step)


def _mids(q):
    t = torch.from_numpy(q)
    return (t[:-1] + t[1:]) * 0.5


def test_search_against_bucketize(oracle_mod):
    qm, qv = workloads.code_maps()
    r = np.random.Generator(np.random.PCG64(21))
    for q in (qm, qv):
        mids = _mids(q).numpy()
        c = np.concatenate([r.uniform(-1.2, 1.2, 1 << 16).astype(np.float32), mids,
                            np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(-np.inf)),
                            q, np.array([np.nan, np.inf, -np.inf, 0.0, -0.0, 1.0, -1.0], np.float32),
                            (r.normal(0, 1, 1 << 14) * 10.0 ** r.uniform(-16, 0, 1 << 14)).astype(np.float32)])
        got = oracle_mod.search_codes(q, c)
        want = torch.bucketize(torch.from_numpy(c), torch.from_numpy(mids)).numpy()
        np.testing.assert_array_equal(got.astype(np.int64), want)


def test_search_is_nearest_entry(oracle_mod):
    qm, _ = workloads.code_maps()
    r = np.random.Generator(np.random.PCG64(22))
    c = np.concatenate([r.uniform(-1, 1, 1 << 16),
                        r.normal(0, 1, 1 << 14) * 10.0 ** r.uniform(-9, 0, 1 << 14)]).astype(np.float32)
    code = oracle_mod.search_codes(qm, c).astype(np.int64)
    q64, c64 = qm.astype(np.float64), c.astype(np.float64)
    dist = np.abs(c64[:, None] - q64[None, :])
    best = dist.min(axis=1)
    chosen = dist[np.arange(len(c)), code]
    exact_mid = 0.5 * (q64[:-1] + q64[1:])
    f32_mid = _mids(qm).numpy().astype(np.float64)
    off = chosen != best
    # a non-nearest choice only where c lies between the exact and the FP32 midpoint
    lo = np.minimum(exact_mid, f32_mid)
    hi = np.maximum(exact_mid, f32_mid)
    between = ((c64[:, None] >= lo[None, :]) & (c64[:, None] <= hi[None, :])).any(axis=1)
    assert np.all(between[off])
    # ties resolve to the lower entry
    first_best = np.argmax(dist == best[:, None], axis=1)
    tie = (dist == best[:, None]).sum(axis=1) > 1
    assert np.all(code[tie & ~off] == first_best[tie & ~off])


def _dequant(q, code, absmax):
    return q[code] * np.repeat(absmax, B)


@pytest.mark.parametrize("step", [1, 7])
def test_blockwise_equals_fp32_on_dequantised_moments(oracle_mod, step):
    qm, qv = workloads.code_maps()
    nb = 6
    n = nb * B
    r = np.random.Generator(np.random.PCG64(23 + step))
    p = r.normal(0, 0.02, n).astype(np.float32)
    g = (r.normal(0, 1e-3, n) * 10.0 ** r.uniform(-2, 1, n)).astype(np.float32)
    mc = r.integers(0, 256, n, dtype=np.uint8)
    vc = r.integers(0, 256, n, dtype=np.uint8)
    ma = (10.0 ** r.uniform(-5, -2, nb)).astype(np.float32)
    va = (10.0 ** r.uniform(-9, -5, nb)).astype(np.float32)
    ma[0] = 0.0            # a block with zero state
    va[0] = 0.0
    g[-B:] = 0.0           # a block whose new first moment is beta1 * m exactly
    s = sc(step)
    m = _dequant(qm, mc, ma).astype(np.float32)
    v = _dequant(qv, vc, va).astype(np.float32)
    p1, m1, v1 = p.copy(), m.copy(), v.copy()
    oracle_mod.step_fp32(p1, g, m1, v1, s)

    p_out = np.zeros(n, np.uint16)
    mc2, vc2, ma2, va2 = mc.copy(), vc.copy(), ma.copy(), va.copy()
    bad = oracle_mod.step_blockwise(p, g, mc2, ma2, vc2, va2, qm, qv, p_out, s)
    assert bad == 0
    want_bf = torch.from_numpy(p1).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(p_out, want_bf)
    for x1, q, code, amax in ((m1, qm, mc2, ma2), (v1, qv, vc2, va2)):
        A = np.abs(x1.reshape(nb, B)).max(axis=1)
        np.testing.assert_array_equal(amax, A)
        d = torch.from_numpy(A).clamp(min=1e-30)
        c = torch.from_numpy(x1).view(nb, B) / d[:, None]
        want = torch.bucketize(c, _mids(q)).numpy().reshape(-1)
        np.testing.assert_array_equal(code.astype(np.int64), want)


def test_zero_block_and_endpoints(oracle_mod):
    qm, qv = workloads.code_maps()
    n = 2 * B
    p = np.full(n, 0.5, np.float32)
    g = np.zeros(n, np.float32)
    g[B + 5] = 3e-3                        # block 1: one nonzero gradient
    g[B + 6] = -3e-3
    mc = np.full(n, 128, np.uint8)         # qm[128] == 0
    vc = np.zeros(n, np.uint8)
    ma = np.zeros(2, np.float32)
    va = np.zeros(2, np.float32)
    p_out = np.zeros(n, np.uint16)
    s = sc(1)
    assert qm[128] == 0.0 and qv[0] == 0.0
    oracle_mod.step_blockwise(p, g, mc, ma, vc, va, qm, qv, p_out, s)
    assert ma[0] == 0.0 and va[0] == 0.0
    assert np.all(mc[:B] == 128) and np.all(vc[:B] == 0)
    # block 1: the two extreme elements normalise to exactly +-1 -> map ends
    assert mc[B + 5] == 255 and mc[B + 6] == 0 and vc[B + 5] == 255 and vc[B + 6] == 255
    assert np.all(np.delete(mc[B:], [5, 6]) == 128)


def test_nan_block(oracle_mod):
    qm, qv = workloads.code_maps()
    n = 2 * B
    p = np.zeros(n, np.float32)
    g = np.full(n, 1e-3, np.float32)
    g[3] = np.nan
    mc = np.full(n, 128, np.uint8)
    vc = np.zeros(n, np.uint8)
    ma = np.zeros(2, np.float32)
    va = np.zeros(2, np.float32)
    p_out = np.zeros(n, np.uint16)
    bad = oracle_mod.step_blockwise(p, g, mc, ma, vc, va, qm, qv, p_out, sc(1))
    assert bad == 1
    assert np.isnan(ma[0]) and np.isnan(va[0]) and np.isfinite(ma[1])
    assert np.all(mc[:B] == 255) and np.all(vc[:B] == 255)   # NaN orders above every midpoint
    assert (p_out[3] & 0x7F80) == 0x7F80 and (p_out[3] & 0x7F) != 0


def test_block_length_rule(oracle_mod):
    qm, qv = workloads.code_maps()
    n = B + 4
    z = np.zeros(n, np.float32)
    with pytest.raises(ValueError):
        oracle_mod.step_blockwise(z, z, np.zeros(n, np.uint8), np.zeros(1, np.float32),
                                  np.zeros(n, np.uint8), np.zeros(1, np.float32), qm, qv,
                                  np.zeros(n, np.uint16), sc(1))
