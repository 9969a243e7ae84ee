"""Pins of the oracle's update against things other than the oracle.

Update rule: TurboAdam package page, "The AdamW update remains AdamW"
(moments, bias corrections, decoupled decay); operation order: KBench
quantized-optimizer-state reference, `quantized_adamw_step`; update order
(FP32 update with the new unquantised moments, pack afterwards): Packed AdamW
Reference README, introduction, and its project page, Release scope.

Pins:
  * torch.optim.AdamW on the CPU (a library routine with its own op order:
    lerp, addcmul, sqrt(v)/sqrt(bc2), addcdiv), compared within a few ulp;
  * closed forms: step 1 from zero state, zero gradient, lr = 0,
    beta1 = beta2 = 0 (then m' = g and sqrt(g*g) = |g| exactly, so the packed
    lanes hold enc(g) and enc(|g|));
  * the packed step equals the FP32 step run on the decoded moments;
  * which moments feed the update (the FP32 ones, not the re-decoded ones);
  * float64 brute force on small tensors.
"""
import numpy as np
import pytest

import workloads

H = workloads.HYPER


def ulp(x):
    return np.spacing(np.abs(np.asarray(x, np.float32))).astype(np.float64)


def sc(step, **kw):
    import oracle
    h = dict(H)
    h.update(kw)
    return oracle.scalars(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], step)


def test_scalars_closed_forms(oracle_mod):
    s1 = sc(1)
    np.testing.assert_array_equal(s1, np.array([0.9, 0.1, 0.999, 1 - 0.999, 1 - 0.999, 1e-3 / 0.1,
                                                1 - 1e-5, 1e-8], np.float32))
    big = sc(10 ** 7)                               # both corrections reach 1
    assert big[4] == np.float32(1.0) and big[5] == np.float32(1e-3)


def _rand(n, seed, scale):
    r = np.random.Generator(np.random.PCG64(seed))
    return (r.normal(0.0, scale, n)).astype(np.float32)


def test_fp32_mode_against_torch_adamw(oracle_mod):
    torch = pytest.importorskip("torch")
    n = 4096
    p = _rand(n, 1, 0.02)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    tp = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([tp], lr=H["lr"], betas=(H["beta1"], H["beta2"]), eps=H["eps"],
                            weight_decay=H["weight_decay"], foreach=False, fused=False)
    for t in range(1, 8):
        g = _rand(n, 100 + t, 1e-3)
        # start torch from the oracle's current state
        with torch.no_grad():
            tp.copy_(torch.from_numpy(p))
        tp.grad = torch.from_numpy(g.copy())
        if t > 1:
            st = opt.state[tp]
            st["exp_avg"].copy_(torch.from_numpy(m))
            st["exp_avg_sq"].copy_(torch.from_numpy(v))
        m_prev = m.copy()
        opt.step()
        oracle_mod.step_fp32(p, g, m, v, sc(t))
        st = opt.state[tp]
        tm, tv, tpp = st["exp_avg"].numpy(), st["exp_avg_sq"].numpy(), tp.detach().numpy()
        big = np.maximum(np.abs(m_prev), np.abs(g))
        assert np.all(np.abs(tm.astype(np.float64) - m) <= 2 * ulp(big))
        assert np.all(np.abs(tv.astype(np.float64) - v) <= 4 * ulp(v))
        upd = np.abs(p.astype(np.float64) - (tpp.astype(np.float64)))
        s = sc(t)
        upd_mag = np.abs(s[5].astype(np.float64) * m / (np.sqrt(v / np.float64(s[4])) + s[7]))
        assert np.all(upd <= 2 * ulp(p) + 8 * ulp(upd_mag)), np.max(upd / (ulp(p) + ulp(upd_mag)))


def test_step1_from_zero_state(oracle_mod):
    n = 8192
    p = _rand(n, 2, 0.02)
    g = _rand(n, 3, 1e-3)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    p1 = p.copy()
    oracle_mod.step_fp32(p1, g, m, v, sc(1))
    s = sc(1)
    np.testing.assert_array_equal(m, s[1] * g)      # beta1*0 + (1-beta1)*g, one rounding
    np.testing.assert_array_equal(v, (s[3] * g) * g)
    lr, wd, eps = H["lr"], H["weight_decay"], H["eps"]
    g64, p64 = g.astype(np.float64), p.astype(np.float64)
    upd = lr * g64 / (np.abs(g64) + eps)
    want = p64 * (1 - lr * wd) - upd
    assert np.all(np.abs(p1 - want) <= 2 * ulp(p1) + 8 * ulp(upd))


def test_zero_grad_zero_state(oracle_mod):
    n = 1000
    p = _rand(n, 4, 0.02)
    g = np.zeros(n, np.float32)
    w = np.zeros(n, np.uint32)
    p1 = p.copy()
    bad = oracle_mod.step_packed(oracle_mod.PACKED_E4, p1, g, w, sc(1))
    assert bad == 0
    np.testing.assert_array_equal(p1, p * sc(1)[6])
    assert np.all(w == 0)


def test_lr_zero_keeps_params(oracle_mod):
    n = 1000
    p = _rand(n, 5, 0.02)
    g = _rand(n, 6, 1e-2)
    w = np.zeros(n, np.uint32)
    p1 = p.copy()
    oracle_mod.step_packed(oracle_mod.PACKED_E4, p1, g, w, sc(3, lr=0.0))
    np.testing.assert_array_equal(p1, p)


@pytest.mark.parametrize("kind", [1, 2])
def test_zero_betas_store_encoded_grad(oracle_mod, kind):
    n = 1 << 16
    r = np.random.Generator(np.random.PCG64(7))
    g = (r.normal(0, 1, n) * 10.0 ** r.uniform(-9, 0, n)).astype(np.float32)
    p = _rand(n, 8, 0.02)
    w = r.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)   # prior state must not matter
    if kind == 2:
        w &= np.uint32(0x3BFF3BFF)   # keep the prior binary16 state finite
    p1 = p.copy()
    s = sc(5, beta1=0.0, beta2=0.0)
    oracle_mod.step_packed(kind, p1, g, w, s)
    lane_m, lane_r = (0, 1) if kind == 1 else (2, 2)
    np.testing.assert_array_equal(w & 0xFFFF, oracle_mod.encode(lane_m, g))
    np.testing.assert_array_equal(w >> 16, oracle_mod.encode(lane_r, np.abs(g)))
    g64 = g.astype(np.float64)
    upd = H["lr"] * g64 / (np.abs(g64) + H["eps"])
    want = p.astype(np.float64) * (1 - H["lr"] * H["weight_decay"]) - upd
    assert np.all(np.abs(p1 - want) <= 2 * ulp(p1) + 8 * ulp(upd))


@pytest.mark.parametrize("kind", [1, 2])
def test_packed_equals_fp32_on_decoded_moments(oracle_mod, kind):
    n = 1 << 15
    r = np.random.Generator(np.random.PCG64(9))
    lane_m, lane_r = (0, 1) if kind == 1 else (2, 2)
    m_codes = oracle_mod.encode(lane_m, (r.normal(0, 1e-3, n)).astype(np.float32))
    r_codes = oracle_mod.encode(lane_r, np.abs(r.normal(0, 1e-3, n)).astype(np.float32))
    w = (r_codes.astype(np.uint32) << 16) | m_codes.astype(np.uint32)
    p = _rand(n, 10, 0.02)
    g = _rand(n, 11, 1e-3)
    s = sc(4)
    m = oracle_mod.decode(lane_m, m_codes)
    rr = oracle_mod.decode(lane_r, r_codes)
    v = rr * rr
    p_ref = p.copy()
    oracle_mod.step_fp32(p_ref, g, m, v, s)
    p_pk = p.copy()
    oracle_mod.step_packed(kind, p_pk, g, w, s)
    np.testing.assert_array_equal(p_pk.view(np.uint32), p_ref.view(np.uint32))
    np.testing.assert_array_equal(w & 0xFFFF, oracle_mod.encode(lane_m, m))
    np.testing.assert_array_equal(w >> 16, oracle_mod.encode(lane_r, np.sqrt(v)))


def test_update_uses_unquantised_moments(oracle_mod):
    n = 4096
    r = np.random.Generator(np.random.PCG64(12))
    g = (r.normal(0, 1e-3, n)).astype(np.float32)
    p = _rand(n, 13, 0.02)
    w = np.zeros(n, np.uint32)
    s = sc(1)
    p_pk = p.copy()
    oracle_mod.step_packed(oracle_mod.PACKED_E4, p_pk, g, w, s)
    # FP32 moments, straight from the recurrence
    m1 = s[1] * g
    v1 = (s[3] * g) * g
    # re-decoded moments differ from them on most elements...
    mq = oracle_mod.decode(0, (w & 0xFFFF).astype(np.uint16))
    rq = oracle_mod.decode(1, (w >> 16).astype(np.uint16))
    assert np.mean(mq != m1) > 0.5
    # ...and the parameters follow the FP32 ones
    upd_fp32 = (s[5] * m1) / (np.sqrt(v1 / s[4]) + s[7])
    np.testing.assert_array_equal(p_pk, p * s[6] - upd_fp32)
    upd_q = (s[5] * mq) / (np.sqrt((rq * rq) / s[4]) + s[7])
    assert np.mean(p_pk != p * s[6] - upd_q) > 0.1


def _nearest_exact(values_table, x):
    """Nearest table entry in float64, returning (index, on_tie)."""
    k = np.clip(np.searchsorted(values_table, x), 1, len(values_table) - 1)
    lo, hi = values_table[k - 1], values_table[k]
    return np.where(x - lo <= hi - x, k - 1, k), (x - lo) == (hi - x)


def test_float64_brute_force_small(oracle_mod):
    n = 1 << 14
    r = np.random.Generator(np.random.PCG64(14))
    p = _rand(n, 15, 0.02)
    g = (r.normal(0, 1, n) * 10.0 ** r.uniform(-7, -1, n)).astype(np.float32)
    m_codes = oracle_mod.encode(0, (r.normal(0, 1, n) * 10.0 ** r.uniform(-7, -1, n)).astype(np.float32))
    r_codes = oracle_mod.encode(1, (np.abs(r.normal(0, 1, n)) * 10.0 ** r.uniform(-7, -1, n))
                                .astype(np.float32))
    w = (r_codes.astype(np.uint32) << 16) | m_codes.astype(np.uint32)
    s = sc(6)
    m = oracle_mod.decode(0, m_codes).astype(np.float64)
    rv = oracle_mod.decode(1, r_codes).astype(np.float64)
    p1 = p.copy()
    oracle_mod.step_packed(1, p1, g, w, s)
    S = s.astype(np.float64)
    g64 = g.astype(np.float64)
    m1 = S[0] * m + S[1] * g64
    v1 = S[2] * rv * rv + S[3] * g64 * g64
    upd = S[5] * m1 / (np.sqrt(v1 / S[4]) + S[7])
    p_want = p.astype(np.float64) * S[6] - upd
    err = np.abs(p1 - p_want)
    assert np.all(err <= 2 * ulp(p1) + 16 * ulp(upd)), np.max(err / ulp(p1))
    # state codes: nearest in exact arithmetic, except next to a midpoint
    mags = oracle_mod.decode(0, np.arange(0x8000, dtype=np.uint16)).astype(np.float64)
    k, _ = _nearest_exact(mags, np.abs(m1))
    got_m = (w & 0x7FFF).astype(np.int64)
    diff = got_m != k
    mids = 0.5 * (mags[np.minimum(k, got_m)] + mags[np.minimum(k, got_m) + 1])
    near_mid = np.abs(np.abs(m1) - mids) <= 4 * ulp(m1)
    assert np.all(np.abs(got_m - k) <= 1)
    assert np.all(near_mid[diff]) and diff.sum() <= n // 200
    rvals = oracle_mod.decode(1, np.arange(0x10000, dtype=np.uint16)).astype(np.float64)
    kr, _ = _nearest_exact(rvals, np.sqrt(v1))
    got_r = (w >> 16).astype(np.int64)
    diff = got_r != kr
    midr = 0.5 * (rvals[np.minimum(kr, got_r)] + rvals[np.minimum(kr, got_r) + 1])
    near = np.abs(np.sqrt(v1) - midr) <= 4 * ulp(np.sqrt(v1))
    assert np.all(np.abs(got_r - kr) <= 1)
    assert np.all(near[diff]) and diff.sum() <= n // 200


def test_nonfinite_grads(oracle_mod):
    p = np.array([0.01, 0.02, -0.03, 0.04], np.float32)
    g = np.array([np.nan, np.inf, -np.inf, 1e-3], np.float32)
    w = np.zeros(4, np.uint32)
    bad = oracle_mod.step_packed(1, p, g, w, sc(1))
    assert bad == 3
    assert w[0] == 0                                   # NaN -> code 0 in both lanes
    assert w[1] == (0xFFFF << 16) | 0x7FFF             # +Inf saturates both lanes
    assert w[2] == (0xFFFF << 16) | 0xFFFF             # -Inf: m lane -max, RMS lane max
    assert np.isnan(p[:3]).all() and np.isfinite(p[3])


def test_e4_tracks_fp32_over_steps(oracle_mod):
    """Ten steps of the single-tensor workload: the packed first moment stays
    within the rounding it picks up at each step (at most half a lane step per
    step, 2^-12 relative in the normal range or 2^-26 absolute below it,
    carried forward with weight beta1 < 1)."""
    n = 262144
    p_e4 = workloads.host_params(1)[0]
    p_32 = p_e4.copy()
    w = np.zeros(n, np.uint32)
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    bound = np.zeros(n)
    for t in range(1, 11):
        g = workloads.host_grads(1, t)[0]
        assert oracle_mod.step_packed(1, p_e4, g, w, sc(t)) == 0
        oracle_mod.step_fp32(p_32, g, m, v, sc(t))
        mq = oracle_mod.decode(0, (w & 0xFFFF).astype(np.uint16))
        bound = 0.9 * bound + np.abs(mq.astype(np.float64)) * 2.0 ** -12 + 2.0 ** -26
    # the FP32 and packed runs see slightly different moments, hence the 2x margin
    assert np.all(np.abs(mq.astype(np.float64) - m) <= 2 * bound)


def test_bf16_decode_against_torch(oracle_mod):
    torch = pytest.importorskip("torch")
    c = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.decode(3, c)
    want = torch.from_numpy(c.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_typed_f32_equals_untyped(oracle_mod, kind):
    n = 5000
    r = np.random.Generator(np.random.PCG64(31))
    p = r.normal(0, 0.02, n).astype(np.float32)
    g = r.normal(0, 1e-3, n).astype(np.float32)
    s = sc(3)
    if kind == 0:
        st_a = (r.normal(0, 1e-3, n).astype(np.float32), (r.normal(0, 1e-3, n) ** 2).astype(np.float32))
        st_b = (st_a[0].copy(), st_a[1].copy())
        pa_, pb = p.copy(), p.copy()
        oracle_mod.step_fp32(pa_, g, st_a[0], st_a[1], s)
        oracle_mod.step_typed(0, 0, 0, pb, g, st_b, s)
        np.testing.assert_array_equal(st_a[1].view(np.uint32), st_b[1].view(np.uint32))
    else:
        wa = r.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
        if kind == 2:
            wa &= np.uint32(0x3BFF3BFF)
        wb = wa.copy()
        pa_, pb = p.copy(), p.copy()
        oracle_mod.step_packed(kind, pa_, g, wa, s)
        oracle_mod.step_typed(kind, 0, 0, pb, g, wb, s)
        np.testing.assert_array_equal(wa, wb)
    np.testing.assert_array_equal(pa_.view(np.uint32), pb.view(np.uint32))


@pytest.mark.parametrize("pdt,gdt", [(1, 1), (2, 2), (1, 0), (2, 0)])
def test_typed_16bit_is_widen_update_narrow(oracle_mod, pdt, gdt):
    """16-bit parameters/gradients: widen (pinned decodes), the FP32 step
    (pinned against torch's AdamW), round back (pinned encodes)."""
    n = 8192
    r = np.random.Generator(np.random.PCG64(40 + pdt))
    lane = {1: 3, 2: 2}
    p16 = oracle_mod.encode(lane[pdt], r.normal(0, 0.02, n).astype(np.float32))
    gf = r.normal(0, 1e-3, n).astype(np.float32)
    g_in = oracle_mod.encode(lane[gdt], gf) if gdt else gf
    w = np.zeros(n, np.uint32)
    s = sc(1)
    p_typed = p16.copy()
    w_typed = w.copy()
    oracle_mod.step_typed(1, pdt, gdt, p_typed, g_in, w_typed, s)
    p32 = oracle_mod.decode(lane[pdt], p16)
    g32 = oracle_mod.decode(lane[gdt], g_in) if gdt else gf
    oracle_mod.step_packed(1, p32, g32, w, s)
    np.testing.assert_array_equal(w_typed, w)
    np.testing.assert_array_equal(p_typed, oracle_mod.encode(lane[pdt], p32))
