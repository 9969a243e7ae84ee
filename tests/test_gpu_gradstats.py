"""Gradient pre-pass and the step's device inputs, through the C ABI, against
the oracle.

  * pa_grad_stats_list: the non-finite count exactly; the sum of squares
    within the rounding bound of any double summation of n non-negative
    terms, (n - 1) * 2^-53 relative, around the oracle's exact sum; the
    clip coefficient within one binary32 ulp of the oracle's (which
    rounds the exact sum); bit-identical results on a repeated call.
  * grad_scale: a scaled GPU step is compared with the oracle's step on
    gradients it scaled itself (one binary32 product each), to the usual
    bar (state bit-exact, params within 2 ulp / 1e-6).
  * skip_if_nonzero: a nonzero flag leaves every output bit untouched.
"""
import math

import numpy as np
import pytest

import oracle
from gpu_util import assert_params, assert_words, banner, hyper, scalars, to_dev, to_host

pytestmark = pytest.mark.gpu

E4, F16, F32, BW = 1, 2, 0, 3
DT_NP = {0: np.float32, 1: np.uint16, 2: np.uint16}


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


def _torch():
    import torch
    return torch


def _grads(rng, n, gdt, scale=1e-3):
    x = (rng.standard_normal(n) * scale * 10.0 ** rng.uniform(-3, 2, n)).astype(np.float32)
    x[rng.random(n) < 0.01] = 0.0
    if gdt == 0:
        return x
    if gdt == 1:
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return x.astype(np.float16).view(np.uint16)


def _outs():
    torch = _torch()
    return (torch.full((1,), -1.0, dtype=torch.float64, device="cuda:0"),
            torch.full((1,), -1, dtype=torch.int64, device="cuda:0"),
            torch.full((1,), -1.0, dtype=torch.float32, device="cuda:0"))


def _views(host_list, phases, gdt):
    """Device tensors holding each array at a given element phase (mod 4)."""
    torch = _torch()
    out, keep = [], []
    for a, ph in zip(host_list, phases):
        big = np.zeros(a.size + 8, DT_NP[gdt])
        big[ph:ph + a.size] = a
        t = to_dev(big)
        keep.append(t)
        v = t[ph:ph + a.size]
        out.append(v.view(torch.bfloat16) if gdt == 1 else v.view(torch.float16) if gdt == 2 else v)
    return out, keep


def _check_sum(got, want, n, what):
    if math.isnan(want):
        assert math.isnan(got), what
        return
    bound = max(n - 1, 0) * 2.0 ** -53 * want
    assert abs(got - want) <= bound, f"{what}: {got!r} vs exact {want!r} (bound {bound:.3g})"


@pytest.mark.parametrize("gdt", [0, 1, 2])
def test_stats_list_parity(pa, gdt):
    torch = _torch()
    rng = np.random.default_rng(100 + gdt)
    sizes = [0, 1, 5, 4096, 4099, 12345, 65536 + 7, 3, 100003]
    phases = [0, 1, 2, 3, 1, 2, 3, 0, 1]
    hg = [_grads(rng, n, gdt) for n in sizes]
    dg, _keep = _views(hg, phases, gdt)
    s, nf, clip = _outs()
    banner(f"grad stats dtype {gdt}, {len(sizes)} tensors, {sum(sizes)} values")
    pa.pa_grad_stats_list(dg, s, nf, clip, max_norm=0.05)
    torch.cuda.synchronize()
    want_s, want_nf, want_clip = oracle.grad_stats(gdt, hg, max_norm=0.05)
    got_s = float(s.item())
    _check_sum(got_s, want_s, sum(sizes), f"dtype {gdt} sumsq")
    assert int(nf.item()) == want_nf == 0
    got_clip = np.float32(clip.item())
    assert got_clip == oracle.clip_scale(got_s, 0.05)      # same formula on the GPU's own sum
    assert abs(int(got_clip.view(np.int32)) - int(np.float32(want_clip).view(np.int32))) <= 1
    assert got_clip < 1.0                                    # this list is clipped
    again = _outs()[0]
    pa.pa_grad_stats_list(dg, again)
    torch.cuda.synchronize()
    assert again.item() == got_s                             # a fixed summation order
    banner(f"dtype {gdt}: sumsq {got_s!r} vs exact {want_s!r}, clip {float(got_clip)!r}")


def test_stats_large_single_tensor(pa):
    torch = _torch()
    rng = np.random.default_rng(9)
    g = _grads(rng, (1 << 22) + 3, 0)
    s, nf, clip = _outs()
    banner("grad stats: one tensor of 4,194,307 values")
    pa.pa_grad_stats_list([to_dev(g)], s, nf, clip, max_norm=1e9)
    torch.cuda.synchronize()
    want_s, want_nf, want_clip = oracle.grad_stats(0, [g], max_norm=1e9)
    _check_sum(float(s.item()), want_s, g.size, "sumsq")
    assert int(nf.item()) == want_nf == 0
    assert np.float32(clip.item()) == np.float32(want_clip) == np.float32(1.0)


@pytest.mark.parametrize("gdt", [0, 1, 2])
def test_stats_streaming_list(pa, gdt):
    """A list above 128 MiB of gradients, which the pre-pass reads with
    nontemporal loads: the same exact-sum bound, the non-finite count, and a
    repeat that gives the same bits."""
    torch = _torch()
    rng = np.random.default_rng(300 + gdt)
    esz = 4 if gdt == 0 else 2
    big = (160 << 20) // esz                     # 160 MiB in the first tensor
    sizes = [big + 7, 3, 100003]
    phases = [1, 0, 3]
    hg = [_grads(rng, n, gdt) for n in sizes]
    bad_at = [(0, 5), (0, big - 11), (2, 777)]
    specials = {0: np.array([np.nan, np.inf, -np.inf], np.float32),     # NaN, +Inf, -Inf
                1: np.array([0x7FC0, 0x7F80, 0xFF80], np.uint16),
                2: np.array([0x7E00, 0x7C00, 0xFC00], np.uint16)}[gdt]
    for k, (t, i) in enumerate(bad_at):
        hg[t][i] = specials[k]
    dg, _keep = _views(hg, phases, gdt)
    s, nf, clip = _outs()
    banner(f"grad stats streaming dtype {gdt}: {sum(sizes) * esz / 2**20:.0f} MiB")
    pa.pa_grad_stats_list(dg, s, nf, clip, max_norm=1.0)
    torch.cuda.synchronize()
    want_s, want_nf, _ = oracle.grad_stats(gdt, hg, max_norm=1.0)
    assert int(nf.item()) == want_nf == 3
    assert math.isnan(float(s.item())) and math.isnan(want_s)
    for t, i in bad_at:                          # finite again: the sum itself
        hg[t][i] = 0
    dg, _keep = _views(hg, phases, gdt)
    pa.pa_grad_stats_list(dg, s, nf, clip, max_norm=1.0)
    torch.cuda.synchronize()
    want_s, want_nf, _ = oracle.grad_stats(gdt, hg, max_norm=1.0)
    _check_sum(float(s.item()), want_s, sum(sizes), f"dtype {gdt} streaming sumsq")
    assert int(nf.item()) == want_nf == 0
    again = _outs()[0]
    pa.pa_grad_stats_list(dg, again)
    torch.cuda.synchronize()
    assert again.item() == s.item()


@pytest.mark.parametrize("gdt", [0, 1, 2])
def test_stats_nonfinite(pa, gdt):
    torch = _torch()
    rng = np.random.default_rng(31)
    a = _grads(rng, 9000, gdt)
    b = _grads(rng, 4097, gdt)
    inf_bits = {0: np.float32(np.inf), 1: np.uint16(0x7F80), 2: np.uint16(0x7C00)}[gdt]
    nan_bits = {0: np.float32(np.nan), 1: np.uint16(0x7FC1), 2: np.uint16(0x7E01)}[gdt]
    a[[3, 4000, 8999]] = inf_bits
    b[[0, 17]] = inf_bits
    dg, _keep = _views([a, b], [1, 3], gdt)
    s, nf, clip = _outs()
    banner(f"grad stats with infinities, dtype {gdt}")
    pa.pa_grad_stats_list(dg, s, nf, clip, max_norm=1.0)
    torch.cuda.synchronize()
    assert math.isinf(s.item()) and s.item() > 0 and int(nf.item()) == 5
    assert clip.item() == 0.0
    b[100] = nan_bits
    dg, _keep = _views([a, b], [1, 3], gdt)
    banner(f"grad stats with NaN, dtype {gdt}")
    pa.pa_grad_stats_list(dg, s, nf, clip, max_norm=1.0)
    torch.cuda.synchronize()
    want = oracle.grad_stats(gdt, [a, b], max_norm=1.0)
    assert math.isnan(s.item()) and math.isnan(want[0])
    assert int(nf.item()) == want[1] == 6
    assert math.isnan(clip.item())


def test_stats_empty_list(pa):
    torch = _torch()
    s, nf, clip = _outs()
    banner("grad stats: empty list")
    pa.pa_grad_stats_list([], s, nf, clip, max_norm=2.0)
    torch.cuda.synchronize()
    assert s.item() == 0.0 and int(nf.item()) == 0 and clip.item() == 1.0
    z = torch.zeros(0, dtype=torch.float32, device="cuda:0")
    pa.pa_grad_stats_list([z, z], s, nf, clip, max_norm=2.0)
    torch.cuda.synchronize()
    assert s.item() == 0.0 and int(nf.item()) == 0 and clip.item() == 1.0


def test_stats_output_inside_gradients_rejected(pa):
    torch = _torch()
    g = torch.zeros(1024, dtype=torch.float32, device="cuda:0")
    inside = g[8:10].view(torch.float64)
    with pytest.raises(pa.PAError) as e:
        pa.pa_grad_stats_list([g], inside)
    assert e.value.rc == pa.PA_ERR_ALIAS


def _state(mode, n, rng):
    if mode == F32:
        return ((rng.normal(0, 1e-3, n)).astype(np.float32), (rng.normal(0, 1e-3, n) ** 2).astype(np.float32))
    if mode == E4:
        return rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    lo = rng.integers(0, 0x7C00, n, dtype=np.uint32)
    hi = rng.integers(0, 0x7C00, n, dtype=np.uint32)
    return (hi << 16) | lo


@pytest.mark.parametrize("mode", [E4, F16, F32])
@pytest.mark.parametrize("scale", [0.37, 2.0 ** -7])
def test_step_with_grad_scale(pa, mode, scale):
    torch = _torch()
    rng = np.random.default_rng(int(scale * 1000) + mode)
    sizes = [1, 4096, 5003, 70001]
    hp = [rng.normal(0, 0.02, n).astype(np.float32) for n in sizes]
    hg = [_grads(rng, n, 0, 1e-2) for n in sizes]
    hs = [_state(mode, n, rng) for n in sizes]
    dp = [to_dev(a) for a in hp]
    dg = [to_dev(a) for a in hg]
    ds = [(to_dev(m), to_dev(v)) for m, v in hs] if mode == F32 else [to_dev(w) for w in hs]
    sc_dev = torch.tensor([scale], dtype=torch.float32, device="cuda:0")
    for t in (1, 2):
        banner(f"scaled step: mode {mode}, scale {scale}, step {t}")
        pa.pa_step_list(mode, dp, dg, ds, hyper(grad_scale=sc_dev), t)
        torch.cuda.synchronize()
        sc = scalars(t)
        for i in range(len(sizes)):
            gs = oracle.scale_grads(0, hg[i], np.float32(scale))
            if mode == F32:
                oracle.step_fp32(hp[i], gs, hs[i][0], hs[i][1], sc)
                assert_words(to_host(ds[i][0]).view(np.uint32), hs[i][0].view(np.uint32), what="m")
                assert_words(to_host(ds[i][1]).view(np.uint32), hs[i][1].view(np.uint32), what="v")
            else:
                oracle.step_packed(mode, hp[i], gs, hs[i], sc)
                assert_words(to_host(ds[i], np.uint32), hs[i], fp16=(mode == F16))
            assert_params(to_host(dp[i]), hp[i])


def test_typed_step_with_grad_scale(pa):
    """bfloat16 parameters and gradients, single-tensor entry, E4 state."""
    torch = _torch()
    rng = np.random.default_rng(44)
    n = 3 * 4096 + 11
    p = (rng.normal(0, 0.02, n).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    g = _grads(rng, n, 1, 1e-2)
    w = np.zeros(n, np.uint32)
    dp = to_dev(p).view(torch.bfloat16)
    dg = to_dev(g).view(torch.bfloat16)
    dw = to_dev(w)
    sc_dev = torch.tensor([0.61], dtype=torch.float32, device="cuda:0")
    for t in (1, 2, 3):
        banner(f"typed scaled step {t}")
        pa.pa_step(E4, dp, dg, dw, hyper(grad_scale=sc_dev), t)
        torch.cuda.synchronize()
        gs = oracle.scale_grads(1, g, np.float32(0.61))
        oracle.step_typed(1, 1, 0, p, gs, w, scalars(t))
        assert_words(to_host(dw, np.uint32), w)
        assert np.array_equal(to_host(dp.view(torch.int16), np.uint16), p)


def test_blockwise_with_grad_scale(pa):
    torch = _torch()
    import workloads
    rng = np.random.default_rng(8)
    n = 5 * 2048
    qm, qv = workloads.code_maps()
    p = rng.normal(0, 0.02, n).astype(np.float32)
    g = _grads(rng, n, 0, 1e-3)
    mc, vc = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    ma, va = np.zeros(n // 2048, np.float32), np.zeros(n // 2048, np.float32)
    pout = np.zeros(n, np.uint16)
    d = dict(p=to_dev(p), g=to_dev(g), mc=to_dev(mc), ma=to_dev(ma), vc=to_dev(vc), va=to_dev(va),
             qm=to_dev(qm), qv=to_dev(qv), po=to_dev(pout))
    sc_dev = torch.tensor([3.5], dtype=torch.float32, device="cuda:0")
    for t in (1, 2):
        banner(f"blockwise scaled step {t}")
        pa.pa_step(BW, d["p"], d["g"], (d["mc"], d["ma"], d["vc"], d["va"], d["qm"], d["qv"], d["po"]),
                   hyper(grad_scale=sc_dev), t)
        torch.cuda.synchronize()
        oracle.step_blockwise(p, oracle.scale_grads(0, g, np.float32(3.5)), mc, ma, vc, va, qm, qv, pout,
                              scalars(t))
        assert np.array_equal(to_host(d["mc"], np.uint8), mc) and np.array_equal(to_host(d["vc"], np.uint8), vc)
        assert np.array_equal(to_host(d["ma"]).view(np.uint32), ma.view(np.uint32))
        assert np.array_equal(to_host(d["va"]).view(np.uint32), va.view(np.uint32))
        assert np.array_equal(to_host(d["po"], np.uint16), pout)


@pytest.mark.parametrize("mode", [E4, F32, BW])
def test_skip_flag(pa, mode):
    torch = _torch()
    import workloads
    rng = np.random.default_rng(12)
    n = 4 * 2048 + (0 if mode == BW else 5)
    p = to_dev(rng.normal(0, 0.02, n).astype(np.float32))
    g = to_dev(_grads(rng, n, 0))
    if mode == E4:
        st = to_dev(rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32))
        bufs = [p, st]
    elif mode == F32:
        st = (to_dev(rng.normal(0, 1e-3, n).astype(np.float32)), to_dev(rng.random(n).astype(np.float32)))
        bufs = [p, *st]
    else:
        qm, qv = workloads.code_maps()
        st = (to_dev(rng.integers(0, 256, n, dtype=np.uint8)), to_dev(rng.random(n // 2048).astype(np.float32)),
              to_dev(rng.integers(0, 256, n, dtype=np.uint8)), to_dev(rng.random(n // 2048).astype(np.float32)),
              to_dev(qm), to_dev(qv), to_dev(np.zeros(n, np.uint16)))
        bufs = [p, st[0], st[1], st[2], st[3], st[6]]
    before = [b.clone() for b in bufs]
    flag = torch.tensor([3], dtype=torch.int64, device="cuda:0")
    counter = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    banner(f"skip flag set, mode {mode}")
    pa.pa_step(mode, p, g, st, hyper(nonfinite=counter, skip_if_nonzero=flag, grad_scale=None), 1)
    torch.cuda.synchronize()
    for a, b in zip(bufs, before):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "a skipped call wrote"
    assert int(counter.item()) == 0
    flag.zero_()
    banner(f"skip flag clear, mode {mode}")
    pa.pa_step(mode, p, g, st, hyper(skip_if_nonzero=flag), 1)
    torch.cuda.synchronize()
    assert not torch.equal(bufs[0].view(torch.uint8), before[0].view(torch.uint8)) or mode == BW
    assert any(not torch.equal(a.view(torch.uint8), b.view(torch.uint8)) for a, b in zip(bufs, before))


def test_clip_pipeline_without_host_sync(pa):
    """Pre-pass, then the list step fed its clip coefficient and non-finite
    count, all enqueued before one synchronisation; then a list with an
    infinite gradient, whose update is skipped."""
    torch = _torch()
    rng = np.random.default_rng(21)
    sizes = [4096, 333, 20000]
    hp = [rng.normal(0, 0.02, n).astype(np.float32) for n in sizes]
    hg = [_grads(rng, n, 0, 1.0) for n in sizes]
    hw = [np.zeros(n, np.uint32) for n in sizes]
    dp, dg, dw = [to_dev(a) for a in hp], [to_dev(a) for a in hg], [to_dev(a) for a in hw]
    s, nf, clip = _outs()
    stats = pa.GradStats(dg)
    banner("clip pipeline: pre-pass then step, one sync")
    stats.run(s, nf, clip, max_norm=1.0)
    pa.pa_step_list(E4, dp, dg, dw, hyper(grad_scale=clip, skip_if_nonzero=nf), 1)
    torch.cuda.synchronize()
    c = np.float32(clip.item())
    assert int(nf.item()) == 0 and c < 1.0
    want_s, _, want_c = oracle.grad_stats(0, hg, max_norm=1.0)
    _check_sum(s.item(), want_s, sum(sizes), "sumsq")
    assert abs(int(c.view(np.int32)) - int(np.float32(want_c).view(np.int32))) <= 1
    for i in range(len(sizes)):
        oracle.step_packed(E4, hp[i], oracle.scale_grads(0, hg[i], c), hw[i], scalars(1))
        assert_words(to_host(dw[i], np.uint32), hw[i])
        assert_params(to_host(dp[i]), hp[i])
    dg[1][7] = float("inf")
    before = [w.clone() for w in dw] + [q.clone() for q in dp]
    banner("clip pipeline: infinite gradient, update skipped")
    stats.run(s, nf, clip, max_norm=1.0)
    pa.pa_step_list(E4, dp, dg, dw, hyper(grad_scale=clip, skip_if_nonzero=nf), 2)
    torch.cuda.synchronize()
    assert int(nf.item()) == 1
    for a, b in zip(dw + dp, before):
        assert torch.equal(a, b)
