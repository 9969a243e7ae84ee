"""GPU path against the oracle over the hyperparameter space.

The step, the betas, lr, eps and weight decay are all arguments of the
update (KBench quantized-optimizer-state reference, `quantized_adamw_step`
signature; TurboAdam package page, "The AdamW update remains AdamW": the
beta^t bias corrections).  Every combination of

    beta1 in {0, 1e-30, 0.5, 0.9, 0.999999}
    beta2 in {0, 0.5, 0.999, 0.99999}
    lr    in {0, 1e-3, 3}
    wd    in {0, 0.01, 0.3}
    eps   in {0, 1e-8, 1e-2}
    t     in {1, 2, 1000, 10^7, 2^40}

(2,700 per mode) runs once in each mode (packed E4, packed FP16, FP32,
blockwise 8-bit) on its own slice of one device buffer, with random prior
state so that every class of code is decoded (zero, subnormal, normal,
largest; for FP16 also Inf), planted special values (signed zeros,
subnormal and huge gradients and parameters) and random gradients spread
over nine decades.  The launches alternate between the single-tensor and
the list entry points, and between the plain, counting and gradient-scaling
kernel variants.  Bar: state words, codes and absmax values bit-exact
(binary16 and bfloat16 NaN by class); parameters within 2 FP32 ulp or 1e-6
relative (NaN and Inf in the same places).  Non-finite counts equal the
oracle's.
"""
import itertools

import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_params, assert_words, banner

pytestmark = pytest.mark.gpu

E4, F16, F32, BW = 1, 2, 0, 3
BETA1 = [0.0, 1e-30, 0.5, 0.9, 0.999999]
BETA2 = [0.0, 0.5, 0.999, 0.99999]
LR = [0.0, 1e-3, 3.0]
WD = [0.0, 0.01, 0.3]
EPS = [0.0, 1e-8, 1e-2]
STEPS = [1, 2, 1000, 10 ** 7, 2 ** 40]
COMBOS = list(itertools.product(BETA1, BETA2, LR, WD, EPS, STEPS))
SCALE = np.float32(0.7)

L = 4096 + 1031          # elements per combination: one full tile and a ragged one
STRIDE = L + 5           # slice k starts at k*STRIDE + k%4: every 16-byte phase


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


def _grads(r, n):
    g = r.normal(0, 1, n) * 10.0 ** r.uniform(-8, 1, n)
    g[r.random(n) < 0.01] = 0.0
    return g.astype(np.float32)


SPECIAL_G = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-38, 3.0, -3.0, 1e3, -1e-20, 2.5e-4,
                      65000.0, 1e-7, -1e-7, 0.0, 1.0, -1.0], np.float32)
SPECIAL_P = np.array([0.0, -0.0, 1e-45, 1e30, -1e-30, 1.0, -1.0, 3e-39, 0.02, -0.02,
                      1e-3, 123.0, -7.0, 0.0, 0.5, -0.5], np.float32)
SPECIAL_E4 = np.array([0x00000000, 0x00008000, 0x00007FFF, 0x0000FFFF, 0xFFFF0000, 0x00010001,
                       0x07FF07FF, 0x08000800, 0xFFFFFFFF, 0x7FFF7FFF, 0x0FFF87FF, 0x10008001,
                       0x00000001, 0x80000000, 0xF0000FFF, 0x00018000], np.uint32)
SPECIAL_F16 = np.array([0x00000000, 0x00008000, 0x7BFF7BFF, 0x7BFFFBFF, 0x00010001, 0x03FF83FF,
                        0x04000400, 0x00007C00, 0x0000FC00, 0x7C000000, 0x3C00BC00, 0x80000001,
                        0x00017BFF, 0x7BFF0001, 0x3555D555, 0x00000001], np.uint32)


def _slices(k):
    off = k * STRIDE + k % 4
    return off, off + L


def _hyper(pa_mod, k, combo, counter, gscale):
    b1, b2, lr, wd, eps, t = combo
    h = dict(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd)
    if k % 2 == 0:
        h["nonfinite"] = counter
    if k % 5 == 1:
        h["grad_scale"] = gscale
    return h, t


def _prior_state(mode, r, n):
    if mode == E4:
        w = r.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
        return w
    if mode == F16:
        lo = r.integers(0, 0x7C00, n, dtype=np.uint32) | (r.integers(0, 2, n, dtype=np.uint32) << 15)
        hi = r.integers(0, 0x7C00, n, dtype=np.uint32)
        return (hi << 16) | lo
    m = (r.normal(0, 1, n) * 10.0 ** r.uniform(-30, 2, n)).astype(np.float32)
    v = (r.normal(0, 1, n) * 10.0 ** r.uniform(-20, 2, n)).astype(np.float32) ** 2
    return m, v


SPECIAL_M = np.array([0.0, -0.0, 1e-45, 1e30, -3e-39, np.inf], np.float32)
SPECIAL_V = np.array([0.0, 1e-45, 1e30, 0.0, np.inf, 3e-39], np.float32)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", [E4, F16, F32])
def test_elementwise_hyper_grid(pa, mode):
    import torch
    r = np.random.Generator(np.random.PCG64(8100 + mode))
    total = len(COMBOS) * STRIDE + 8
    hp = r.normal(0, 0.02, total).astype(np.float32)
    hg = _grads(r, total)
    if mode == F32:
        hm, hv = _prior_state(mode, r, total)
    else:
        hw = _prior_state(mode, r, total)
    for k in range(len(COMBOS)):
        a, _ = _slices(k)
        hp[a:a + 16] = SPECIAL_P
        hg[a:a + 16] = SPECIAL_G
        if mode == E4:
            hw[a:a + 16] = SPECIAL_E4
        elif mode == F16:
            hw[a:a + 16] = SPECIAL_F16
        else:
            hm[a + 16:a + 22] = SPECIAL_M
            hv[a + 16:a + 22] = SPECIAL_V
    dp = torch.from_numpy(hp.copy()).cuda()
    dg = torch.from_numpy(hg.copy()).cuda()
    if mode == F32:
        dm = torch.from_numpy(hm.copy()).cuda()
        dv = torch.from_numpy(hv.copy()).cuda()
    else:
        dw = torch.from_numpy(hw.view(np.int32).copy()).cuda()
    counter = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    gscale = torch.tensor([float(SCALE)], dtype=torch.float32, device="cuda:0")
    banner(f"hyper grid mode {mode}: {len(COMBOS)} combinations, {L} elements each")
    for k, combo in enumerate(COMBOS):
        a, b = _slices(k)
        h, t = _hyper(pa, k, combo, counter, gscale)
        st = (dm[a:b], dv[a:b]) if mode == F32 else dw[a:b]
        if k % 3 == 0:
            pa.pa_step(mode, dp[a:b], dg[a:b], st, h, t)
        else:
            cuts = [a, a + 1, a + 4100, b] if k % 3 == 1 else [a, b]
            ps = [dp[x:y] for x, y in zip(cuts, cuts[1:])]
            gs = [dg[x:y] for x, y in zip(cuts, cuts[1:])]
            if mode == F32:
                ss = [(dm[x:y], dv[x:y]) for x, y in zip(cuts, cuts[1:])]
            else:
                ss = [dw[x:y] for x, y in zip(cuts, cuts[1:])]
            pa.pa_step_list(mode, ps, gs, ss, h, t)
    torch.cuda.synchronize()
    got_p = dp.cpu().numpy()
    if mode == F32:
        got_m, got_v = dm.cpu().numpy(), dv.cpu().numpy()
    else:
        got_w = dw.cpu().numpy().view(np.uint32)
    want_bad = 0
    same = 0
    for k, combo in enumerate(COMBOS):
        a, b = _slices(k)
        b1, b2, lr, wd, eps, t = combo
        sc = oracle.scalars(lr, b1, b2, eps, wd, t)
        g = hg[a:b].copy()
        if k % 5 == 1:
            g = oracle.scale_grads(0, g, SCALE)
        p = hp[a:b].copy()
        what = f"mode {mode} combo {k} {combo}"
        if mode == F32:
            m, v = hm[a:b].copy(), hv[a:b].copy()
            bad = oracle.step_fp32(p, g, m, v, sc)
            assert_words(got_m[a:b].view(np.uint32), m.view(np.uint32), what=what + " m")
            assert_words(got_v[a:b].view(np.uint32), v.view(np.uint32), what=what + " v")
        else:
            w = hw[a:b].copy()
            bad = oracle.step_packed(mode, p, g, w, sc)
            assert_words(got_w[a:b], w, fp16=(mode == F16), what=what + " words")
        same += assert_params(got_p[a:b], p, what=what + " params")[0]
        if k % 2 == 0:
            want_bad += bad
    assert int(counter.item()) == want_bad
    banner(f"hyper grid mode {mode}: bit-identical params {same}/{len(COMBOS) * L}, "
           f"non-finite {want_bad}")


@pytest.fixture
def bw_path(pa, request):
    pa.blockwise_path(request.param)
    yield request.param
    pa.blockwise_path(0)


# Two blocks per combination take the persistent launch by size; the grid
# runs again through the ordered launch (one block per workgroup, tables
# built once per call), forced.
@pytest.mark.timeout(600)
@pytest.mark.parametrize("bw_path", [0, 1], indirect=True, ids=["by-size", "ordered-k1"])
def test_blockwise_hyper_grid(pa, bw_path):
    import torch
    nb_per = 2
    n_per = nb_per * 2048
    K = len(COMBOS)
    n = K * n_per
    r = np.random.Generator(np.random.PCG64(8200))
    qm, qv = workloads.code_maps()
    hp = r.normal(0, 0.02, n).astype(np.float32)
    hg = _grads(r, n)
    hmc = r.integers(0, 256, n, dtype=np.uint8)
    hvc = r.integers(0, 256, n, dtype=np.uint8)
    hma = (10.0 ** r.uniform(-6, 0, K * nb_per)).astype(np.float32)
    hva = (10.0 ** r.uniform(-12, 0, K * nb_per)).astype(np.float32)
    hma[1::7] = 0.0
    hva[1::5] = 0.0
    for k in range(K):
        a = k * n_per
        hp[a:a + 16] = SPECIAL_P
        hg[a:a + 16] = SPECIAL_G
    dp = torch.from_numpy(hp.copy()).cuda()
    dg = torch.from_numpy(hg.copy()).cuda()
    dmc = torch.from_numpy(hmc.copy()).cuda()
    dvc = torch.from_numpy(hvc.copy()).cuda()
    dma = torch.from_numpy(hma.copy()).cuda()
    dva = torch.from_numpy(hva.copy()).cuda()
    dqm = torch.from_numpy(qm.copy()).cuda()
    dqv = torch.from_numpy(qv.copy()).cuda()
    pout = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    counter = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    gscale = torch.tensor([float(SCALE)], dtype=torch.float32, device="cuda:0")
    banner(f"hyper grid blockwise: {K} combinations, {nb_per} blocks each")
    for k, combo in enumerate(COMBOS):
        a, b = k * n_per, (k + 1) * n_per
        ba, bb = k * nb_per, (k + 1) * nb_per
        h, t = _hyper(pa, k, combo, counter, gscale)
        st = (dmc[a:b], dma[ba:bb], dvc[a:b], dva[ba:bb], dqm, dqv, pout[a:b])
        if k % 3 == 0:
            pa.pa_step(BW, dp[a:b], dg[a:b], st, h, t)
        else:
            pa.pa_step_list(BW, [dp[a:b]], [dg[a:b]], [st], h, t)
    torch.cuda.synchronize()
    got = dict(p=pout.cpu().numpy().view(np.uint16), mc=dmc.cpu().numpy(), vc=dvc.cpu().numpy(),
               ma=dma.cpu().numpy(), va=dva.cpu().numpy())
    want_bad = 0
    for k, combo in enumerate(COMBOS):
        a, b = k * n_per, (k + 1) * n_per
        ba, bb = k * nb_per, (k + 1) * nb_per
        b1, b2, lr, wd, eps, t = combo
        sc = oracle.scalars(lr, b1, b2, eps, wd, t)
        g = hg[a:b].copy()
        if k % 5 == 1:
            g = oracle.scale_grads(0, g, SCALE)
        mc, vc = hmc[a:b].copy(), hvc[a:b].copy()
        ma, va = hma[ba:bb].copy(), hva[ba:bb].copy()
        po = np.zeros(n_per, np.uint16)
        bad = oracle.step_blockwise(hp[a:b].copy(), g, mc, ma, vc, va, qm, qv, po, sc)
        what = f"blockwise combo {k} {combo}"
        gp = got["p"][a:b]
        nan_w = ((po & 0x7F80) == 0x7F80) & ((po & 0x7F) != 0)
        nan_g = ((gp & 0x7F80) == 0x7F80) & ((gp & 0x7F) != 0)
        assert np.array_equal(nan_g, nan_w), what + ": NaN outputs differ"
        assert np.array_equal(gp[~nan_w], po[~nan_w]), what + ": BF16 outputs differ"
        assert np.array_equal(got["mc"][a:b], mc), what + ": first-moment codes differ"
        assert np.array_equal(got["vc"][a:b], vc), what + ": second-moment codes differ"
        for gx, wx, nm in ((got["ma"][ba:bb], ma, "m absmax"), (got["va"][ba:bb], va, "v absmax")):
            nan = np.isnan(wx)
            assert np.array_equal(np.isnan(gx), nan), what + f": {nm} NaN differs"
            assert np.array_equal(gx[~nan].view(np.uint32), wx[~nan].view(np.uint32)), what + f": {nm} differs"
        if k % 2 == 0:
            want_bad += bad
    assert int(counter.item()) == want_bad
    banner(f"hyper grid blockwise: all {K} combinations bit-exact, non-finite {want_bad}")
