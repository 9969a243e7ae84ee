"""GPU path (through the C ABI) against the CPU oracle, element by element.

Bar: state words bit-exact; parameters within 2 FP32 ulp or 1e-6 relative
(reported: how many are bit-identical).  Sizes span several 4096-element
tiles plus ragged tails and every 16-byte phase; lists mix empty, tiny and
large tensors; the non-finite counter, determinism and guard bands around
every buffer are checked too.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_params, assert_words, banner, hyper, scalars, to_dev, to_host

pytestmark = pytest.mark.gpu

E4, F16, F32, BW = 1, 2, 0, 3
GUARD = 1024
SENT = np.float32(-1.2345678e-37)


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


def _torch():
    import torch
    return torch


def _random_state(mode, n, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    if mode == E4:
        return r.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    if mode == F16:
        lo = r.integers(0, 0x7C00, n, dtype=np.uint32) | (r.integers(0, 2, n, dtype=np.uint32) << 15)
        hi = r.integers(0, 0x7C00, n, dtype=np.uint32)
        return (hi << 16) | lo
    m = (r.normal(0, 1e-3, n)).astype(np.float32)
    v = (r.normal(0, 1e-3, n) ** 2).astype(np.float32)
    return m, v


class DevTensor:
    """A device buffer of n elements at a chosen 4-byte phase, with guard bands."""

    def __init__(self, host, phase):
        torch = _torch()
        host = np.ascontiguousarray(host)
        self.n = host.size
        self.phase = phase
        self.dtype = host.dtype
        f = host.view(np.float32) if host.dtype.itemsize == 4 else None
        assert f is not None
        big = np.full(self.n + 2 * GUARD + 4, SENT, np.float32)
        self.off = GUARD + phase
        big[self.off:self.off + self.n] = f
        self.big = torch.from_numpy(big).to("cuda:0")
        view = self.big[self.off:self.off + self.n]
        self.t = view if host.dtype == np.float32 else view.view(torch.int32)

    def host(self):
        return self.big.cpu().numpy()[self.off:self.off + self.n].view(self.dtype).copy()

    def guards_intact(self):
        b = self.big.cpu().numpy()
        return bool(np.all(b[:self.off] == SENT) and np.all(b[self.off + self.n:] == SENT))


def _run_case(pa, mode, sizes, phases, steps, seed, use_list=True, grad_scale=1e-3, check_guards=True):
    """Run `steps` updates on GPU and oracle; compare after every step."""
    torch = _torch()
    r = np.random.Generator(np.random.PCG64(seed))
    hp = [r.normal(0, 0.02, n).astype(np.float32) for n in sizes]
    hs = [_random_state(mode, n, seed + 7 + i) for i, n in enumerate(sizes)]
    dp = [DevTensor(p, ph) for p, ph in zip(hp, phases)]
    if mode == F32:
        ds = [(DevTensor(m, ph), DevTensor(v, ph)) for (m, v), ph in zip(hs, phases)]
    else:
        ds = [DevTensor(s, ph) for s, ph in zip(hs, phases)]
    stats = []
    for t in range(1, steps + 1):
        hg = [(r.normal(0, 1, n) * grad_scale * 10.0 ** r.uniform(-2, 1)).astype(np.float32) for n in sizes]
        dg = [DevTensor(g, ph) for g, ph in zip(hg, phases)]
        states = [(a.t, b.t) for a, b in ds] if mode == F32 else [d.t for d in ds]
        banner(f"mode {mode} sizes {sizes[:4]}{'...' if len(sizes) > 4 else ''} phases {phases[:4]} step {t}")
        if use_list:
            pa.pa_step_list(mode, [d.t for d in dp], [d.t for d in dg], states, hyper(), t)
        else:
            for d, g, s in zip(dp, dg, states):
                pa.pa_step(mode, d.t, g.t, s, hyper(), t)
        torch.cuda.synchronize()
        sc = scalars(t)
        for i in range(len(sizes)):
            if mode == F32:
                m, v = hs[i]
                oracle.step_fp32(hp[i], hg[i], m, v, sc)
                assert_words(ds[i][0].host().view(np.uint32), m.view(np.uint32), what="m")
                assert_words(ds[i][1].host().view(np.uint32), v.view(np.uint32), what="v")
            else:
                oracle.step_packed(mode, hp[i], hg[i], hs[i], sc)
                assert_words(ds[i].host(), hs[i], fp16=(mode == F16))
            stats.append(assert_params(dp[i].host(), hp[i]))
        if check_guards:
            for d in dp + dg + ([x for pair in ds for x in pair] if mode == F32 else ds):
                assert d.guards_intact(), "a kernel wrote outside its buffer"
    return stats


SIZES = [1, 3, 4, 5, 255, 1000, 4095, 4096, 4097, 8191, 3 * 4096 + 7, 100003]


@pytest.mark.parametrize("mode", [E4, F16, F32])
@pytest.mark.parametrize("phase", [0, 1, 2, 3])
def test_single_tensor_sizes_and_phases(pa, mode, phase):
    for n in SIZES:
        _run_case(pa, mode, [n], [phase], steps=2, seed=1000 + n, use_list=False)


@pytest.mark.parametrize("mode", [E4, F16, F32])
def test_mixed_list(pa, mode):
    sizes = [0, 1, 3, 256, 4096, 5000, 0, 77, 65536 + 13, 2, 12288]
    phases = [0, 1, 2, 3, 0, 1, 2, 3, 1, 2, 0]
    stats = _run_case(pa, mode, sizes, phases, steps=3, seed=77)
    banner(f"mode {mode}: bit-identical params {sum(s[0] for s in stats)}/{3 * sum(sizes)}, "
           f"max ulp {max(s[1] for s in stats)}")


def test_single_262k_e4_ten_steps(pa):
    """The single-tensor workload: 262,144 parameters, E4, 10 steps."""
    torch = _torch()
    p = workloads.host_params(1)[0]
    w = np.zeros(p.size, np.uint32)
    dp, dw = to_dev(p), to_dev(w)
    same = 0
    for t in range(1, 11):
        g = workloads.host_grads(1, t)[0]
        banner(f"single-262k step {t}")
        pa.pa_step(E4, dp, to_dev(g), dw, hyper(), t)
        torch.cuda.synchronize()
        oracle.step_packed(E4, p, g, w, scalars(t))
        assert_words(to_host(dw, np.uint32), w)
        same += assert_params(to_host(dp), p)[0]
    banner(f"single-262k: bit-identical params {same}/{10 * p.size}")


def _list_workload(pa, cfg, mode, steps, count=False, grad_scale=None):
    """The workload's tensor list over `steps` steps against the oracle.
    count: pass a non-finite counter (the kernel variant that counts);
    grad_scale: a device gradient scale (the variant that scales)."""
    torch = _torch()
    hp = workloads.host_params(cfg)
    sizes = [a.size for a in hp]
    dp = [to_dev(a) for a in hp]
    if mode == F32:
        hs = [(np.zeros(n, np.float32), np.zeros(n, np.float32)) for n in sizes]
        ds = [(to_dev(m), to_dev(v)) for m, v in hs]
    else:
        hs = [np.zeros(n, np.uint32) for n in sizes]
        ds = [to_dev(s) for s in hs]
    extra = {}
    if count:
        extra["nonfinite"] = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    if grad_scale is not None:
        extra["grad_scale"] = torch.tensor([grad_scale], dtype=torch.float32, device="cuda:0")
    same = total = 0
    for t in range(1, steps + 1):
        hg = workloads.host_grads(cfg, t)
        if count:   # non-finite gradients in the first, a middle and the last tensor
            for i in (0, len(hg) // 2, len(hg) - 1):
                hg[i][[1, hg[i].size // 2, hg[i].size - 1]] = [np.nan, np.inf, -np.inf]
        dg = [to_dev(g) for g in hg]
        banner(f"{workloads.NAMES[cfg]} mode {mode} step {t} count={count} grad_scale={grad_scale}")
        pa.pa_step_list(mode, dp, dg, ds, hyper(**extra), t)
        torch.cuda.synchronize()
        if grad_scale is not None:
            hg = [oracle.scale_grads(0, g, np.float32(grad_scale)) for g in hg]
        sc = scalars(t)
        bad = 0
        for i in range(len(sizes)):
            if mode == F32:
                bad += oracle.step_fp32(hp[i], hg[i], hs[i][0], hs[i][1], sc)
                assert_words(to_host(ds[i][0]).view(np.uint32), hs[i][0].view(np.uint32), what="m")
                assert_words(to_host(ds[i][1]).view(np.uint32), hs[i][1].view(np.uint32), what="v")
            else:
                bad += oracle.step_packed(mode, hp[i], hg[i], hs[i], sc)
                assert_words(to_host(ds[i], np.uint32), hs[i], fp16=(mode == F16))
            s, _ = assert_params(to_host(dp[i]), hp[i])
            same += s
            total += sizes[i]
        if count:
            assert bad > 0 and int(extra["nonfinite"].item()) == bad
            extra["nonfinite"].zero_()
    banner(f"{workloads.NAMES[cfg]} mode {mode}: bit-identical params {same}/{total}")


def test_gpt_11m_list_e4(pa):
    _list_workload(pa, 2, E4, steps=5)


@pytest.mark.parametrize("mode", [E4, F32, F16])
def test_gpt2_small_124m_list(pa, mode):
    _list_workload(pa, 3, mode, steps=2)


@pytest.mark.parametrize("mode", [E4, F32, F16])
def test_gpt2_layer_7m_list(pa, mode):
    """The GPT-2-layer list of the TurboAdam page's benchmark (as read from
    its memory table) in each elementwise mode, three steps."""
    _list_workload(pa, 6, mode, steps=3)


@pytest.mark.parametrize("mode", [E4, F32])
def test_gpt2_small_124m_list_counting_and_scaled(pa, mode):
    """The kernel variant that counts non-finite values and scales the
    gradients (the optimizers' clipped path) over a list of about 30,000
    tiles, some two dozen per workgroup: bit-exact, and the count equals
    the oracle's."""
    _list_workload(pa, 3, mode, steps=2, count=True, grad_scale=0.37)


@pytest.mark.parametrize("mode", [E4, F16, F32])
def test_nonfinite_counter(pa, mode):
    torch = _torch()
    n = 3 * 4096 + 5
    r = np.random.Generator(np.random.PCG64(5))
    p = r.normal(0, 0.02, n).astype(np.float32)
    g = r.normal(0, 1e-3, n).astype(np.float32)
    bad_at = r.choice(n, 37, replace=False)
    g[bad_at[:12]] = np.nan
    g[bad_at[12:25]] = np.inf
    g[bad_at[25:]] = -np.inf
    g[-1] = np.nan                       # in the ragged tail
    counter = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    if mode == F32:
        m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
        st = (to_dev(m), to_dev(v))
    else:
        w = np.zeros(n, np.uint32)
        st = to_dev(w)
    dp = to_dev(p)
    banner(f"nonfinite mode {mode}")
    pa.pa_step(mode, dp, to_dev(g), st, hyper(nonfinite=counter), 1)
    pa.pa_step_list(mode, [dp], [to_dev(g)], [st], hyper(nonfinite=counter), 2)
    torch.cuda.synchronize()
    if mode == F32:
        want = oracle.step_fp32(p, g, m, v, scalars(1)) + oracle.step_fp32(p, g, m, v, scalars(2))
        assert_words(to_host(st[0]).view(np.uint32), m.view(np.uint32))
    else:
        want = oracle.step_packed(mode, p, g, w, scalars(1)) + oracle.step_packed(mode, p, g, w, scalars(2))
        assert_words(to_host(st, np.uint32), w, fp16=(mode == F16))
    assert int(counter.item()) == want
    assert_params(to_host(dp), p)


def test_determinism_and_plan_cache(pa):
    torch = _torch()
    sizes = [4096 * 7 + 3, 129, 50000]
    hp = [np.random.default_rng(i).normal(0, 0.02, n).astype(np.float32) for i, n in enumerate(sizes)]
    hg = [np.random.default_rng(10 + i).normal(0, 1e-3, n).astype(np.float32) for i, n in enumerate(sizes)]
    outs = []
    for rep in range(2):
        dp = [to_dev(p) for p in hp]
        dg = [to_dev(g) for g in hg]
        dw = [torch.zeros(n, dtype=torch.int32, device="cuda:0") for n in sizes]
        banner(f"determinism rep {rep}")
        for t in range(1, 4):
            pa.pa_step_list(E4, dp, dg, dw, hyper(), t)   # second and third calls hit the plan cache
        torch.cuda.synchronize()
        outs.append([to_host(x).copy() for x in dp] + [to_host(x).copy() for x in dw])
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    pa.pa_release_plans()


def test_blockwise_counting_many_blocks_per_workgroup(pa):
    """The counting variant of the blockwise kernel (its own register
    allocation) on 16,384 blocks, some thirteen per workgroup, over two
    steps, with NaN and infinite gradients planted in a few blocks: codes,
    absmax values and BF16 output bit-exact, and the count the oracle's."""
    torch = _torch()
    nb = 16384
    n = nb * 2048
    qm, qv = workloads.code_maps()
    r = np.random.Generator(np.random.PCG64(57))
    p = r.normal(0, 0.02, n).astype(np.float32)
    mc, vc = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    mc[:] = int(np.nonzero(qm == 0.0)[0][0])
    ma, va = np.zeros(nb, np.float32), np.zeros(nb, np.float32)
    dmc, dvc = torch.from_numpy(mc.copy()).cuda(), torch.from_numpy(vc.copy()).cuda()
    dma, dva = to_dev(ma), to_dev(va)
    dqm, dqv = to_dev(qm), to_dev(qv)
    pout = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    hpout = np.zeros(n, np.uint16)
    dp = to_dev(p)
    counter = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    want_bad = 0
    for t in (1, 2):
        g = (r.normal(0, 1e-3, n) * np.repeat(10.0 ** r.uniform(-2, 1, nb), 2048)).astype(np.float32)
        for b, x in ((3, np.nan), (nb // 2 + 1, np.inf), (nb - 2, -np.inf)):
            g[b * 2048 + 100 * t] = x
        banner(f"blockwise counting, {nb} blocks, step {t}")
        pa.pa_step(BW, dp, to_dev(g), (dmc, dma, dvc, dva, dqm, dqv, pout), hyper(nonfinite=counter), t)
        torch.cuda.synchronize()
        want_bad += oracle.step_blockwise(p, g, mc, ma, vc, va, qm, qv, hpout, scalars(t))
        got = to_host(pout, np.uint16)
        nan_w = ((hpout & 0x7F80) == 0x7F80) & ((hpout & 0x7F) != 0)
        nan_g = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        assert np.array_equal(nan_g, nan_w)
        np.testing.assert_array_equal(got[~nan_w], hpout[~nan_w])
        np.testing.assert_array_equal(to_host(dmc), mc)
        np.testing.assert_array_equal(to_host(dvc), vc)
        for got, want in ((to_host(dma), ma), (to_host(dva), va)):
            nan = np.isnan(want)
            assert np.array_equal(np.isnan(got), nan)
            np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
        p = (hpout.astype(np.uint32) << 16).view(np.float32)
        p = np.where(np.isnan(p), np.float32(0), p).astype(np.float32)
        dp = to_dev(p)
    assert want_bad > 0 and int(counter.item()) == want_bad


def test_blockwise_small_multi_step(pa):
    """Blockwise 8-bit mode on 64 blocks for the blockwise configuration's own
    20 steps, full oracle; between steps the BF16 output becomes the next
    step's FP32 parameters on both sides."""
    torch = _torch()
    nb = 64
    n = nb * 2048
    qm, qv = workloads.code_maps()
    r = np.random.Generator(np.random.PCG64(55))
    p = r.normal(0, 0.02, n).astype(np.float32)
    mc, vc = np.zeros(n, np.uint8), np.zeros(n, np.uint8)
    mc[:] = int(np.nonzero(qm == 0.0)[0][0])
    ma, va = np.zeros(nb, np.float32), np.zeros(nb, np.float32)
    dmc, dvc = torch.from_numpy(mc.copy()).cuda(), torch.from_numpy(vc.copy()).cuda()
    dma, dva = to_dev(ma), to_dev(va)
    dqm, dqv = to_dev(qm), to_dev(qv)
    pout = torch.zeros(n, dtype=torch.int16, device="cuda:0")
    hpout = np.zeros(n, np.uint16)
    dp = to_dev(p)
    counter = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    want_bad = 0
    for t in range(1, 21):
        g = (r.normal(0, 1e-3, n) * np.repeat(10.0 ** r.uniform(-2, 1, nb), 2048)).astype(np.float32)
        if t == 3:
            g[5 * 2048 + 17] = np.nan
        banner(f"blockwise 64 blocks step {t}")
        pa.pa_step(BW, dp, to_dev(g), (dmc, dma, dvc, dva, dqm, dqv, pout), hyper(nonfinite=counter), t)
        torch.cuda.synchronize()
        want_bad += oracle.step_blockwise(p, g, mc, ma, vc, va, qm, qv, hpout, scalars(t))
        got = to_host(pout, np.uint16)
        nan_w = ((hpout & 0x7F80) == 0x7F80) & ((hpout & 0x7F) != 0)
        nan_g = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        assert np.array_equal(nan_g, nan_w)
        np.testing.assert_array_equal(got[~nan_w], hpout[~nan_w])
        np.testing.assert_array_equal(to_host(dmc), mc)
        np.testing.assert_array_equal(to_host(dvc), vc)
        for got, want in ((to_host(dma), ma), (to_host(dva), va)):
            nan = np.isnan(want)
            assert np.array_equal(np.isnan(got), nan)
            np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))
        # next step's parameters: the BF16 output, widened (exact) on both sides
        p = (hpout.astype(np.uint32) << 16).view(np.float32)
        p = np.where(np.isnan(p), np.float32(0), p).astype(np.float32)
        dp = to_dev(p)
    assert int(counter.item()) == want_bad


@pytest.mark.parametrize("mode", [E4, F32])
def test_prepared_step_list(pa, mode):
    """StepList (validated once, one C call per step) against the oracle."""
    torch = _torch()
    sizes = [4096 * 3 + 1, 7, 20000, 256]
    r = np.random.Generator(np.random.PCG64(91))
    hp = [r.normal(0, 0.02, n).astype(np.float32) for n in sizes]
    dp = [to_dev(p) for p in hp]
    dg = [torch.empty(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    if mode == F32:
        hs = [(np.zeros(n, np.float32), np.zeros(n, np.float32)) for n in sizes]
        ds = [(to_dev(m), to_dev(v)) for m, v in hs]
    else:
        hs = [np.zeros(n, np.uint32) for n in sizes]
        ds = [to_dev(w) for w in hs]
    sl = pa.StepList(mode, dp, dg, ds)
    for t in range(1, 5):
        hg = [r.normal(0, 1e-3, n).astype(np.float32) for n in sizes]
        for d, g in zip(dg, hg):
            d.copy_(torch.from_numpy(g))      # same storage, new values
        banner(f"StepList mode {mode} step {t}")
        sl.step(hyper(), t)
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            if mode == F32:
                oracle.step_fp32(hp[i], hg[i], hs[i][0], hs[i][1], scalars(t))
                assert_words(to_host(ds[i][0]).view(np.uint32), hs[i][0].view(np.uint32))
            else:
                oracle.step_packed(mode, hp[i], hg[i], hs[i], scalars(t))
                assert_words(to_host(ds[i], np.uint32), hs[i])
            assert_params(to_host(dp[i]), hp[i])


@pytest.mark.parametrize("kind", ["linear", "clustered"])
def test_blockwise_other_maps(pa, kind):
    """Blockwise mode with maps whose midpoints crowd into few buckets of the
    search table (a linear map, and one with 200 entries packed into
    [0.5, 0.5 + 2^-10]), against the oracle."""
    torch = _torch()
    nb = 16
    n = nb * 2048
    if kind == "linear":
        qm = np.linspace(-1, 1, 256).astype(np.float32)
        qv = np.linspace(0, 1, 256).astype(np.float32)
    else:
        inner = 0.5 + np.arange(200, dtype=np.float64) * 2.0 ** -18
        rest = np.linspace(0.51, 1.0, 27)
        pos = np.concatenate([[0.25], inner, rest])
        qm = np.concatenate([-pos[::-1][:27], [0.0], pos])[:256].astype(np.float32)
        qm = np.unique(qm)
        qm = np.concatenate([qm, np.linspace(1.5, 2.0, 256 - qm.size)]).astype(np.float32)
        qv = np.concatenate([[0.0], pos, np.linspace(1.1, 2.0, 255 - pos.size)]).astype(np.float32)
    assert qm.size == 256 and qv.size == 256 and np.all(np.diff(qm) > 0) and np.all(np.diff(qv) > 0)
    r = np.random.Generator(np.random.PCG64(66))
    p = r.normal(0, 0.02, n).astype(np.float32)
    mc = r.integers(0, 256, n, dtype=np.uint8)
    vc = r.integers(0, 256, n, dtype=np.uint8)
    ma = (10.0 ** r.uniform(-4, -1, nb)).astype(np.float32)
    va = (10.0 ** r.uniform(-8, -4, nb)).astype(np.float32)
    dst = [torch.from_numpy(mc.copy()).cuda(), to_dev(ma), torch.from_numpy(vc.copy()).cuda(), to_dev(va),
           to_dev(qm), to_dev(qv), torch.zeros(n, dtype=torch.int16, device="cuda:0")]
    hout = np.zeros(n, np.uint16)
    for t in (1, 2):
        g = (r.normal(0, 1e-2, n) * np.repeat(10.0 ** r.uniform(-2, 1, nb), 2048)).astype(np.float32)
        banner(f"blockwise {kind} map step {t}")
        pa.pa_step(BW, to_dev(p), to_dev(g), tuple(dst), hyper(), t)
        torch.cuda.synchronize()
        oracle.step_blockwise(p, g, mc, ma, vc, va, qm, qv, hout, scalars(t))
        np.testing.assert_array_equal(to_host(dst[0]), mc)
        np.testing.assert_array_equal(to_host(dst[2]), vc)
        np.testing.assert_array_equal(to_host(dst[1]).view(np.uint32), ma.view(np.uint32))
        np.testing.assert_array_equal(to_host(dst[3]).view(np.uint32), va.view(np.uint32))
        np.testing.assert_array_equal(to_host(dst[6], np.uint16), hout)


TYPE_PAIRS = [(1, 1), (2, 2), (1, 0), (2, 0)]       # (param dtype, grad dtype): bf16/f16, 16-bit params + f32 grads


def _typed_case(pa, mode, pdt, gdt, n, phase, steps, seed):
    torch = _torch()
    tdt = {0: torch.float32, 1: torch.bfloat16, 2: torch.float16}
    lane = {1: 3, 2: 2}
    r = np.random.Generator(np.random.PCG64(seed))

    def host16(x, dt):
        return oracle.encode(lane[dt], x) if dt else x.astype(np.float32)

    def dev_at(host, dt):
        big = torch.zeros(n + 8, dtype=tdt[dt] if host.dtype != np.uint32 else torch.int32, device="cuda:0")
        view = big[phase:phase + n]
        src = torch.from_numpy(host.view(np.int16) if host.dtype == np.uint16 else
                               (host.view(np.int32) if host.dtype == np.uint32 else host))
        view.view(src.dtype).copy_(src.to("cuda:0"))
        return big, view

    hp = host16(r.normal(0, 0.02, n).astype(np.float32), pdt)
    _, dp = dev_at(hp, pdt)
    if mode == F32:
        hs = (np.zeros(n, np.float32), np.zeros(n, np.float32))
        keep = [dev_at(hs[0], 0), dev_at(hs[1], 0)]
        ds = (keep[0][1], keep[1][1])
    else:
        hs = _random_state(mode, n, seed + 1)
        keep = dev_at(hs, 0)
        ds = keep[1].view(torch.int32)
    for t in range(1, steps + 1):
        hg = host16((r.normal(0, 1, n) * 1e-3).astype(np.float32), gdt)
        _, dg = dev_at(hg, gdt)
        pa.pa_step(mode, dp, dg, ds, hyper(), t)
        torch.cuda.synchronize()
        oracle.step_typed({F32: 0, E4: 1, F16: 2}[mode], pdt, gdt, hp, hg, hs, scalars(t))
        got_p = dp.cpu().view(torch.int16).numpy().view(np.uint16) if pdt else dp.cpu().numpy()
        if pdt:
            nan = ((hp & 0x7F80) == 0x7F80) & ((hp & 0x7F) != 0) if pdt == 1 else ((hp & 0x7C00) == 0x7C00) & ((hp & 0x3FF) != 0)
            np.testing.assert_array_equal(got_p[~nan], hp[~nan])
        else:
            assert_params(got_p, hp)
        if mode == F32:
            assert_words(ds[0].cpu().numpy().view(np.uint32), hs[0].view(np.uint32), what="m")
            assert_words(ds[1].cpu().numpy().view(np.uint32), hs[1].view(np.uint32), what="v")
        else:
            assert_words(ds.cpu().numpy().view(np.uint32), hs, fp16=(mode == F16))


@pytest.mark.parametrize("mode", [E4, F16, F32])
@pytest.mark.parametrize("pdt,gdt", TYPE_PAIRS)
def test_typed_params_and_grads(pa, mode, pdt, gdt):
    """16-bit parameters (and gradients): the new parameter, rounded to its
    own type, and the state equal the oracle's bit for bit."""
    for n in (5, 4097, 100003):
        for phase in (0, 1, 3):
            banner(f"typed mode {mode} pdt {pdt} gdt {gdt} n {n} phase {phase}")
            _typed_case(pa, mode, pdt, gdt, n, phase, steps=2, seed=n + phase)


@pytest.mark.parametrize("pdt,gdt,count", [(1, 1, False), (2, 0, False), (1, 1, True)])
def test_typed_lists_several_tiles_per_workgroup(pa, pdt, gdt, count):
    """16-bit parameter lists of about 20 M values (some 5,000 tiles, about
    four per workgroup) through StepList, packed E4, two steps: BF16
    parameters and gradients, FP16 parameters with FP32 gradients, and the
    BF16 pair through the variant that counts non-finite values and scales
    the gradients (NaN and infinities planted). New parameters (in their
    own type) and state words equal the oracle's bit for bit."""
    torch = _torch()
    tdt = {0: torch.float32, 1: torch.bfloat16, 2: torch.float16}
    sizes = [4096 * 1500 + 7, 3, 4096 * 1200 + 1, 70001, 4096 * 2300 + 99]
    r = np.random.Generator(np.random.PCG64(200 + 10 * pdt + gdt + count))

    def host(x, dt):
        return x if dt == 0 else oracle.encode(3 if dt == 1 else 2, x)

    def dev(h, dt):
        if dt == 0:
            return to_dev(h)
        return torch.from_numpy(h.view(np.int16).copy()).cuda().view(tdt[dt])

    hp = [host(r.normal(0, 0.02, n).astype(np.float32), pdt) for n in sizes]
    dp = [dev(h, pdt) for h in hp]
    dg = [torch.empty(n, dtype=tdt[gdt], device="cuda:0") for n in sizes]
    hw = [np.zeros(n, np.uint32) for n in sizes]
    dw = [torch.zeros(n, dtype=torch.int32, device="cuda:0") for n in sizes]
    sl = pa.StepList(E4, dp, dg, dw)
    extra, scale = {}, None
    if count:
        scale = np.float32(0.5)
        extra = {"nonfinite": torch.zeros(1, dtype=torch.int64, device="cuda:0"),
                 "grad_scale": torch.tensor([float(scale)], dtype=torch.float32, device="cuda:0")}
    for t in (1, 2):
        g32 = [(r.normal(0, 1, n) * 1e-3).astype(np.float32) for n in sizes]
        if count:
            for i in (0, 2, 4):
                g32[i][[5, sizes[i] // 2, sizes[i] - 1]] = [np.nan, np.inf, -np.inf]
        hg = [host(g, gdt) for g in g32]
        for d, g in zip(dg, hg):
            d.copy_(dev(g, gdt))
        banner(f"typed list pdt {pdt} gdt {gdt} count {count} step {t}")
        sl.step(hyper(**extra), t)
        torch.cuda.synchronize()
        bad = 0
        for i in range(len(sizes)):
            if scale is not None:
                bad += oracle.step_typed(1, pdt, 0, hp[i], oracle.scale_grads(gdt, hg[i], scale), hw[i], scalars(t))
            else:
                bad += oracle.step_typed(1, pdt, gdt, hp[i], hg[i], hw[i], scalars(t))
            got = dp[i].cpu().view(torch.int16).numpy().view(np.uint16)
            want = hp[i]
            nan = (((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0) if pdt == 1
                   else ((want & 0x7C00) == 0x7C00) & ((want & 0x3FF) != 0))
            np.testing.assert_array_equal(got[~nan], want[~nan])
            assert_words(dw[i].cpu().numpy().view(np.uint32), hw[i])
        if count:
            assert bad > 0 and int(extra["nonfinite"].item()) == bad
            extra["nonfinite"].zero_()


def test_typed_list_bf16(pa):
    """A bfloat16 parameter list through StepList (one launch)."""
    torch = _torch()
    sizes = [4096 * 5 + 1, 33, 70000]
    r = np.random.Generator(np.random.PCG64(123))
    hp = [oracle.encode(3, r.normal(0, 0.02, n).astype(np.float32)) for n in sizes]
    dp = [torch.from_numpy(h.view(np.int16).copy()).cuda().view(torch.bfloat16) for h in hp]
    dg = [torch.empty(n, dtype=torch.bfloat16, device="cuda:0") for n in sizes]
    hw = [np.zeros(n, np.uint32) for n in sizes]
    dw = [torch.zeros(n, dtype=torch.int32, device="cuda:0") for n in sizes]
    sl = pa.StepList(E4, dp, dg, dw)
    for t in range(1, 4):
        hg = [oracle.encode(3, r.normal(0, 1e-3, n).astype(np.float32)) for n in sizes]
        for d, g in zip(dg, hg):
            d.view(torch.int16).copy_(torch.from_numpy(g.view(np.int16)))
        banner(f"bf16 StepList step {t}")
        sl.step(hyper(), t)
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            oracle.step_typed(1, 1, 1, hp[i], hg[i], hw[i], scalars(t))
            np.testing.assert_array_equal(dp[i].view(torch.int16).cpu().numpy().view(np.uint16), hp[i])
            assert_words(dw[i].cpu().numpy().view(np.uint32), hw[i])
