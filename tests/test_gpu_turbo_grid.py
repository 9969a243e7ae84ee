"""TurboAdam away from the default hyperparameters: every combination of
beta1 in {0, 0.5, 0.9}, beta2 in {0.5, 0.999}, lr in {0, 1e-3, 3}, weight
decay in {0, 0.3}, eps in {0, 1e-8, 1e-2} and a first step t in {1, 2,
1000}, each over two consecutive steps t and t + 1 from the empty state, so
that the second decodes what the first wrote: every state word, scale and
parameter bit for bit against the oracle (a NaN matches a NaN), and the
non-finite count equal to the oracle's.  The points with beta1^2 >= beta2 (0.9 with 0.5) break the
rule the TurboAdam page sets for its compressed first moment: there the
call is refused and leaves parameters and state as they were.
The list mixes a tensor that keeps FP32 moments with two compressed ones
whose tails are ragged, through the tuned kernel; a slice of the grid also
runs through the general kernel.  The other index widths (2, 3, 6 and 8
bits) run at four corners of the grid through both kernels, the general
one at a 256-value 1Q block and 32-value UState groups."""
import itertools

import numpy as np
import pytest

import oracle
from gpu_util import banner, to_dev, to_host
from test_gpu_turbo import _host_words

pytestmark = pytest.mark.gpu

SIZES = [300, 4096 + 77, 20001]
GRID = list(itertools.product([0.0, 0.5, 0.9], [0.5, 0.999], [0.0, 1e-3, 3.0], [0.0, 0.3], [0.0, 1e-8, 1e-2],
                              [1, 2, 1000]))


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


def _bits_equal_or_both_nan(got, want):
    g, w = got.view(np.uint32), want.view(np.uint32)
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    return np.array_equal(nan_g, nan_w) and np.array_equal(g[~nan_w], w[~nan_w])


def _compare_state(dev, host, what):
    """Integer state words bit for bit; float state (the moment scales, FP32
    moments) bit for bit where finite and NaN where the oracle has NaN: the
    sign and payload of a NaN made by an invalid operation (0/0 at eps = 0) are
    left open by IEEE 754 and differ between x86 and the GPU's reductions."""
    f32 = lambda a: _host_words(a, np.uint32).view(np.float32)
    if host.compress_m:
        assert np.array_equal(_host_words(dev.m_codes, np.uint32), host.m_codes), f"{what}: UState codes"
        assert np.array_equal(_host_words(dev.m_means, np.uint16), host.m_means), f"{what}: UState means"
        assert _bits_equal_or_both_nan(f32(dev.scalars), host.scal), f"{what}: scales"
    else:
        assert _bits_equal_or_both_nan(f32(dev.m_fp32), host.m_fp32), f"{what}: m"
    if host.compress_v:
        assert np.array_equal(_host_words(dev.v_index, np.uint32), host.v_index), f"{what}: 1Q index words"
        assert np.array_equal(_host_words(dev.v_ends, np.uint16), host.v_ends), f"{what}: 1Q endpoints"
    else:
        assert _bits_equal_or_both_nan(f32(dev.v_fp32), host.v_fp32), f"{what}: v"


@pytest.mark.parametrize("general", [False, True], ids=["tuned", "general"])
def test_turbo_hyperparameter_grid(pa, general):
    import torch
    grid = GRID if not general else GRID[::7]
    r = np.random.Generator(np.random.PCG64(700 + general))
    total_bad, refused = 0, 0
    for k, (b1, b2, lr, wd, eps, t0) in enumerate(grid):
        hp = [r.normal(0, 0.02, n).astype(np.float32) for n in SIZES]
        dp = [to_dev(a) for a in hp]
        hs = [oracle.TurboState(n, n >= 4096, n >= 4096) for n in SIZES]
        ds = [pa.TurboState(n, "cuda:0", n >= 4096, n >= 4096, tensor_id=i) for i, n in enumerate(SIZES)]
        gs = [torch.zeros(n, dtype=torch.float32, device="cuda:0") for n in SIZES]
        tl = pa.TurboList(dp, gs, ds, general=general)
        nf = torch.zeros(1, dtype=torch.int64, device="cuda:0")
        hyper = dict(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, nonfinite=nf)
        want_bad = 0
        if not b1 * b1 < b2:
            with pytest.raises(pa.PAError):
                tl.step(hyper, t0)
            torch.cuda.synchronize()
            for i in range(len(SIZES)):
                assert np.array_equal(to_host(dp[i]).view(np.uint32), hp[i].view(np.uint32)), f"refused {k}"
                _compare_state(ds[i], hs[i], f"refused point {k}")
            refused += 1
            continue
        for t in (t0, t0 + 1):
            hg = [(r.normal(0, 1e-3, n) * 10.0 ** r.uniform(-3, 1)).astype(np.float32) for n in SIZES]
            hg[1][:3] = 0.0                          # zero gradients in a compressed tensor
            for gdev, g in zip(gs, hg):
                gdev.copy_(torch.from_numpy(g))
            tl.step(hyper, t)
            torch.cuda.synchronize()
            sc = oracle.scalars(lr, b1, b2, eps, wd, t)
            ts = oracle.turbo_scalars(b1, b2, t)
            for i in range(len(SIZES)):
                want_bad += oracle.turbo_step(hp[i], hg[i], hs[i], sc, ts, t, tensor_id=i)
                what = f"point {k} (b1 {b1}, b2 {b2}, lr {lr}, wd {wd}, eps {eps}, t {t}) tensor {i}"
                _compare_state(ds[i], hs[i], what)
                assert _bits_equal_or_both_nan(to_host(dp[i]), hp[i]), f"{what}: params"
        assert int(nf.item()) == want_bad, (k, int(nf.item()), want_bad)
        total_bad += want_bad
        if k % 50 == 0:
            banner(f"turbo grid ({'general' if general else 'tuned'}): point {k} of {len(grid)}")
    assert refused == sum(1 for pt in grid if not pt[0] * pt[0] < pt[1])
    banner(f"turbo grid: {len(grid) - refused} points bit-exact, {refused} refused, "
           f"{total_bad} non-finite values counted on both sides")


# Other index widths, at the grid's corners: each width through the tuned
# kernel (default blocks) and the general one (1Q block 256, UState group 32).
CORNERS = [(0.0, 0.5, 3.0, 0.3, 0.0, 1000), (0.9, 0.999, 1e-3, 0.0, 1e-8, 2), (0.5, 0.999, 0.0, 0.3, 1e-2, 1),
           (0.9, 0.5, 1e-3, 0.0, 1e-8, 1)]


@pytest.mark.parametrize("bits", [2, 3, 6, 8])
@pytest.mark.parametrize("general", [False, True], ids=["tuned", "general"])
def test_turbo_widths_at_grid_corners(pa, bits, general):
    import torch
    block, group = (256, 32) if general else (128, 64)
    r = np.random.Generator(np.random.PCG64(760 + bits + 10 * general))
    for k, (b1, b2, lr, wd, eps, t0) in enumerate(CORNERS):
        hp = [r.normal(0, 0.02, n).astype(np.float32) for n in SIZES]
        dp = [to_dev(a) for a in hp]
        hs = [oracle.TurboState(n, n >= 4096, n >= 4096, bits, block, group) for n in SIZES]
        ds = [pa.TurboState(n, "cuda:0", n >= 4096, n >= 4096, bits, tensor_id=i, block_size=block,
                            m_block_size=group) for i, n in enumerate(SIZES)]
        gs = [torch.zeros(n, dtype=torch.float32, device="cuda:0") for n in SIZES]
        tl = pa.TurboList(dp, gs, ds, v_bits=bits, block_size=block, m_block_size=group, general=general)
        nf = torch.zeros(1, dtype=torch.int64, device="cuda:0")
        hyper = dict(lr=lr, beta1=b1, beta2=b2, eps=eps, weight_decay=wd, nonfinite=nf)
        if not b1 * b1 < b2:
            with pytest.raises(pa.PAError):
                tl.step(hyper, t0)
            continue
        want_bad = 0
        for t in (t0, t0 + 1):
            hg = [(r.normal(0, 1e-3, n) * 10.0 ** r.uniform(-3, 1)).astype(np.float32) for n in SIZES]
            hg[1][:3] = 0.0
            for gdev, g in zip(gs, hg):
                gdev.copy_(torch.from_numpy(g))
            banner(f"turbo widths: {bits} bits, {'general' if general else 'tuned'}, corner {k}, step {t}")
            tl.step(hyper, t)
            torch.cuda.synchronize()
            sc = oracle.scalars(lr, b1, b2, eps, wd, t)
            ts = oracle.turbo_scalars(b1, b2, t)
            for i in range(len(SIZES)):
                want_bad += oracle.turbo_step(hp[i], hg[i], hs[i], sc, ts, t, tensor_id=i)
                what = f"{bits} bits corner {k} (b1 {b1}, b2 {b2}, lr {lr}, wd {wd}, eps {eps}, t {t}) tensor {i}"
                _compare_state(ds[i], hs[i], what)
                assert _bits_equal_or_both_nan(to_host(dp[i]), hp[i]), f"{what}: params"
        assert int(nf.item()) == want_bad, (bits, k, int(nf.item()), want_bad)
