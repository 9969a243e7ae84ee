"""Each list configuration for its own number of steps, once, against the
oracle (the configurations name the step counts: gpt-11m 100 steps,
gpt2-small-124m 50 steps in packed E4, FP32 and packed FP16 mode).

  * gpt-11m, packed E4, 100 steps: every element, every step.
  * gpt2-small-124m, 50 steps in each of the three elementwise modes: the
    whole list is updated on the device every step; the oracle follows a
    fixed seeded sample of elements (every tensor's first and last 4096
    values and a sixteenth of its 4096-value tiles) from the zero state for
    all 50 steps.  The update is elementwise and the gradients of a step are
    fixed, so the sampled elements' whole trajectories are determined by
    their own inputs.

Gradients are drawn on the device from the workloads' seeded generator
(gpt-11m: per-tensor scales log-uniform over 1e-6..1e-1; gpt2-small:
N(0, 1e-3)) and copied to the host for the oracle; parameters start from the
workloads' seeded draws.  Bar: state words bit-exact (binary16 NaN lanes by
class), parameters within 2 FP32 ulp or 1e-6 relative, after every step.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_params, assert_words, banner, gather, hyper, scalars, to_dev, to_host

pytestmark = pytest.mark.gpu

E4, F16, F32 = 1, 2, 0


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


@pytest.mark.timeout(300)
def test_gpt_11m_e4_100_steps(pa):
    import torch
    cfg = 2
    hp = workloads.host_params(cfg)
    sizes = [a.size for a in hp]
    dp = [to_dev(a) for a in hp]
    hw = [np.zeros(n, np.uint32) for n in sizes]
    dw = [to_dev(w) for w in hw]
    dg = [torch.empty(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    sl = pa.StepList(E4, dp, dg, dw)
    same = 0
    for t in range(1, workloads.STEPS[cfg] + 1):
        workloads.device_fill_grads(cfg, t, dg)
        torch.cuda.synchronize()
        hg = [to_host(g) for g in dg]
        if t % 10 == 1:
            banner(f"gpt-11m E4 step {t}/100")
        sl.step(hyper(), t)
        torch.cuda.synchronize()
        sc = scalars(t)
        for i in range(len(sizes)):
            oracle.step_packed(E4, hp[i], hg[i], hw[i], sc)
            assert_words(to_host(dw[i], np.uint32), hw[i], what=f"step {t} tensor {i} words")
            same += assert_params(to_host(dp[i]), hp[i], what=f"step {t} tensor {i} params")[0]
    banner(f"gpt-11m E4 100 steps: bit-identical params {same}/{100 * sum(sizes)}")


def _sample(n, rng, tile=4096):
    tiles = (n + tile - 1) // tile
    pick = set(rng.choice(tiles, size=max(1, tiles // 16), replace=False).tolist())
    idx = np.concatenate([np.arange(k * tile, min(n, (k + 1) * tile)) for k in sorted(pick)])
    return np.union1d(idx, np.union1d(np.arange(min(n, tile)), np.arange(max(0, n - tile), n)))


@pytest.mark.timeout(600)
@pytest.mark.parametrize("mode", [E4, F32, F16])
def test_gpt2_small_124m_50_steps(pa, mode):
    import torch
    cfg = 3
    sizes = workloads.sizes(cfg)
    ps = [torch.empty(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    gs = [torch.empty(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    if mode == F32:
        ss = [(torch.zeros(n, dtype=torch.float32, device="cuda:0"),
               torch.zeros(n, dtype=torch.float32, device="cuda:0")) for n in sizes]
    else:
        ss = [torch.zeros(n, dtype=torch.int32, device="cuda:0") for n in sizes]
    workloads.device_fill_params(cfg, ps)
    rng = np.random.Generator(np.random.PCG64(3300 + mode))
    idx = [_sample(n, rng) for n in sizes]
    didx = [torch.from_numpy(i).to("cuda:0") for i in idx]
    hp = [to_host(gather(p, i)) for p, i in zip(ps, didx)]
    if mode == F32:
        hs = [(np.zeros(i.size, np.float32), np.zeros(i.size, np.float32)) for i in idx]
    else:
        hs = [np.zeros(i.size, np.uint32) for i in idx]
    sl = pa.StepList(mode, ps, gs, ss)
    total = sum(i.size for i in idx)
    banner(f"gpt2-small mode {mode}: {len(sizes)} tensors, {sum(sizes)} params, {total} followed by the oracle")
    same = 0
    try:
        for t in range(1, workloads.STEPS[cfg] + 1):
            workloads.device_fill_grads(cfg, t, gs)
            torch.cuda.synchronize()
            hg = [to_host(gather(g, i)) for g, i in zip(gs, didx)]
            if t % 10 == 1:
                banner(f"gpt2-small mode {mode} step {t}/50")
            sl.step(hyper(), t)
            torch.cuda.synchronize()
            sc = scalars(t)
            for k in range(len(sizes)):
                what = f"mode {mode} step {t} tensor {k}"
                if mode == F32:
                    m, v = hs[k]
                    oracle.step_fp32(hp[k], hg[k], m, v, sc)
                    assert_words(to_host(gather(ss[k][0], didx[k])).view(np.uint32), m.view(np.uint32), what=what + " m")
                    assert_words(to_host(gather(ss[k][1], didx[k])).view(np.uint32), v.view(np.uint32), what=what + " v")
                else:
                    oracle.step_packed(mode, hp[k], hg[k], hs[k], sc)
                    assert_words(to_host(gather(ss[k], didx[k]), np.uint32), hs[k], fp16=(mode == F16),
                                 what=what + " words")
                same += assert_params(to_host(gather(ps[k], didx[k])), hp[k], what=what + " params")[0]
        banner(f"gpt2-small mode {mode} 50 steps: bit-identical params {same}/{50 * total}")
    finally:
        del ps, gs, ss, sl
        torch.cuda.empty_cache()
