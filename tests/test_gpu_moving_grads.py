"""Gradients that move between calls.  torch gives every parameter a freshly
allocated gradient after zero_grad(set_to_none=True), its default, so a
training loop hands the library new gradient pointers on every step.  The
cached plans are keyed on the parameters and state buffers; the new
gradient pointers are checked and written into the cached table by small
kernels on the stream.  These tests step lists, TurboAdam lists, the
gradient pre-pass and both optimizers with fresh gradients on every call,
bit for bit against the oracle, and check that the plan cache holds one
plan per list throughout; bad gradients are refused before anything is
enqueued and leave the plan as it was; and a graph replay between eager
calls with other gradients still steps with the gradients it captured."""
import numpy as np
import pytest

import oracle
from gpu_util import assert_params, assert_words, banner, scalars, to_dev, to_host

pytestmark = pytest.mark.gpu

E4, F32 = 1, 0
H = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
SIZES = [1, 4093, 65536 + 7, 300001]


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


def _states(torch, mode, sizes, r):
    if mode == F32:
        hs = [(r.normal(0, 1e-4, n).astype(np.float32), (r.normal(0, 1e-4, n) ** 2).astype(np.float32))
              for n in sizes]
        return hs, [(to_dev(m), to_dev(v)) for m, v in hs]
    hs = [r.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32) for n in sizes]
    return hs, [to_dev(w) for w in hs]


def _check_states(mode, ds, hs, what):
    for i, (d, h) in enumerate(zip(ds, hs)):
        if mode == F32:
            assert np.array_equal(to_host(d[0]).view(np.uint32), h[0].view(np.uint32)), f"{what} m {i}"
            assert np.array_equal(to_host(d[1]).view(np.uint32), h[1].view(np.uint32)), f"{what} v {i}"
        else:
            assert_words(to_host(d).view(np.uint32), h, what=f"{what} words {i}")


def _oracle_step(mode, hp, hg, hs, t):
    for i in range(len(hp)):
        if mode == F32:
            oracle.step_fp32(hp[i], hg[i], hs[i][0], hs[i][1], scalars(t))
        else:
            oracle.step_packed(1, hp[i], hg[i], hs[i], scalars(t))


@pytest.mark.parametrize("mode", [E4, F32], ids=["e4", "fp32"])
def test_list_step_with_fresh_gradients_every_call(pa, mode):
    import torch
    pa.pa_release_plans()
    r = np.random.Generator(np.random.PCG64(500 + mode))
    hp = [r.normal(0, 0.02, n).astype(np.float32) for n in SIZES]
    dp = [to_dev(a) for a in hp]
    hs, ds = _states(torch, mode, SIZES, r)
    held = []                                  # earlier gradients stay alive, so every call's are new
    for t in range(1, 6):
        hg = [r.normal(0, 1e-3, n).astype(np.float32) for n in SIZES]
        gs = [to_dev(g) for g in hg]
        held.append(gs)
        banner(f"moving gradients, mode {mode}, step {t}")
        pa.pa_step_list(mode, dp, gs, ds, H, t)
        torch.cuda.synchronize()
        _oracle_step(mode, hp, hg, hs, t)
        for i in range(len(SIZES)):
            assert_params(to_host(dp[i]), hp[i], what=f"step {t} params {i}")
        _check_states(mode, ds, hs, f"step {t}")
        if t == 3:
            # gradients refused before anything is enqueued: one at another
            # phase than its parameter, then the parameters themselves
            base = torch.zeros(SIZES[2] + 4, dtype=torch.float32, device="cuda:0")
            bad = list(gs)
            bad[2] = base[1:1 + SIZES[2]]
            with pytest.raises(Exception):
                pa.pa_step_list(mode, dp, bad, ds, H, t + 1)
            with pytest.raises(Exception):
                pa.pa_step_list(mode, dp, list(dp), ds, H, t + 1)
            torch.cuda.synchronize()
            for i in range(len(SIZES)):
                assert_params(to_host(dp[i]), hp[i], what=f"after refused calls, params {i}")
    assert pa.plan_counts()[0] == 1, pa.plan_counts()


def test_turbo_and_prepass_with_fresh_gradients(pa):
    import torch
    pa.pa_release_plans()
    r = np.random.Generator(np.random.PCG64(510))
    sizes = [300, 4096 + 77, 70001]
    hp = [r.normal(0, 0.02, n).astype(np.float32) for n in sizes]
    dp = [to_dev(a) for a in hp]
    hs = [oracle.TurboState(n, n >= 4096, n >= 4096) for n in sizes]
    ds = [pa.TurboState(n, "cuda:0", n >= 4096, n >= 4096, tensor_id=i) for i, n in enumerate(sizes)]
    gs0 = [torch.zeros(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    tl = pa.TurboList(dp, gs0, ds)
    stats = pa.GradStats(gs0)
    sumsq = torch.zeros(1, dtype=torch.float64, device="cuda:0")
    held = []
    for t in range(1, 5):
        hg = [r.normal(0, 1e-3, n).astype(np.float32) for n in sizes]
        gs = [to_dev(g) for g in hg]
        held.append(gs)
        tl.set_grads(gs)
        stats.set_grads(gs)
        banner(f"moving gradients, TurboAdam and pre-pass, step {t}")
        stats.run(sumsq)
        tl.step(H, t)
        torch.cuda.synchronize()
        want, _, _ = oracle.grad_stats(0, hg)
        got = float(sumsq.item())
        assert abs(got - want) <= sum(sizes) * 2.0 ** -53 * want, (got, want)   # a sum in double, any order
        sc = scalars(t)
        ts = oracle.turbo_scalars(H["beta1"], H["beta2"], t)
        for i in range(len(sizes)):
            oracle.turbo_step(hp[i], hg[i], hs[i], sc, ts, t, tensor_id=i)
            assert_params(to_host(dp[i]), hp[i], what=f"step {t} params {i}")
            if hs[i].compress_m:
                assert np.array_equal(to_host(ds[i].m_codes).view(np.uint32), hs[i].m_codes)
                assert np.array_equal(to_host(ds[i].v_index).view(np.uint32), hs[i].v_index)
            else:
                assert np.array_equal(to_host(ds[i].m_fp32).view(np.uint32), hs[i].m_fp32.view(np.uint32))
    steps, pre, turbo = pa.plan_counts()
    assert (pre, turbo) == (1, 1), (steps, pre, turbo)


def test_graph_replay_keeps_its_gradients_between_eager_calls(pa):
    """A step captured with gradients A; eager calls on the same list with
    gradients B; each replay still steps with A.  The same sequence made
    eagerly on a copy (A, then B and A alternating) gives the same bits."""
    import torch
    pa.pa_release_plans()
    r = np.random.Generator(np.random.PCG64(520))
    hp = [r.normal(0, 0.02, n).astype(np.float32) for n in SIZES]
    hs = [r.integers(0, 2 ** 32, n, dtype=np.uint64).astype(np.uint32) for n in SIZES]
    ga = [to_dev(r.normal(0, 1e-3, n).astype(np.float32)) for n in SIZES]
    gb = [to_dev(r.normal(0, 1e-3, n).astype(np.float32)) for n in SIZES]
    p1, s1 = [to_dev(a) for a in hp], [to_dev(w) for w in hs]     # graph + eager
    p2, s2 = [to_dev(a) for a in hp], [to_dev(w) for w in hs]     # eager only
    pa.pa_step_list(E4, p1, ga, s1, H, 1)
    pa.pa_step_list(E4, p2, ga, s2, H, 1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    banner("moving gradients: capturing step 2 with gradients A")
    with torch.cuda.graph(graph, stream=side):
        pa.pa_step_list(E4, p1, ga, s1, H, 2, stream=side)
    torch.cuda.synchronize()
    for k in range(3):
        banner(f"moving gradients: eager B, then replay {k}")
        pa.pa_step_list(E4, p1, gb, s1, H, 2)
        graph.replay()
        pa.pa_step_list(E4, p2, gb, s2, H, 2)
        pa.pa_step_list(E4, p2, ga, s2, H, 2)
        torch.cuda.synchronize()
        for i in range(len(SIZES)):
            assert torch.equal(p1[i].view(torch.int32), p2[i].view(torch.int32)), f"round {k} params {i}"
            assert torch.equal(s1[i], s2[i]), f"round {k} words {i}"


@pytest.mark.parametrize("kind", ["e4-clip-skip", "turbo"])
def test_optimizers_with_zero_grad_set_to_none(pa, kind):
    """torch's default zero_grad: fresh gradients every step; the optimizers
    match the oracle and the plan cache holds one plan per list."""
    import torch
    from adamw_step_amd.optim import PackedAdamW, TurboAdam
    pa.pa_release_plans()
    sizes = [70000, 4096, 333]
    r = np.random.Generator(np.random.PCG64(530))
    ps = [torch.nn.Parameter(torch.from_numpy(r.normal(0, 0.02, n).astype(np.float32)).cuda()) for n in sizes]
    hp = [p.detach().cpu().numpy().copy() for p in ps]
    if kind == "turbo":
        opt = TurboAdam(ps, lr=1e-3, weight_decay=0.01)
        hs = [oracle.TurboState(n, n >= 4096, n >= 4096) for n in sizes]
    else:
        opt = PackedAdamW(ps, lr=1e-3, weight_decay=0.01, mode="e4", max_grad_norm=0.5, skip_nonfinite=True)
        hs = [np.zeros(n, np.uint32) for n in sizes]
    pointers = set()
    for t in range(1, 5):
        opt.zero_grad(set_to_none=True)
        hg = [r.normal(0, 1e-2, n).astype(np.float32) for n in sizes]
        for p, g in zip(ps, hg):
            p.grad = torch.from_numpy(g).cuda()
            pointers.add(p.grad.data_ptr())
        banner(f"{kind}: zero_grad(set_to_none=True), step {t}")
        opt.step()
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            if kind == "turbo":
                oracle.turbo_step(hp[i], hg[i], hs[i], scalars(t), oracle.turbo_scalars(0.9, 0.999, t), t,
                                  tensor_id=i)
            else:
                c = np.float32(opt._clip.item())
                oracle.step_packed(1, hp[i], oracle.scale_grads(0, hg[i], c), hs[i], scalars(t))
                assert_words(opt.state[ps[i]]["words"].cpu().numpy().view(np.uint32), hs[i])
            assert_params(ps[i].detach().cpu().numpy(), hp[i], what=f"{kind} step {t} params {i}")
    assert len(pointers) > len(sizes)          # the gradients did move
    steps, pre, turbo = pa.plan_counts()
    assert (steps, pre, turbo) == ((0, 0, 1) if kind == "turbo" else (1, 1, 0)), (steps, pre, turbo)
