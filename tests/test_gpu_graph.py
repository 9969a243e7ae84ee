"""The list step captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Once a list's launch plan exists, pa_step_list enqueues its kernel launch
and nothing else (no allocation, copy or memset); pa_step_list_noalloc
enqueues its table-upload kernels and the step.  Either can be captured.
A captured call keeps the step number and scalars it was captured with, so
every replay repeats that step on the current contents of the buffers.

Each replay is checked bit for bit against the same call made eagerly on a
copy of the inputs, with eager work (a change to the gradients) and
synchronisations between replays, and the non-finite counters must agree.
"""
import pytest

from gpu_util import banner

pytestmark = pytest.mark.gpu

E4, F32 = 1, 0
HYPER = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


def _lists(torch, sizes, mode, seed):
    g = torch.Generator(device="cuda:0").manual_seed(seed)
    ps = [torch.randn(n, device="cuda:0", generator=g) * 0.02 for n in sizes]
    gs = [torch.randn(n, device="cuda:0", generator=g) * 1e-3 for n in sizes]
    if mode == F32:
        ss = [(torch.randn(n, device="cuda:0", generator=g) * 1e-4,
               (torch.randn(n, device="cuda:0", generator=g) * 1e-4) ** 2) for n in sizes]
    else:
        ss = [torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, device="cuda:0", generator=g)
              for n in sizes]
    gs[1][7] = float("inf")            # a non-finite gradient, so the counter moves
    return ps, gs, ss


def _clone(ps, gs, ss, mode):
    if mode == F32:
        return [p.clone() for p in ps], [g.clone() for g in gs], [(m.clone(), v.clone()) for m, v in ss]
    return [p.clone() for p in ps], [g.clone() for g in gs], [s.clone() for s in ss]


def _flat(ss, mode):
    return [t for pair in ss for t in pair] if mode == F32 else list(ss)


def _same_bits(a, b):
    import torch
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("mode", [E4, F32], ids=["e4", "fp32"])
@pytest.mark.parametrize("noalloc", [False, True], ids=["plan", "noalloc"])
def test_graph_replay_matches_eager(pa, mode, noalloc):
    import torch
    sizes = [1, 4093, 65536 + 7, 300001, 1 << 20]
    ps, gs, ss = _lists(torch, sizes, mode, 31 + mode)
    pe, ge, se = _clone(ps, gs, ss, mode)
    cnt_g = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    cnt_e = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    banner(f"graph: mode {mode} noalloc {noalloc}: eager step 1 on both copies (plan / table set-up)")
    pa.pa_step_list(mode, ps, gs, ss, dict(HYPER, nonfinite=cnt_g), 1, noalloc=noalloc)
    pa.pa_step_list(mode, pe, ge, se, dict(HYPER, nonfinite=cnt_e), 1, noalloc=noalloc)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    banner("graph: capturing step 2")
    with torch.cuda.graph(graph, stream=side):
        pa.pa_step_list(mode, ps, gs, ss, dict(HYPER, nonfinite=cnt_g), 2, stream=side, noalloc=noalloc)
    torch.cuda.synchronize()
    for r in range(4):
        banner(f"graph: replay {r}")
        graph.replay()
        pa.pa_step_list(mode, pe, ge, se, dict(HYPER, nonfinite=cnt_e), 2, noalloc=noalloc)
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            assert _same_bits(ps[i], pe[i]), f"replay {r}: params of tensor {i}"
        for i, (a, b) in enumerate(zip(_flat(ss, mode), _flat(se, mode))):
            assert _same_bits(a, b), f"replay {r}: state {i}"
        assert int(cnt_g.item()) == int(cnt_e.item()) > 0
        # eager work between replays, on both copies alike
        for a, b in zip(gs, ge):
            a.mul_(1.5)
            b.mul_(1.5)
        torch.cuda.synchronize()
    banner(f"graph: 4 replays bit-identical to eager, counter {int(cnt_g.item())}")


@pytest.mark.parametrize("general,dtype", [(False, "fp32"), (True, "fp32"), (False, "bf16")],
                         ids=["tuned", "general", "tuned-bf16"])
def test_turbo_graph_replay_matches_eager(pa, general, dtype):
    """The TurboAdam list step (its step kernel, the chunk pass over the
    residual sums and the per-tensor scale rotation) captured once its plan
    exists and replayed: every replay is the eager call with the same step
    number on a copy, bit for bit, state words and scales included."""
    import torch
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]
    sizes = [1, 300, 4096 + 77, 70001, 1 << 18]
    g = torch.Generator(device="cuda:0").manual_seed(77)
    ps = [(torch.randn(n, device="cuda:0", generator=g) * 0.02).to(tdt) for n in sizes]
    gs = [(torch.randn(n, device="cuda:0", generator=g) * 1e-3).to(tdt) for n in sizes]
    pe, ge = [p.clone() for p in ps], [x.clone() for x in gs]

    def states():
        return [pa.TurboState(n, "cuda:0", n >= 4096, n >= 4096, tensor_id=i) for i, n in enumerate(sizes)]
    sg, se = states(), states()
    tl_g = pa.TurboList(ps, gs, sg, general=general)
    tl_e = pa.TurboList(pe, ge, se, general=general)
    H = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    banner(f"turbo graph ({'general' if general else 'tuned'}, {dtype}): eager step 1 on both (plans)")
    tl_g.step(H, 1)
    tl_e.step(H, 1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        tl_g.step(H, 2, stream=side)
    torch.cuda.synchronize()
    for r in range(4):
        banner(f"turbo graph: replay {r}")
        graph.replay()
        tl_e.step(H, 2)
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            assert torch.equal(ps[i].view(torch.int16 if dtype == "bf16" else torch.int32),
                               pe[i].view(torch.int16 if dtype == "bf16" else torch.int32)), f"replay {r} params {i}"
            for a, b in zip(sg[i].tensors(), se[i].tensors()):
                assert torch.equal(a, b), f"replay {r} state of tensor {i}"
        for a, b in zip(gs, ge):
            a.mul_(1.5)
            b.mul_(1.5)
        torch.cuda.synchronize()
