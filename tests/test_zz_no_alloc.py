"""pa_step_list_noalloc (the entry point for callers that cannot allocate)
against pa_step_list on the same inputs, through the C ABI: two calls in a
row, the second with a smaller list, in each elementwise mode; outputs
bit-identical (the two run the same kernels; only where the tensor table
lives differs).  In blockwise mode the entry point takes the persistent
launch (no table buffer) and matches pa_step_list's ordered one.  Also: a
list over the table's capacity is refused before anything is enqueued."""
import ctypes

import pytest

from gpu_util import banner

pytestmark = pytest.mark.gpu

E4, F16, F32 = 1, 2, 0


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
        ss = [((torch.randn(n, device="cuda:0", generator=g) * 1e-4),
               (torch.randn(n, device="cuda:0", generator=g) * 1e-4) ** 2) for n in sizes]
    else:
        ss = [torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, device="cuda:0", generator=g)
              for n in sizes]
    return ps, gs, ss


def _clone(ps, gs, ss, mode):
    if mode == F32:
        return [p.clone() for p in ps], [g.clone() for g in gs], [(m.clone(), v.clone()) for m, v in ss]
    return [p.clone() for p in ps], [g.clone() for g in gs], [s.clone() for s in ss]


def _call_noalloc(pa, mode, ps, gs, ss, hyper, step):
    """pa_step_list_noalloc through ctypes, marshalled like pa_step_list."""
    L = pa.lib()
    k = len(ps)
    P = (ctypes.c_void_p * k)(*[p.data_ptr() for p in ps])
    G = (ctypes.c_void_p * k)(*[g.data_ptr() for g in gs])
    keep = []
    S = (ctypes.c_void_p * k)(*[pa._state_arg(mode, p, s, keep) for p, s in zip(ps, ss)])
    N = (ctypes.c_size_t * k)(*[p.numel() for p in ps])
    h = pa._hyper(hyper)
    rc = L.pa_step_list_noalloc(mode, pa.PA_DT_F32, pa.PA_DT_F32, k, P, G, S, N, ctypes.byref(h), int(step),
                                pa._stream(None))
    pa._check(rc)


def torch_equal_bits(a, b):
    import torch
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("mode", [E4, F16, F32])
def test_noalloc_matches_step_list(pa, mode):
    import torch
    hyper = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    counter_a = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    counter_b = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    for call, sizes in enumerate(([4096 * 3 + 5, 1, 0, 70000, 4096, 33], [129, 4096 + 1])):
        ps, gs, ss = _lists(torch, sizes, mode, 40 + call)
        ps2, gs2, ss2 = _clone(ps, gs, ss, mode)
        gs[-1][0] = float("nan")
        gs2[-1][0] = float("nan")
        banner(f"no-alloc mode {mode} call {call + 1}: {len(sizes)} tensors")
        pa.pa_step_list(mode, ps, gs, ss, dict(hyper, nonfinite=counter_a), call + 1)
        _call_noalloc(pa, mode, ps2, gs2, ss2, dict(hyper, nonfinite=counter_b), call + 1)
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            assert torch_equal_bits(ps[i], ps2[i]), f"call {call + 1} tensor {i}: params differ"
            if mode == F32:
                assert torch_equal_bits(ss[i][0], ss2[i][0]) and torch_equal_bits(ss[i][1], ss2[i][1])
            else:
                assert torch.equal(ss[i], ss2[i]), f"call {call + 1} tensor {i}: state words differ"
        assert int(counter_a.item()) == int(counter_b.item()) > 0


def test_noalloc_rejects_a_list_over_capacity(pa):
    import torch
    L = pa.lib()
    k = pa.PA_NOALLOC_MAX_TENSORS + 1
    buf = torch.zeros(4 * k, dtype=torch.float32, device="cuda:0")
    words = torch.zeros(4 * k, dtype=torch.int32, device="cuda:0")
    gbuf = torch.zeros(4 * k, dtype=torch.float32, device="cuda:0")
    P = (ctypes.c_void_p * k)(*[buf.data_ptr() + 16 * i for i in range(k)])
    G = (ctypes.c_void_p * k)(*[gbuf.data_ptr() + 16 * i for i in range(k)])
    S = (ctypes.c_void_p * k)(*[words.data_ptr() + 16 * i for i in range(k)])
    N = (ctypes.c_size_t * k)(*([4] * k))
    h = pa._hyper(dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0))
    rc = L.pa_step_list_noalloc(E4, pa.PA_DT_F32, pa.PA_DT_F32, k, P, G, S, N, ctypes.byref(h), 1, pa._stream(None))
    assert rc == pa.PA_ERR_CAPACITY
    torch.cuda.synchronize()
    assert int(buf.abs().sum().item()) == 0 and int(words.abs().sum().item()) == 0


def test_noalloc_blockwise_matches_the_ordered_launch(pa):
    """Blockwise mode: the no-allocation entry point takes the persistent
    launch, pa_step_list the ordered one (forced here at 5 blocks per
    workgroup); two calls in a row, the second with a smaller list, give
    bit-identical codes, absmax values, BF16 outputs and counts."""
    import numpy as np
    import torch
    import workloads
    BW = 3
    qm, qv = (torch.from_numpy(x).cuda() for x in workloads.code_maps())
    zero = int(np.argmin(np.abs(workloads.code_maps()[0])))
    hyper = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    counter_a = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    counter_b = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    pa.blockwise_path(5)
    try:
        for call, blocks in enumerate(([3, 40, 1], [7])):
            g = torch.Generator(device="cuda:0").manual_seed(60 + call)
            sets = []
            for _ in range(2):
                sets.append(([], [], []))
            for nb in blocks:
                n = nb * 2048
                p = torch.randn(n, device="cuda:0", generator=g) * 0.02
                gr = torch.randn(n, device="cuda:0", generator=g) * 1e-3
                gr[n // 2] = float("inf")
                mc = torch.full((n,), zero, dtype=torch.uint8, device="cuda:0")
                vc = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda:0", generator=g)
                ma = torch.rand(nb, device="cuda:0", generator=g) * 1e-3
                va = torch.rand(nb, device="cuda:0", generator=g) * 1e-6
                for ps, gs, ss in sets:
                    ps.append(p.clone())
                    gs.append(gr.clone())
                    ss.append((mc.clone(), ma.clone(), vc.clone(), va.clone(), qm, qv,
                               torch.zeros(n, dtype=torch.int16, device="cuda:0")))
            (pa_, ga, sa), (pb, gb, sb) = sets
            banner(f"no-alloc blockwise call {call + 1}: {len(blocks)} tensors")
            pa.pa_step_list(BW, pa_, ga, sa, dict(hyper, nonfinite=counter_a), call + 1)
            pa.pa_step_list(BW, pb, gb, sb, dict(hyper, nonfinite=counter_b), call + 1, noalloc=True)
            torch.cuda.synchronize()
            for i in range(len(blocks)):
                for j in (0, 1, 2, 3, 6):
                    x, y = sa[i][j], sb[i][j]
                    assert torch.equal(x.view(torch.uint8), y.view(torch.uint8)), f"call {call + 1} tensor {i} field {j}"
            assert int(counter_a.item()) == int(counter_b.item()) > 0
    finally:
        pa.blockwise_path(0)
