"""TurboAdam with bfloat16 and float16 parameters (and gradients) through
pa_turbo_step_list_typed, against the oracle's typed step, bit for bit: the
16-bit parameters, every state word, the tensor scales and the non-finite
count.  The TurboAdam package page's verification runs fp16, bf16 and fp32
parameters; the update runs in FP32 and only the new parameter is rounded
back to its type.  Both kernels (the tuned one and the general one) at
ragged sizes, mixed representation pairs, and a run that pushes binary16
parameters past the largest finite value."""
import numpy as np
import pytest

import oracle
from gpu_util import banner
from test_gpu_turbo import _compare_state

pytestmark = pytest.mark.gpu

PAIRS = [(1, 1), (2, 2), (1, 0), (2, 0), (0, 0)]
PAIR_IDS = ["bf16", "f16", "bf16-f32grad", "f16-f32grad", "f32"]


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


def _host_typed(x32, dt):
    """Host bits of float32 values in type dt, by the oracle's own encoders."""
    x32 = np.ascontiguousarray(x32, np.float32)
    if dt == 0:
        return x32.copy()
    return oracle.encode(3 if dt == 1 else 2, x32)


def _dev_typed(h, dt):
    import torch
    tdt = {0: torch.float32, 1: torch.bfloat16, 2: torch.float16}[dt]
    if dt == 0:
        return torch.from_numpy(h.copy()).cuda()
    return torch.from_numpy(h.view(np.int16).copy()).cuda().view(tdt)


def _bits(t, dt):
    import torch
    if dt == 0:
        return t.cpu().numpy().view(np.uint32)
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _same_params(got, want, dt, what):
    if dt == 0:
        nan_g, nan_w = np.isnan(got.view(np.float32)), np.isnan(want.view(np.float32))
    else:
        exp_mask, man_mask = (0x7F80, 0x007F) if dt == 1 else (0x7C00, 0x03FF)
        nan_g = ((got & exp_mask) == exp_mask) & ((got & man_mask) != 0)
        nan_w = ((want & exp_mask) == exp_mask) & ((want & man_mask) != 0)
    assert np.array_equal(nan_g, nan_w), f"{what}: NaN positions differ"
    diff = np.nonzero((got != want) & ~nan_w)[0]
    assert diff.size == 0, f"{what}: {diff.size} parameters differ, first at {diff[:5]}"


def _run(pa, sizes, flags, pdt, gdt, bits, block, group, steps, seed, hyper_over=None, count=True, plant=None,
         gplant=None):
    import torch
    r = np.random.Generator(np.random.PCG64(seed))
    H = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    if hyper_over:
        H.update(hyper_over)
    hp = []
    for n in sizes:
        x = r.normal(0, 0.02, n).astype(np.float32)
        if plant is not None:
            plant(x)
        hp.append(_host_typed(x, pdt))
    dp = [_dev_typed(h, pdt) for h in hp]
    hs = [oracle.TurboState(n, cm, cv, bits, block, group) for n, (cm, cv) in zip(sizes, flags)]
    ds = [pa.TurboState(n, "cuda:0", cm, cv, bits, tensor_id=i, block_size=block, m_block_size=group)
          for i, (n, (cm, cv)) in enumerate(zip(sizes, flags))]
    hg0 = [_host_typed(np.zeros(n, np.float32), gdt) for n in sizes]
    grads = [_dev_typed(h, gdt) for h in hg0]
    tl = pa.TurboList(dp, grads, ds, v_bits=bits, block_size=block, m_block_size=group)
    hyper = dict(H)
    if count:
        hyper["nonfinite"] = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    want_bad = 0
    for t in range(1, steps + 1):
        hg = []
        for n in sizes:
            g = (r.normal(0, 1, n) * 1e-3 * 10.0 ** r.uniform(-2, 1)).astype(np.float32)
            if gplant is not None:
                gplant(g)
            hg.append(_host_typed(g, gdt))
        for gdev, g in zip(grads, hg):
            gdev.copy_(_dev_typed(g, gdt))
        banner(f"turbo typed p{pdt} g{gdt} bits {bits} block {block} group {group} sizes {sizes[:4]}.. step {t}")
        tl.step(hyper, t)
        torch.cuda.synchronize()
        sc = oracle.scalars(H["lr"], H["beta1"], H["beta2"], H["eps"], H["weight_decay"], t)
        ts = oracle.turbo_scalars(H["beta1"], H["beta2"], t)
        for i in range(len(sizes)):
            want_bad += oracle.turbo_step_typed(pdt, gdt, hp[i], hg[i], hs[i], sc, ts, t, tensor_id=i)
            _compare_state(ds[i], hs[i], f"step {t} tensor {i} (n={sizes[i]}, flags {flags[i]})")
            _same_params(_bits(dp[i], pdt), hp[i].view(np.uint32 if pdt == 0 else np.uint16), pdt,
                         f"step {t} tensor {i} params")
        if count:
            assert int(hyper["nonfinite"].item()) == want_bad
    return hp, pdt


SIZES = [1, 5, 63, 64, 65, 255, 256, 257, 1023, 1025, 4096 + 77, 70001]
FLAGS = [(True, True), (False, True), (True, False), (False, False)] * 3


@pytest.mark.parametrize("pdt,gdt", PAIRS, ids=PAIR_IDS)
@pytest.mark.parametrize("bits,block,group", [(4, 128, 64), (6, 128, 64), (3, 256, 32)], ids=str)
def test_turbo_typed_matches_oracle(pa, pdt, gdt, bits, block, group):
    _run(pa, SIZES, FLAGS, pdt, gdt, bits, block, group, steps=3, seed=300 + 10 * pdt + gdt + bits,
         count=(pdt + gdt + bits) % 2 == 0)


def test_turbo_f16_parameters_overflow_to_inf(pa):
    """lr 30 without decay moves binary16 parameters at 65504 past the largest
    finite value: the kernel rounds them to Inf as the oracle does.  The
    non-finite count looks at the FP32 result, which stays finite."""
    def plant(x):
        x[:4] = [65504.0, -65504.0, 65000.0, -60000.0]

    def gplant(g):   # each update pushes those four away from zero
        g[:4] = [-1e-3, 1e-3, -1e-3, 1e-3]
    hp, _ = _run(pa, [4096 + 13, 300], [(True, True), (False, False)], 2, 2, 4, 128, 64, steps=2, seed=9,
                 hyper_over=dict(lr=30.0, weight_decay=0.0), count=True, plant=plant, gplant=gplant)
    for h in hp:
        assert np.isinf(h[:2].view(np.float16)).all(), h[:4].view(np.float16)


def test_turbo_typed_rejects_bad_pairs_and_alignment(pa):
    """FP32 parameters with 16-bit gradients, and a 16-bit buffer off its
    8-byte alignment, are errors before anything is enqueued."""
    import torch
    n = 1000
    st = pa.TurboState(n, "cuda:0")
    p32 = torch.zeros(n, dtype=torch.float32, device="cuda:0")
    g16 = torch.zeros(n, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(Exception):
        pa.TurboList([p32], [g16], [st]).step(dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0), 1)
    base = torch.zeros(n + 8, dtype=torch.bfloat16, device="cuda:0")
    p_off = base[2:2 + n]            # 4-byte aligned, not 8
    g_ok = torch.zeros(n, dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(Exception):
        pa.TurboList([p_off], [g_ok], [st]).step(dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0),
                                                 1)
