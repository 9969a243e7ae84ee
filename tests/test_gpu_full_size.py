"""Full-size workloads, in the launch configuration the benchmark times,
checked against the oracle on sampled outputs.

  * llama-7b: 291 tensors, 6,738,415,616 parameters, in each elementwise
    mode (packed E4, packed FP16, FP32), two steps of one persistent launch
    each; sampled: every tensor's first and last 64 Ki
    elements plus a seeded 1/1024 of its 64 Ki-element tiles.  The step is
    elementwise, so the sampled inputs, gathered from the device before the
    step, determine the sampled outputs exactly.
  * blockwise-268m: one flat tensor of 2^28 parameters (131,072 blocks),
    three steps; sampled: the first, last and 254 seeded blocks (blocks are
    independent).  Between steps the BF16 output, widened on the device,
    becomes the next step's FP32 parameters.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import assert_params, assert_words, banner, gather, hyper, scalars, to_host

pytestmark = pytest.mark.gpu

CHUNK = 1 << 16


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


def _sample_index(n, rng):
    tiles = (n + CHUNK - 1) // CHUNK
    pick = {0, tiles - 1}
    k = max(1, tiles // 1024)
    pick.update(rng.choice(tiles, size=min(k, tiles), replace=False).tolist())
    idx = np.concatenate([np.arange(t * CHUNK, min(n, (t + 1) * CHUNK)) for t in sorted(pick)])
    if n > CHUNK:
        idx = np.union1d(idx, np.arange(n - CHUNK, n))
    return idx


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["e4", "fp16", "fp32"])
def test_llama_7b_sampled(pa, mode):
    import torch
    cfg = 4
    sizes = workloads.sizes(cfg)
    state_bytes = 8 if mode == "fp32" else 4
    banner(f"llama-7b {mode}: allocating {sum(sizes) * (8 + state_bytes) / 1e9:.1f} GB")
    ps = [torch.empty(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    gs = [torch.empty(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    if mode == "fp32":
        ss = [(torch.zeros(n, dtype=torch.float32, device="cuda:0"), torch.zeros(n, dtype=torch.float32, device="cuda:0"))
              for n in sizes]
    else:
        ss = [torch.zeros(n, dtype=torch.int32, device="cuda:0") for n in sizes]
    code = {"fp32": 0, "e4": 1, "fp16": 2}[mode]
    workloads.device_fill_params(cfg, ps)
    rng = np.random.Generator(np.random.PCG64(4242 + code))
    idx = [_sample_index(n, rng) for n in sizes]
    didx = [torch.from_numpy(i).to("cuda:0") for i in idx]
    total = sum(i.size for i in idx)

    def gather_state(k):
        if mode == "fp32":
            return tuple(to_host(gather(x, didx[k])) for x in ss[k])
        return to_host(gather(ss[k], didx[k]), np.uint32)

    try:
        for t in (1, 2):
            workloads.device_fill_grads(cfg, t, gs)
            torch.cuda.synchronize()
            hp = [to_host(p[i]) for p, i in zip(ps, didx)]
            hg = [to_host(g[i]) for g, i in zip(gs, didx)]
            hs = [gather_state(k) for k in range(len(sizes))]
            banner(f"llama-7b {mode} step {t}: one persistent launch over 291 tensors")
            pa.pa_step_list(code, ps, gs, ss, hyper(), t)
            torch.cuda.synchronize()
            sc = scalars(t)
            same = 0
            for k in range(len(sizes)):
                if mode == "fp32":
                    m, v = hs[k]
                    oracle.step_fp32(hp[k], hg[k], m, v, sc)
                    gm, gv = gather_state(k)
                    assert_words(gm, m, what=f"tensor {k} m")
                    assert_words(gv, v, what=f"tensor {k} v")
                else:
                    oracle.step_packed(code, hp[k], hg[k], hs[k], sc)
                    assert_words(gather_state(k), hs[k], fp16=mode == "fp16", what=f"tensor {k} words")
                same += assert_params(to_host(gather(ps[k], didx[k])), hp[k], what=f"tensor {k} params")[0]
            banner(f"llama-7b {mode} step {t}: {total} sampled elements, bit-identical params {same}")
    finally:
        del ps, gs, ss
        torch.cuda.empty_cache()
        pa.pa_release_plans()


@pytest.mark.timeout(600)
def test_blockwise_268m_sampled(pa):
    import torch
    cfg = 5
    n = workloads.total(cfg)
    nb = n // 2048
    qm, qv = workloads.code_maps()
    zero_m = int(np.nonzero(qm == 0.0)[0][0])
    p = torch.empty(n, dtype=torch.float32, device="cuda:0")
    g = torch.empty(n, dtype=torch.float32, device="cuda:0")
    workloads.device_fill_params(cfg, [p])
    mc = torch.full((n,), zero_m, dtype=torch.uint8, device="cuda:0")
    vc = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
    ma = torch.zeros(nb, dtype=torch.float32, device="cuda:0")
    va = torch.zeros(nb, dtype=torch.float32, device="cuda:0")
    dqm = torch.from_numpy(qm).to("cuda:0")
    dqv = torch.from_numpy(qv).to("cuda:0")
    pout = torch.empty(n, dtype=torch.int16, device="cuda:0")
    rng = np.random.Generator(np.random.PCG64(5151))
    blocks = np.union1d([0, nb - 1], rng.choice(nb, 254, replace=False))
    eidx = torch.from_numpy((blocks[:, None] * 2048 + np.arange(2048)[None, :]).reshape(-1)).to("cuda:0")
    bidx = torch.from_numpy(blocks).to("cuda:0")
    try:
        for t in (1, 2, 3):
            workloads.device_fill_grads(cfg, t, [g])
            torch.cuda.synchronize()
            hp, hg = to_host(gather(p, eidx)), to_host(gather(g, eidx))
            hmc, hvc = to_host(gather(mc, eidx)).copy(), to_host(gather(vc, eidx)).copy()
            hma, hva = to_host(gather(ma, bidx)).copy(), to_host(gather(va, bidx)).copy()
            banner(f"blockwise-268m step {t}")
            pa.pa_step(3, p, g, (mc, ma, vc, va, dqm, dqv, pout), hyper(), t)
            torch.cuda.synchronize()
            hout = np.zeros(hp.size, np.uint16)
            oracle.step_blockwise(hp, hg, hmc, hma, hvc, hva, qm, qv, hout, scalars(t))
            np.testing.assert_array_equal(to_host(gather(pout, eidx), np.uint16), hout)
            np.testing.assert_array_equal(to_host(gather(mc, eidx)), hmc)
            np.testing.assert_array_equal(to_host(gather(vc, eidx)), hvc)
            assert_words(to_host(gather(ma, bidx)).view(np.uint32), hma.view(np.uint32), what="m absmax")
            assert_words(to_host(gather(va, bidx)).view(np.uint32), hva.view(np.uint32), what="v absmax")
            assert_params(to_host(gather(pout, eidx).view(torch.bfloat16).float()),
                          (hout.astype(np.uint32) << 16).view(np.float32))
            p = pout.view(torch.bfloat16).float()
    finally:
        del p, g, mc, vc
        torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_llama_7b_grad_stats_exact(pa):
    """The gradient pre-pass over all 6,738,415,616 gradients of the 291-tensor
    list, in the launch configuration the benchmark times, against the
    oracle's exact sum (accumulated tensor by tensor on the host) and its
    non-finite count."""
    import math
    import torch
    cfg = 4
    sizes = workloads.sizes(cfg)
    banner(f"llama-7b grad stats: allocating {sum(sizes) * 4 / 1e9:.1f} GB of gradients")
    gs = [torch.empty(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    try:
        workloads.device_fill_grads(cfg, 1, gs)
        k = next(i for i, n in enumerate(sizes) if n > 1 << 20 and i > 10)
        gs[k][12345] = float("inf")
        s = torch.zeros(1, dtype=torch.float64, device="cuda:0")
        nf = torch.zeros(1, dtype=torch.int64, device="cuda:0")
        clip = torch.zeros(1, dtype=torch.float32, device="cuda:0")
        banner("llama-7b grad stats: one pre-pass over 291 tensors (one infinity planted)")
        pa.pa_grad_stats_list(gs, s, nf, clip, max_norm=1.0)
        torch.cuda.synchronize()
        assert math.isinf(s.item()) and int(nf.item()) == 1 and clip.item() == 0.0
        gs[k][12345] = 0.0
        banner("llama-7b grad stats: finite gradients")
        pa.pa_grad_stats_list(gs, s, nf, clip, max_norm=1.0)
        torch.cuda.synchronize()
        acc = oracle.SumsqAcc()
        for g in gs:
            oracle.sumsq_add(acc, oracle.DT_F32, to_host(g))
        want = oracle.sumsq_value(acc)
        n = sum(sizes)
        got = s.item()
        assert acc.nonfinite == 0 and int(nf.item()) == 0
        assert abs(got - want) <= (n - 1) * 2.0 ** -53 * want, (got, want)
        c = np.float32(clip.item())
        assert abs(int(c.view(np.int32)) - int(oracle.clip_scale(want, 1.0).view(np.int32))) <= 1
        banner(f"llama-7b grad stats: sumsq {got!r} vs exact {want!r} (rel {abs(got - want) / want:.2e})")
    finally:
        del gs
        torch.cuda.empty_cache()
        pa.pa_release_plans()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("bits,block,group,general,dtype",
                         [(4, 128, 64, False, "fp32"), (3, 128, 64, False, "fp32"), (3, 128, 64, True, "fp32"),
                          (4, 128, 64, False, "bf16")],
                         ids=["default", "3bit", "3bit-general", "bf16"])
def test_llama_7b_turbo_sampled_tensors(pa, bits, block, group, general, dtype):
    """The TurboAdam step over the whole 291-tensor list in the benchmark's
    launch configuration; five whole tensors (tensors are independent: each
    has its own draws, groups, blocks and scales) against the oracle for
    three steps, so that codes written with a nonzero scale are decoded: the
    embedding (131 M values, 256 chunks of residual sums), the first RMSNorm
    gain (FP32 moments), the first query and gate projections, and the final
    norm.  The configurations the benchmark times: the page's defaults and
    3-bit indices on the tuned kernel, 3-bit indices on the general kernel
    (--turbo-general), and bfloat16 parameters and gradients
    (--param-dtype bf16)."""
    import torch
    cfg = 4
    sizes = workloads.sizes(cfg)
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]
    pdt = {"fp32": oracle.DT_F32, "bf16": oracle.DT_BF16}[dtype]

    def host(t):
        return to_host(t).copy() if dtype == "fp32" else to_host(t.view(torch.int16)).view(np.uint16).copy()
    banner(f"llama-7b TurboAdam ({dtype}): allocating params and grads for {sum(sizes) / 1e9:.2f} G values")
    ps = [torch.empty(n, dtype=tdt, device="cuda:0") for n in sizes]
    gs = [torch.empty(n, dtype=tdt, device="cuda:0") for n in sizes]
    states = [pa.TurboState(n, "cuda:0", n >= 4096, n >= 4096, bits, tensor_id=i, block_size=block,
                            m_block_size=group) for i, n in enumerate(sizes)]
    pick = [i for i, (name, _) in enumerate(workloads.shapes(cfg)) if "norm" in name][:1]
    pick += [i for i, (name, _) in enumerate(workloads.shapes(cfg)) if "q_proj" in name][:1]
    pick += [len(sizes) - 2 if "norm" in workloads.shapes(cfg)[-2][0] else len(sizes) - 1]
    pick += [0] + [i for i, (name, _) in enumerate(workloads.shapes(cfg)) if "gate_proj" in name][:1]
    pick = sorted(set(pick))
    try:
        workloads.device_fill_params(cfg, ps)
        tl = pa.TurboList(ps, gs, states, v_bits=bits, block_size=block, m_block_size=group, general=general)
        hp = {i: host(ps[i]) for i in pick}
        hs = {i: oracle.TurboState(sizes[i], sizes[i] >= 4096, sizes[i] >= 4096, bits, block, group) for i in pick}
        for t in (1, 2, 3):
            workloads.device_fill_grads(cfg, t, gs)
            torch.cuda.synchronize()
            hg = {i: host(gs[i]) for i in pick}
            banner(f"llama-7b TurboAdam ({bits} bits, {block}/{group}, general {general}, {dtype}) step {t}: "
                   "one launch over 291 tensors")
            tl.step(dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01), t)
            torch.cuda.synchronize()
            sc = scalars(t)
            ts = oracle.turbo_scalars(0.9, 0.999, t)
            for i in pick:
                oracle.turbo_step_typed(pdt, pdt, hp[i], hg[i], hs[i], sc, ts, t, tensor_id=i)
                st = states[i]
                if hs[i].compress_m:
                    assert np.array_equal(to_host(st.m_codes).view(np.uint32), hs[i].m_codes), f"tensor {i} codes"
                    assert np.array_equal(to_host(st.m_means).view(np.uint16), hs[i].m_means), f"tensor {i} means"
                    assert np.array_equal(to_host(st.scalars).view(np.uint32), hs[i].scal.view(np.uint32))
                    assert np.array_equal(to_host(st.v_index).view(np.uint32), hs[i].v_index), f"tensor {i} index"
                    assert np.array_equal(to_host(st.v_ends).view(np.uint16), hs[i].v_ends), f"tensor {i} ends"
                if dtype == "fp32":
                    assert_params(to_host(ps[i]), hp[i], what=f"tensor {i} params")
                else:
                    assert np.array_equal(host(ps[i]), hp[i]), f"tensor {i} bf16 params"
            banner(f"llama-7b TurboAdam step {t}: tensors {pick} bit-exact")
    finally:
        del ps, gs, states
        torch.cuda.empty_cache()
        pa.pa_release_plans()



def _fill(t, seed, std):
    import torch
    gen = torch.Generator(device="cuda:0").manual_seed(seed)
    step = 1 << 28
    for i in range(0, t.numel(), step):
        t[i:i + step].normal_(0.0, std, generator=gen)


def _gather(t, ranges, dtype=None):
    """Host copy of t over contiguous [a, b) ranges, through slice copies:
    torch's advanced-indexing kernel faults on tensors of more than 2^31
    elements on this stack, so these tests never index such a tensor."""
    return np.concatenate([to_host(t[a:b], dtype) for a, b in ranges])


@pytest.mark.timeout(600)
def test_e4_single_tensor_past_int32(pa):
    """One tensor of 2^31 + 1237 elements (64-bit element indexing, a ragged
    tail), two steps of the packed E4 update; sampled: the first and last
    64 Ki elements, 64 Ki around element 2^31, and 64 seeded 64 Ki tiles."""
    import torch
    n = (1 << 31) + 1237
    banner(f"E4 single tensor of {n} elements: allocating {12 * n / 1e9:.1f} GB")
    p = torch.empty(n, dtype=torch.float32, device="cuda:0")
    g = torch.empty(n, dtype=torch.float32, device="cuda:0")
    w = torch.zeros(n, dtype=torch.int32, device="cuda:0")
    rng = np.random.Generator(np.random.PCG64(2031))
    ranges = [(0, CHUNK), (n - CHUNK, n), ((1 << 31) - CHUNK // 2, (1 << 31) + CHUNK // 2)]
    ranges += [(int(t) * CHUNK, (int(t) + 1) * CHUNK) for t in rng.choice(n // CHUNK, 64, replace=False)]
    try:
        _fill(p, 11, 0.02)
        for t in (1, 2):
            _fill(g, 100 + t, 1e-3)
            torch.cuda.synchronize()
            hp, hg, hw = _gather(p, ranges), _gather(g, ranges), _gather(w, ranges, np.uint32)
            banner(f"E4 single tensor step {t}")
            pa.pa_step(1, p, g, w, hyper(), t)
            torch.cuda.synchronize()
            oracle.step_packed(1, hp, hg, hw, scalars(t))
            assert_words(_gather(w, ranges, np.uint32), hw, what="words")
            same = assert_params(_gather(p, ranges), hp)[0]
            banner(f"E4 single tensor step {t}: {hp.size} sampled elements, bit-identical params {same}")
    finally:
        del p, g, w
        torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_blockwise_single_tensor_past_int32(pa):
    """One blockwise tensor of 2^31 + 5 * 2048 elements (1,048,581 blocks),
    two steps; sampled: the first and last blocks, the two blocks on either
    side of element 2^31, and 60 seeded blocks."""
    import torch
    nb = (1 << 20) + 5
    n = nb * 2048
    qm, qv = workloads.code_maps()
    zero_m = int(np.nonzero(qm == 0.0)[0][0])
    banner(f"blockwise single tensor of {n} elements: allocating {14 * n / 1e9:.1f} GB")
    p = torch.empty(n, dtype=torch.float32, device="cuda:0")
    g = torch.empty(n, dtype=torch.float32, device="cuda:0")
    mc = torch.full((n,), zero_m, dtype=torch.uint8, device="cuda:0")
    vc = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
    ma = torch.zeros(nb, dtype=torch.float32, device="cuda:0")
    va = torch.zeros(nb, dtype=torch.float32, device="cuda:0")
    dqm, dqv = torch.from_numpy(qm).to("cuda:0"), torch.from_numpy(qv).to("cuda:0")
    pout = torch.empty(n, dtype=torch.int16, device="cuda:0")
    rng = np.random.Generator(np.random.PCG64(2032))
    blocks = np.union1d([0, nb - 1, (1 << 20) - 1, 1 << 20], rng.choice(nb, 60, replace=False)).tolist()
    er = [(b * 2048, (b + 1) * 2048) for b in blocks]
    br = [(b, b + 1) for b in blocks]
    try:
        _fill(p, 12, 0.02)
        for t in (1, 2):
            _fill(g, 200 + t, 1e-3)
            torch.cuda.synchronize()
            hp, hg = _gather(p, er), _gather(g, er)
            hmc, hvc = _gather(mc, er).copy(), _gather(vc, er).copy()
            hma, hva = _gather(ma, br).copy(), _gather(va, br).copy()
            banner(f"blockwise single tensor step {t}")
            pa.pa_step(3, p, g, (mc, ma, vc, va, dqm, dqv, pout), hyper(), t)
            torch.cuda.synchronize()
            hout = np.zeros(hp.size, np.uint16)
            oracle.step_blockwise(hp, hg, hmc, hma, hvc, hva, qm, qv, hout, scalars(t))
            assert np.array_equal(_gather(mc, er), hmc) and np.array_equal(_gather(vc, er), hvc), "codes"
            assert np.array_equal(_gather(ma, br).view(np.uint32), hma.view(np.uint32)), "m absmax"
            assert np.array_equal(_gather(va, br).view(np.uint32), hva.view(np.uint32)), "v absmax"
            got = _gather(pout, er).view(np.uint16)
            assert np.array_equal(got, hout), f"{int((got != hout).sum())} bf16 outputs differ"
            widened = (hout.astype(np.uint32) << 16).view(np.float32)
            for k, (a, b) in enumerate(er):             # the next step's parameters, sampled blocks only
                p[a:b].copy_(torch.from_numpy(widened[k * 2048:(k + 1) * 2048]))
            banner(f"blockwise single tensor step {t}: {len(blocks)} sampled blocks bit-exact")
    finally:
        del p, g, mc, vc, ma, va, pout
        torch.cuda.empty_cache()
