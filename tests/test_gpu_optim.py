"""PackedAdamW (torch.optim front end) on the GPU: parity with the oracle,
bit-exact checkpoint resume, and the reference's one-update smoke gates."""
import io

import numpy as np
import pytest

import oracle
from gpu_util import assert_params, assert_words, banner, scalars

pytestmark = pytest.mark.gpu


def _params(torch, sizes, seed):
    g = torch.Generator().manual_seed(seed)
    return [torch.nn.Parameter((torch.randn(n, generator=g) * 0.02).cuda()) for n in sizes]


@pytest.mark.parametrize("mode", ["e4", "fp16", "fp32"])
def test_optimizer_matches_oracle(mode):
    import torch
    from adamw_step_amd.optim import PackedAdamW
    sizes = [3096576, 262144, 768, 256, 65536 + 3]
    ps = _params(torch, sizes, 1)
    hp = [p.detach().cpu().numpy().copy() for p in ps]
    opt = PackedAdamW(ps, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, mode=mode)
    kind = {"e4": 1, "fp16": 2}.get(mode)
    hs = [np.zeros(n, np.uint32) for n in sizes] if kind else \
         [(np.zeros(n, np.float32), np.zeros(n, np.float32)) for n in sizes]
    r = np.random.Generator(np.random.PCG64(3))
    for t in range(1, 4):
        hg = [(r.normal(0, 1e-3, n)).astype(np.float32) for n in sizes]
        for p, g in zip(ps, hg):
            p.grad = torch.from_numpy(g).cuda()
        banner(f"PackedAdamW {mode} step {t}")
        opt.step()
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            if kind:
                oracle.step_packed(kind, hp[i], hg[i], hs[i], scalars(t))
                assert_words(opt.state[ps[i]]["words"].cpu().numpy().view(np.uint32), hs[i], fp16=(kind == 2))
            else:
                oracle.step_fp32(hp[i], hg[i], hs[i][0], hs[i][1], scalars(t))
                assert_words(opt.state[ps[i]]["exp_avg"].cpu().numpy().view(np.uint32), hs[i][0].view(np.uint32))
            assert_params(ps[i].detach().cpu().numpy(), hp[i])
    assert opt.nonfinite_count() == 0
    assert opt.state_bytes() == (8 if mode == "fp32" else 4) * sum(sizes)


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "float16"])
@pytest.mark.parametrize("mode", ["e4", "fp32"])
def test_checkpoint_resume_is_bit_exact(mode, dtype):
    """6 steps straight == 3 steps, save to bytes, load into fresh objects, 3
    steps; with FP32, BF16 and FP16 parameters (the FP32 moments and the
    packed words must come back in their own dtypes)."""
    import torch
    from adamw_step_amd.optim import PackedAdamW
    dt = getattr(torch, dtype)
    sizes = [40000, 4096, 77]
    r = np.random.Generator(np.random.PCG64(8))
    grads = [[torch.from_numpy(r.normal(0, 1e-3, n).astype(np.float32)).to(dt).cuda() for n in sizes]
             for _ in range(6)]

    def run(ps, opt, steps):
        for gs in steps:
            for p, g in zip(ps, gs):
                p.grad = g.clone()
            opt.step()

    def params():
        return [torch.nn.Parameter(p.detach().to(dt)) for p in _params(torch, sizes, 5)]

    a = params()
    oa = PackedAdamW(a, weight_decay=0.01, mode=mode)
    run(a, oa, grads)

    b = params()
    ob = PackedAdamW(b, weight_decay=0.01, mode=mode)
    run(b, ob, grads[:3])
    buf = io.BytesIO()
    torch.save({"params": [p.detach() for p in b], "opt": ob.state_dict()}, buf)
    buf.seek(0)
    ck = torch.load(buf, map_location="cpu", weights_only=True)
    c = [torch.nn.Parameter(t.cuda()) for t in ck["params"]]
    oc = PackedAdamW(c, weight_decay=0.01, mode=mode)
    oc.load_state_dict(ck["opt"])
    assert oc.step_count == 3
    for pc in c:
        for k, t in oc.state[pc].items():
            assert t.dtype == (torch.int32 if k == "words" else torch.float32), (k, t.dtype)
    banner(f"resume {mode} {dtype}: 3 more steps after the round trip")
    run(c, oc, grads[3:])
    torch.cuda.synchronize()
    keys = ["words"] if mode == "e4" else ["exp_avg", "exp_avg_sq"]
    for pa_, pc in zip(a, c):
        assert torch.equal(pa_.detach(), pc.detach())
        for key in keys:
            assert torch.equal(oa.state[pa_][key], oc.state[pc][key])


def test_smoke_gates():
    from trainer.loop import smoke
    banner("trainer smoke: one synthetic update")
    gates, losses, val = smoke()
    assert all(gates.values()), gates


def test_short_training_run():
    import torch
    from trainer.gpt import GPT
    from trainer.loop import Tape, make_optimizer, train
    torch.manual_seed(0)
    model = GPT(layers=2).cuda()
    opt = make_optimizer(model, "e4", lr=3e-3)
    tape = Tape.synthetic(30 * 256 + 1, 12096, seed=3)
    tape.batch, tape.seq = 1, 256
    banner("trainer: 30 synthetic updates")
    losses = train(model, opt, tape, 30, 3e-3, 5, "cuda:0")
    assert all(np.isfinite(losses)) and opt.nonfinite_count() == 0
    # uniformly random tokens carry nothing to learn: the loss stays near ln(vocab)
    assert abs(np.mean(losses[-10:]) - np.log(12096)) < 0.5


def test_optimizer_clipping_matches_oracle():
    """max_grad_norm: the pre-pass coefficient scales every gradient on the
    device; the oracle steps on gradients scaled by that same coefficient,
    and the coefficient itself agrees with the oracle's exact-norm one."""
    import torch
    from adamw_step_amd.optim import PackedAdamW
    sizes = [70000, 4096, 333]
    ps = _params(torch, sizes, 5)
    hp = [p.detach().cpu().numpy().copy() for p in ps]
    hs = [np.zeros(n, np.uint32) for n in sizes]
    opt = PackedAdamW(ps, lr=1e-3, weight_decay=0.01, mode="e4", max_grad_norm=0.5)
    r = np.random.Generator(np.random.PCG64(6))
    for t in range(1, 4):
        hg = [(r.normal(0, 1e-2, n)).astype(np.float32) for n in sizes]
        for p, g in zip(ps, hg):
            p.grad = torch.from_numpy(g).cuda()
        banner(f"PackedAdamW clipped step {t}")
        opt.step()
        torch.cuda.synchronize()
        c = np.float32(opt._clip.item())
        _, bad, want_c = oracle.grad_stats(0, hg, max_norm=0.5)
        assert bad == 0 and c < 1.0
        assert abs(int(c.view(np.int32)) - int(np.float32(want_c).view(np.int32))) <= 1
        assert abs(opt.last_grad_norm() - float(np.sqrt(sum(float(np.dot(g.astype(np.float64), g)) for g in hg)))) \
            <= 1e-9 * opt.last_grad_norm()
        for i in range(len(sizes)):
            oracle.step_packed(1, hp[i], oracle.scale_grads(0, hg[i], c), hs[i], scalars(t))
            assert_words(opt.state[ps[i]]["words"].cpu().numpy().view(np.uint32), hs[i])
            assert_params(ps[i].detach().cpu().numpy(), hp[i])


def test_optimizer_skips_nonfinite_updates():
    """skip_nonfinite: an update whose gradients hold an Inf changes nothing,
    and the following update reuses its step number."""
    import torch
    from adamw_step_amd.optim import PackedAdamW
    sizes = [5000, 64]
    ps = _params(torch, sizes, 9)
    hp = [p.detach().cpu().numpy().copy() for p in ps]
    hs = [np.zeros(n, np.uint32) for n in sizes]
    opt = PackedAdamW(ps, lr=1e-3, weight_decay=0.01, mode="e4", skip_nonfinite=True)
    r = np.random.Generator(np.random.PCG64(10))
    plan = ["ok", "inf", "ok", "nan", "ok"]
    t_oracle = 0
    for kind in plan:
        hg = [(r.normal(0, 1e-3, n)).astype(np.float32) for n in sizes]
        if kind == "inf":
            hg[0][17] = np.inf
        elif kind == "nan":
            hg[1][3] = np.nan
        for p, g in zip(ps, hg):
            p.grad = torch.from_numpy(g).cuda()
        banner(f"PackedAdamW skip test: {kind} gradients")
        opt.step()
        torch.cuda.synchronize()
        if kind == "ok":
            t_oracle += 1
            for i in range(len(sizes)):
                oracle.step_packed(1, hp[i], hg[i], hs[i], scalars(t_oracle))
        for i in range(len(sizes)):
            assert_words(opt.state[ps[i]]["words"].cpu().numpy().view(np.uint32), hs[i])
            assert_params(ps[i].detach().cpu().numpy(), hp[i])
    opt._reconcile()
    assert opt.skipped_steps == 2 and opt.step_count == 3 and opt.nonfinite_count() == 0


def _turbo_oracle_states(sizes, thr=4096, bits=4, block=128, group=64):
    return [oracle.TurboState(n, n >= thr, n >= thr, bits, block, group) for n in sizes]


# (v_bits, block_size, m_block_size): the page's defaults, then two layouts
# of the general kernel
TURBO_LAYOUTS = [(4, 128, 64), (3, 256, 16), (6, 64, 64)]


@pytest.mark.parametrize("bits,block,group", TURBO_LAYOUTS, ids=lambda x: str(x))
def test_turboadam_optimizer_matches_oracle(bits, block, group):
    """TurboAdam front end: three steps of every state word and parameter
    against the oracle; tensors below 4096 values keep FP32 moments."""
    import torch
    from adamw_step_amd.optim import TurboAdam
    sizes = [70000, 4096, 4095, 300, 131072]
    ps = _params(torch, sizes, 21)
    hp = [p.detach().cpu().numpy().copy() for p in ps]
    opt = TurboAdam(ps, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01, v_bits=bits, block_size=block,
                    m_block_size=group)
    hs = _turbo_oracle_states(sizes, bits=bits, block=block, group=group)
    r = np.random.Generator(np.random.PCG64(22))
    for t in range(1, 4):
        hg = [(r.normal(0, 1e-3, n)).astype(np.float32) for n in sizes]
        for p, g in zip(ps, hg):
            p.grad = torch.from_numpy(g).cuda()
        banner(f"TurboAdam step {t}")
        opt.step()
        torch.cuda.synchronize()
        sc = scalars(t)
        ts = oracle.turbo_scalars(0.9, 0.999, t)
        for i in range(len(sizes)):
            oracle.turbo_step(hp[i], hg[i], hs[i], sc, ts, t, tensor_id=i)
            st = opt._states[i]
            if hs[i].compress_m:
                assert np.array_equal(st.m_codes.cpu().numpy().view(np.uint32), hs[i].m_codes)
                assert np.array_equal(st.m_means.cpu().numpy().view(np.uint16), hs[i].m_means)
                assert np.array_equal(st.scalars.cpu().numpy().view(np.uint32), hs[i].scal.view(np.uint32))
                assert np.array_equal(st.v_index.cpu().numpy().view(np.uint32), hs[i].v_index)
                assert np.array_equal(st.v_ends.cpu().numpy().view(np.uint16), hs[i].v_ends)
            else:
                assert np.array_equal(st.m_fp32.cpu().numpy().view(np.uint32), hs[i].m_fp32.view(np.uint32))
                assert np.array_equal(st.v_fp32.cpu().numpy().view(np.uint32), hs[i].v_fp32.view(np.uint32))
            assert_params(ps[i].detach().cpu().numpy(), hp[i])
    assert opt.nonfinite_count() == 0
    n = 131072
    assert opt._states[4].nbytes() == oracle.turbo_state_bytes(1, 1, bits, n, block, group)
    if (bits, block, group) == (4, 128, 64):
        assert opt._states[4].nbytes() == 106508


@pytest.mark.parametrize("bits,block,group", TURBO_LAYOUTS, ids=lambda x: str(x))
def test_turboadam_checkpoint_resume_is_bit_exact(bits, block, group):
    import torch
    from adamw_step_amd.optim import TurboAdam
    lay = dict(v_bits=bits, block_size=block, m_block_size=group)
    sizes = [40000, 5000, 77]
    r = np.random.Generator(np.random.PCG64(23))
    grads = [[torch.from_numpy(r.normal(0, 1e-3, n).astype(np.float32)).cuda() for n in sizes] for _ in range(6)]

    def run(ps, opt, steps):
        for gs in steps:
            for p, g in zip(ps, gs):
                p.grad = g.clone()
            opt.step()

    ps_a = _params(torch, sizes, 24)
    opt_a = TurboAdam(ps_a, lr=1e-3, weight_decay=0.01, **lay)
    banner("TurboAdam checkpoint: six straight steps")
    run(ps_a, opt_a, grads)
    ps_b = _params(torch, sizes, 24)
    opt_b = TurboAdam(ps_b, lr=1e-3, weight_decay=0.01, **lay)
    run(ps_b, opt_b, grads[:3])
    buf = io.BytesIO()
    torch.save({"p": [p.detach().cpu() for p in ps_b], "opt": opt_b.state_dict()}, buf)
    buf.seek(0)
    ck = torch.load(buf, weights_only=True)
    ps_c = [torch.nn.Parameter(t.cuda()) for t in ck["p"]]
    if (block, group) != (128, 64):   # a checkpoint of another layout is refused
        other = TurboAdam([torch.nn.Parameter(t.cuda()) for t in ck["p"]], lr=1e-3, v_bits=bits)
        with pytest.raises(ValueError):
            other.load_state_dict(ck["opt"])
    opt_c = TurboAdam(ps_c, lr=1e-3, weight_decay=0.01, **lay)
    opt_c.load_state_dict(ck["opt"])
    banner("TurboAdam checkpoint: three steps, save, load, three steps")
    run(ps_c, opt_c, grads[3:])
    torch.cuda.synchronize()
    for a, c in zip(ps_a, ps_c):
        assert torch.equal(a.detach(), c.detach())
    for sa, sc_ in zip(opt_a._states, opt_c._states):
        for ta, tc in zip(sa.tensors(), sc_.tensors()):
            assert torch.equal(ta, tc)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_turboadam_16bit_parameters_match_oracle_and_resume(dtype):
    """TurboAdam over bfloat16 or float16 parameters (the TurboAdam package
    page's tests run fp16, bf16 and fp32 parameters), gradients of the same
    type, as torch's autograd leaves them: three steps against the oracle's
    typed step, every state word and every 16-bit parameter bit for bit, then
    a checkpoint written and restored mid-run continues bit for bit, the
    packed codes keeping their dtypes."""
    import torch
    from adamw_step_amd.optim import TurboAdam
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    pdt = {"bf16": oracle.DT_BF16, "fp16": oracle.DT_F16}[dtype]
    sizes = [70000, 4096, 4095, 300]
    r = np.random.Generator(np.random.PCG64(71))
    ps = [torch.nn.Parameter(torch.from_numpy(r.normal(0, 0.02, n).astype(np.float32)).to(tdt).cuda())
          for n in sizes]
    hp = [p.detach().cpu().view(torch.int16).numpy().view(np.uint16).copy() for p in ps]
    opt = TurboAdam(ps, lr=1e-3, weight_decay=0.01)
    hs = _turbo_oracle_states(sizes)
    grads = [[torch.from_numpy(r.normal(0, 1e-3, n).astype(np.float32)).to(tdt).cuda() for n in sizes]
             for _ in range(6)]
    for t in range(1, 4):
        for p, g in zip(ps, grads[t - 1]):
            p.grad = g.clone()
        banner(f"TurboAdam {dtype} step {t}")
        opt.step()
        torch.cuda.synchronize()
        sc = scalars(t)
        ts = oracle.turbo_scalars(0.9, 0.999, t)
        for i in range(len(sizes)):
            hg = grads[t - 1][i].cpu().view(torch.int16).numpy().view(np.uint16).copy()
            oracle.turbo_step_typed(pdt, pdt, hp[i], hg, hs[i], sc, ts, t, tensor_id=i)
            got = ps[i].detach().cpu().view(torch.int16).numpy().view(np.uint16)
            assert np.array_equal(got, hp[i]), f"step {t} tensor {i}: 16-bit parameters"
            st = opt._states[i]
            if hs[i].compress_m:
                assert np.array_equal(st.m_codes.cpu().numpy().view(np.uint32), hs[i].m_codes)
                assert np.array_equal(st.v_index.cpu().numpy().view(np.uint32), hs[i].v_index)
                assert np.array_equal(st.scalars.cpu().numpy().view(np.uint32), hs[i].scal.view(np.uint32))
            else:
                assert np.array_equal(st.m_fp32.cpu().numpy().view(np.uint32), hs[i].m_fp32.view(np.uint32))
    assert opt.nonfinite_count() == 0
    buf = io.BytesIO()
    torch.save({"p": [p.detach().cpu() for p in ps], "opt": opt.state_dict()}, buf)
    buf.seek(0)
    ck = torch.load(buf, weights_only=True)
    ps_c = [torch.nn.Parameter(t.cuda()) for t in ck["p"]]
    opt_c = TurboAdam(ps_c, lr=1e-3, weight_decay=0.01)
    opt_c.load_state_dict(ck["opt"])
    for sa, sc_ in zip(opt._states, opt_c._states):
        for ta, tc in zip(sa.tensors(), sc_.tensors()):
            assert ta.dtype == tc.dtype and torch.equal(ta, tc)
    for run_ps, run_opt in ((ps, opt), (ps_c, opt_c)):
        for gs in grads[3:]:
            for p, g in zip(run_ps, gs):
                p.grad = g.clone()
            run_opt.step()
    torch.cuda.synchronize()
    for a, c in zip(ps, ps_c):
        assert a.dtype == tdt and torch.equal(a.detach(), c.detach())
    for sa, sc_ in zip(opt._states, opt_c._states):
        for ta, tc in zip(sa.tensors(), sc_.tensors()):
            assert torch.equal(ta, tc)
