"""Parameter groups in both optimizers (the TurboAdam package page's API takes
"parameters or parameter groups"): each group its own lr, betas, eps and
weight decay, one launch per group, every group on the same step number.
PackedAdamW's gradient pre-pass runs over the gradients of every group, so
clipping uses the global norm and a non-finite gradient in one group skips
the update of all.  Every state word and parameter against the oracle, and
checkpoints of grouped optimizers resume bit for bit."""
import io

import numpy as np
import pytest

import oracle
from gpu_util import assert_params, assert_words, banner

pytestmark = pytest.mark.gpu


def _params(torch, sizes, seed):
    r = np.random.Generator(np.random.PCG64(seed))
    return [torch.nn.Parameter(torch.from_numpy(r.normal(0, 0.02, n).astype(np.float32)).cuda()) for n in sizes]


GROUPS = [dict(lr=1e-3, weight_decay=0.1), dict(lr=3e-3, weight_decay=0.0, betas=(0.8, 0.99), eps=1e-6)]


def _full(g):
    return dict(lr=g["lr"], betas=g.get("betas", (0.9, 0.999)), eps=g.get("eps", 1e-8),
                weight_decay=g["weight_decay"])


def _sc(g, t):
    f = _full(g)
    return oracle.scalars(f["lr"], f["betas"][0], f["betas"][1], f["eps"], f["weight_decay"], t)


def test_packed_groups_global_clip_skip_and_resume():
    import torch
    from adamw_step_amd.optim import PackedAdamW
    sizes = [[70000, 4096], [333, 64, 5000]]
    ps = [_params(torch, s, 80 + k) for k, s in enumerate(sizes)]
    flat = [p for grp in ps for p in grp]
    hp = [p.detach().cpu().numpy().copy() for p in flat]
    hs = [np.zeros(p.numel(), np.uint32) for p in flat]
    gid = [k for k, s in enumerate(sizes) for _ in s]

    def make(plist):
        return PackedAdamW([dict(params=grp, **GROUPS[k]) for k, grp in enumerate(plist)], mode="e4",
                           max_grad_norm=0.5, skip_nonfinite=True)
    opt = make(ps)
    r = np.random.Generator(np.random.PCG64(81))
    plan = ["ok", "ok", "inf", "ok", "ok"]
    grads_by_step = []
    t_oracle = 0
    for s, kind in enumerate(plan):
        hg = [(r.normal(0, 1e-2, p.numel())).astype(np.float32) for p in flat]
        if kind == "inf":
            hg[3][7] = np.inf                       # in the second group only
        grads_by_step.append(hg)
        for p, g in zip(flat, hg):
            p.grad = torch.from_numpy(g).cuda()
        banner(f"PackedAdamW groups: update {s} ({kind})")
        opt.step()
        torch.cuda.synchronize()
        if kind == "ok":
            t_oracle += 1
            _, bad, want_c = oracle.grad_stats(0, hg, max_norm=0.5)   # the norm over both groups
            c = np.float32(opt._clip.item())
            assert bad == 0 and abs(int(c.view(np.int32)) - int(np.float32(want_c).view(np.int32))) <= 1
            for i in range(len(flat)):
                oracle.step_packed(1, hp[i], oracle.scale_grads(0, hg[i], c), hs[i], _sc(GROUPS[gid[i]], t_oracle))
        for i, p in enumerate(flat):
            assert_words(opt.state[p]["words"].cpu().numpy().view(np.uint32), hs[i], what=f"update {s} tensor {i}")
            assert_params(p.detach().cpu().numpy(), hp[i], what=f"update {s} tensor {i}")
        if s == 1:
            buf = io.BytesIO()
            torch.save({"p": [p.detach().cpu() for p in flat], "opt": opt.state_dict()}, buf)
    opt._reconcile()
    assert opt.skipped_steps == 1 and opt.step_count == 4
    # resume from the checkpoint taken after update 1 and replay updates 2..4
    buf.seek(0)
    ck = torch.load(buf, weights_only=True)
    it = iter(ck["p"])
    ps_c = [[torch.nn.Parameter(next(it).cuda()) for _ in grp] for grp in ps]
    flat_c = [p for grp in ps_c for p in grp]
    opt_c = make(ps_c)
    opt_c.load_state_dict(ck["opt"])
    assert [g["lr"] for g in opt_c.param_groups] == [g["lr"] for g in opt.param_groups]
    for hg in grads_by_step[2:]:
        for p, g in zip(flat_c, hg):
            p.grad = torch.from_numpy(g).cuda()
        opt_c.step()
    torch.cuda.synchronize()
    for a, b in zip(flat, flat_c):
        assert torch.equal(a.detach(), b.detach())
        assert torch.equal(opt.state[a]["words"], opt_c.state[b]["words"])


def test_turbo_groups_match_oracle_and_add_group():
    import torch
    from adamw_step_amd.optim import TurboAdam
    sizes = [[70000, 4095], [5000, 300]]
    ps = [_params(torch, s, 90 + k) for k, s in enumerate(sizes)]
    opt = TurboAdam([dict(params=grp, **GROUPS[k]) for k, grp in enumerate(ps)])
    late = _params(torch, [9000], 93)
    flat = [p for grp in ps for p in grp]
    hp = [p.detach().cpu().numpy().copy() for p in flat]
    hs = [oracle.TurboState(p.numel(), p.numel() >= 4096, p.numel() >= 4096) for p in flat]
    gid = [k for k, s in enumerate(sizes) for _ in s]
    r = np.random.Generator(np.random.PCG64(94))
    for t in range(1, 5):
        if t == 3:      # a group added between updates: new tensor ids, its own first step
            opt.add_param_group(dict(params=late, lr=2e-3, weight_decay=0.05))
            flat.append(late[0])
            hp.append(late[0].detach().cpu().numpy().copy())
            hs.append(oracle.TurboState(9000))
            gid.append(2)
        hg = [(r.normal(0, 1e-3, p.numel())).astype(np.float32) for p in flat]
        for p, g in zip(flat, hg):
            p.grad = torch.from_numpy(g).cuda()
        banner(f"TurboAdam groups: step {t}")
        opt.step()
        torch.cuda.synchronize()
        groups = GROUPS + [dict(lr=2e-3, weight_decay=0.05)]
        for i in range(len(flat)):
            g = _full(groups[gid[i]])
            ts = oracle.turbo_scalars(g["betas"][0], g["betas"][1], t)
            oracle.turbo_step(hp[i], hg[i], hs[i], _sc(groups[gid[i]], t), ts, t, tensor_id=i)
            st = opt.state[flat[i]]["turbo"]
            assert st.tensor_id == i
            if hs[i].compress_m:
                assert np.array_equal(st.m_codes.cpu().numpy().view(np.uint32), hs[i].m_codes)
                assert np.array_equal(st.scalars.cpu().numpy().view(np.uint32), hs[i].scal.view(np.uint32))
                assert np.array_equal(st.v_index.cpu().numpy().view(np.uint32), hs[i].v_index)
            else:
                assert np.array_equal(st.m_fp32.cpu().numpy().view(np.uint32), hs[i].m_fp32.view(np.uint32))
            assert_params(flat[i].detach().cpu().numpy(), hp[i], what=f"step {t} tensor {i}")
    assert opt.nonfinite_count() == 0
    # the page's beta rule holds per group, at construction and when a group is added
    with pytest.raises(ValueError):
        TurboAdam([dict(params=_params(torch, [10], 95)), dict(params=_params(torch, [10], 96), betas=(0.99, 0.98))])
    n_groups = len(opt.param_groups)
    with pytest.raises(ValueError):
        opt.add_param_group(dict(params=_params(torch, [10], 97), betas=(0.99, 0.98)))
    assert len(opt.param_groups) == n_groups
