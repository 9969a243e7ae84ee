"""Both launches of the blockwise 8-bit step against the oracle.

The persistent launch builds the search tables in every workgroup; the
ordered launch builds them once per tensor into a device buffer the library
keeps per stream and gives each workgroup K consecutive blocks in dispatch
order.  Which one runs is chosen by size; here pa_debug_blockwise_path
forces each (persistent, and ordered at K = 1, 5 and 12) on a list of three
tensors of 1, 37 and 301 blocks (partial last groups for every K), the
middle one with other maps than its neighbours so that consecutive tensors
rebuild the stream's shared buffer.  Three steps each, with NaN and Inf
planted in the gradients; the plain, counting and gradient-scaling kernels.
Codes, absmax values and BF16 output bit for bit against the oracle, the
non-finite count equal to the oracle's."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_util import banner, hyper, scalars, to_dev, to_host

pytestmark = pytest.mark.gpu

BW = 3
BLOCKS = [1, 37, 301]
SCALE = np.float32(0.37)


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


@pytest.fixture
def path(pa, request):
    pa.blockwise_path(request.param)
    yield request.param
    pa.blockwise_path(0)


def _maps(i):
    if i == 1:
        return np.linspace(-1, 1, 256).astype(np.float32), np.linspace(0, 1, 256).astype(np.float32)
    return workloads.code_maps()


def _nan_bf16(x):
    return ((x & 0x7F80) == 0x7F80) & ((x & 0x7F) != 0)


@pytest.mark.parametrize("variant", ["plain", "count", "scale"])
@pytest.mark.parametrize("path", [-1, 1, 5, 12], indirect=True, ids=["persistent", "k1", "k5", "k12"])
def test_blockwise_launches(pa, path, variant):
    import torch
    r = np.random.Generator(np.random.PCG64(1200 + path))
    host, dev = [], []
    for i, nb in enumerate(BLOCKS):
        n = nb * 2048
        qm, qv = _maps(i)
        h = dict(p=r.normal(0, 0.02, n).astype(np.float32), mc=np.zeros(n, np.uint8), vc=np.zeros(n, np.uint8),
                 ma=np.zeros(nb, np.float32), va=np.zeros(nb, np.float32), qm=qm, qv=qv, out=np.zeros(n, np.uint16))
        h["mc"][:] = int(np.argmin(np.abs(qm)))       # decodes to 0 while the absmax is 0
        host.append(h)
        dev.append(dict(p=to_dev(h["p"]), st=(torch.from_numpy(h["mc"].copy()).cuda(), to_dev(h["ma"]),
                                              torch.from_numpy(h["vc"].copy()).cuda(), to_dev(h["va"]),
                                              to_dev(qm), to_dev(qv),
                                              torch.zeros(n, dtype=torch.int16, device="cuda:0"))))
    counter = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    scale = torch.tensor([SCALE], dtype=torch.float32, device="cuda:0")
    kw = {"count": dict(nonfinite=counter), "scale": dict(grad_scale=scale)}.get(variant, {})
    want_bad = 0
    for t in (1, 2, 3):
        gs = []
        for i, nb in enumerate(BLOCKS):
            g = (r.normal(0, 1e-3, nb * 2048) * np.repeat(10.0 ** r.uniform(-2, 1, nb), 2048)).astype(np.float32)
            if t == 2 and i == 2:
                g[200 * 2048 + 5] = np.nan
            if t == 3 and i == 1:
                g[36 * 2048 + 2047] = -np.inf
            gs.append(g)
        banner(f"blockwise launch {path}, {variant}, step {t}")
        pa.pa_step_list(BW, [d["p"] for d in dev], [to_dev(g) for g in gs], [d["st"] for d in dev],
                        hyper(**kw), t)
        torch.cuda.synchronize()
        for i, (h, d) in enumerate(zip(host, dev)):
            g = oracle.scale_grads(0, gs[i], SCALE) if variant == "scale" else gs[i]
            want_bad += oracle.step_blockwise(h["p"], g, h["mc"], h["ma"], h["vc"], h["va"], h["qm"], h["qv"],
                                              h["out"], scalars(t))
            mc, ma, vc, va, _, _, out = d["st"]
            got = to_host(out, np.uint16)
            assert np.array_equal(_nan_bf16(got), _nan_bf16(h["out"])), f"step {t} tensor {i}: NaN outputs"
            keep = ~_nan_bf16(h["out"])
            assert np.array_equal(got[keep], h["out"][keep]), f"step {t} tensor {i}: BF16 output"
            assert np.array_equal(to_host(mc), h["mc"]), f"step {t} tensor {i}: m codes"
            assert np.array_equal(to_host(vc), h["vc"]), f"step {t} tensor {i}: v codes"
            for gd, want in ((to_host(ma), h["ma"]), (to_host(va), h["va"])):
                nan = np.isnan(want)
                assert np.array_equal(np.isnan(gd), nan), f"step {t} tensor {i}: NaN absmax"
                assert np.array_equal(gd[~nan].view(np.uint32), want[~nan].view(np.uint32)), f"step {t} tensor {i}"
            # the BF16 output, widened (exact), is the next step's FP32 parameters on both sides
            p = (h["out"].astype(np.uint32) << 16).view(np.float32)
            h["p"] = np.where(np.isnan(p), np.float32(0), p).astype(np.float32)
            d["p"] = to_dev(h["p"])
    if variant == "count":
        assert want_bad > 0 and int(counter.item()) == want_bad
