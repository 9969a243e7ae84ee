"""TurboAdam compressed-state step (UState + 1Q) through the C ABI against
the oracle, value by value and bit for bit: parameters, 2-bit codes, bf16
means, 1Q indices, fp16 endpoints, tensor scales, and the FP32 moments of
tensors that keep them.  Sizes span tiles, blocks and groups with ragged
tails; lists mix the four representation pairs and the index widths.  Every
layout of the page's fused path runs through the general kernel (blocks of
32 to 1024 values, groups of 1 to 1024, 2 to 8 index bits), and so does the
default layout, against the same oracle."""
import json
import os

import numpy as np
import pytest

import oracle
from gpu_util import assert_params, banner, to_dev, to_host

pytestmark = pytest.mark.gpu

H = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


def _host_words(t, dtype):
    return None if t is None else to_host(t).view(dtype)


def _compare_state(dev, host, what):
    if host.compress_m:
        assert np.array_equal(_host_words(dev.m_codes, np.uint32), host.m_codes), f"{what}: UState codes"
        assert np.array_equal(_host_words(dev.m_means, np.uint16), host.m_means), f"{what}: UState means"
        assert np.array_equal(_host_words(dev.scalars, np.uint32), host.scal.view(np.uint32)), f"{what}: scales"
    else:
        assert np.array_equal(_host_words(dev.m_fp32, np.uint32), host.m_fp32.view(np.uint32)), f"{what}: m"
    if host.compress_v:
        got, want = _host_words(dev.v_index, np.uint32), host.v_index
        diff = np.nonzero(got != want)[0]
        assert diff.size == 0, f"{what}: 1Q index words differ at {diff[:5]}"
        assert np.array_equal(_host_words(dev.v_ends, np.uint16), host.v_ends), f"{what}: 1Q endpoints"
    else:
        assert np.array_equal(_host_words(dev.v_fp32, np.uint32), host.v_fp32.view(np.uint32)), f"{what}: v"


def _run(pa, sizes, flags, bits, steps, seed, grad_scale=1e-3, count=False, block=128, group=64, general=False):
    import torch
    r = np.random.Generator(np.random.PCG64(seed))
    hp = [r.normal(0, 0.02, n).astype(np.float32) for n in sizes]
    dp = [to_dev(a) for a in hp]
    hs = [oracle.TurboState(n, cm, cv, bits, block, group) for n, (cm, cv) in zip(sizes, flags)]
    ds = [pa.TurboState(n, "cuda:0", cm, cv, bits, tensor_id=i, block_size=block, m_block_size=group)
          for i, (n, (cm, cv)) in enumerate(zip(sizes, flags))]
    grads = [torch.zeros(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    tl = pa.TurboList(dp, grads, ds, v_bits=bits, block_size=block, m_block_size=group, general=general)
    hyper = dict(H)
    if count:   # the kernel variant that counts non-finite values (the optimizers' default)
        hyper["nonfinite"] = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    same = total = 0
    for t in range(1, steps + 1):
        hg = [(r.normal(0, 1, n) * grad_scale * 10.0 ** r.uniform(-2, 1)).astype(np.float32) for n in sizes]
        for gdev, g in zip(grads, hg):
            gdev.copy_(torch.from_numpy(g))
        banner(f"turbo bits {bits} block {block} group {group} general {general} sizes {sizes[:5]}.. step {t}")
        tl.step(hyper, t)
        torch.cuda.synchronize()
        if count:
            assert int(hyper["nonfinite"].item()) == 0
        sc = oracle.scalars(H["lr"], H["beta1"], H["beta2"], H["eps"], H["weight_decay"], t)
        ts = oracle.turbo_scalars(H["beta1"], H["beta2"], t)
        for i in range(len(sizes)):
            oracle.turbo_step(hp[i], hg[i], hs[i], sc, ts, t, tensor_id=i)
            _compare_state(ds[i], hs[i], f"step {t} tensor {i} (n={sizes[i]}, flags {flags[i]})")
            s_, _ = assert_params(to_host(dp[i]), hp[i], what=f"step {t} tensor {i} params")
            same += s_
            total += sizes[i]
    banner(f"turbo bits {bits} block {block} group {group}: bit-identical params {same}/{total}")


SIZES = [1, 5, 63, 64, 65, 127, 128, 129, 255, 256, 257, 4096 + 77, 70001]


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_turbo_both_compressed(pa, bits):
    _run(pa, SIZES, [(True, True)] * len(SIZES), bits, steps=4, seed=100 + bits)


def test_turbo_mixed_representations(pa):
    flags = [(True, True), (False, True), (True, False), (False, False)] * 4
    sizes = [3, 300, 4097, 128, 64, 1000, 257, 9, 513, 2048, 7, 65536, 129, 255, 1, 12345]
    _run(pa, sizes, flags, 4, steps=4, seed=7)


@pytest.mark.parametrize("bits,count", [(2, False), (3, False), (4, False), (6, True), (8, False), (4, True),
                                        (8, True)])
def test_turbo_large_list(pa, bits, count):
    """A list of about 27,800 tiles, one wavefront each, more than a full
    grid of the chip holds at once, over sixteen tensors of every
    representation pair with ragged tails: the tensor search of every
    wavefront, the dense index words of the 3- and 6-bit widths across
    blocks and tensor ends, in both kernel variants (with and without the
    non-finite count)."""
    sizes = [1500001, 3, 900017, 129, 1200003, 257, 700007, 65, 1000011, 4097, 800013, 1, 600009, 12345,
             400001, 255]
    flags = [(True, True), (False, True), (True, False), (False, False)] * 4
    assert sum((n + 255) // 256 for n in sizes) > 3 * 256 * 8 * 4
    _run(pa, sizes, flags, bits, steps=3, seed=40 + bits, count=count)


# (index bits, 1Q block, UState group): the widths that straddle words, the
# smallest and largest blocks and groups, and segments of one lane up to
# four wavefronts.
LAYOUTS = [(3, 128, 64), (6, 128, 64), (2, 32, 32), (4, 32, 8), (8, 1024, 1024), (3, 1024, 2), (6, 256, 1),
           (4, 512, 128), (2, 64, 4), (8, 32, 16), (3, 256, 256), (6, 1024, 512)]
LAYOUT_SIZES = [1, 5, 31, 32, 33, 255, 1023, 1024, 1025, 2047, 4096 + 77, 70001]


@pytest.mark.parametrize("bits,block,group", LAYOUTS, ids=lambda x: str(x))
def test_turbo_other_layouts(pa, bits, block, group):
    flags = [(True, True)] * 8 + [(False, True), (True, False), (True, True), (False, False)]
    _run(pa, LAYOUT_SIZES, flags, bits, steps=3, seed=500 + 7 * bits + block + group, block=block, group=group)


@pytest.mark.parametrize("bits,count", [(2, False), (3, False), (4, False), (6, False), (8, False), (4, True)])
def test_turbo_general_kernel_at_default_layout(pa, bits, count):
    """The general kernel forced at the tuned kernel's layout gives the same
    (oracle) results."""
    _run(pa, SIZES, [(True, True)] * len(SIZES), bits, steps=3, seed=600 + bits, count=count, general=True)


@pytest.mark.parametrize("bits,block,group,count", [(3, 128, 64, True), (6, 64, 2, False)])
def test_turbo_general_many_tiles(pa, bits, block, group, count):
    """About 4,300 general-kernel tiles over sixteen tensors of every
    representation pair: the tensor search of each workgroup and the
    residual partial sums of many tiles per tensor."""
    sizes = [1500001, 3, 900017, 129, 1200003, 257, 100007, 65, 300011, 4097, 200013, 1, 60009, 12345, 40001, 255]
    flags = [(True, True), (False, True), (True, False), (False, False)] * 4
    _run(pa, sizes, flags, bits, steps=3, seed=700 + bits, count=count, block=block, group=group)


def test_turbo_large_tensor(pa):
    _run(pa, [1 << 20, 3 * 65536 + 11], [(True, True), (True, True)], 4, steps=3, seed=9)


# (v_bits, block, group, general kernel): the tuned kernel at the defaults,
# the general kernel at the defaults and at a 3-bit, 64/8 layout
PATHS = [(4, 128, 64, False), (4, 128, 64, True), (3, 64, 8, True)]


@pytest.mark.parametrize("bits,block,group,general", PATHS, ids=lambda x: str(x))
def test_turbo_skip_and_scale(pa, bits, block, group, general):
    import torch
    n = 5000
    r = np.random.default_rng(3)
    hp = r.normal(0, 0.02, n).astype(np.float32)
    dp = to_dev(hp)
    hs = oracle.TurboState(n, True, True, bits, block, group)
    ds = pa.TurboState(n, "cuda:0", True, True, bits, block_size=block, m_block_size=group)
    g = to_dev(r.normal(0, 1e-3, n).astype(np.float32))
    tl = pa.TurboList([dp], [g], [ds], v_bits=bits, block_size=block, m_block_size=group, general=general)
    scale = torch.tensor([0.25], dtype=torch.float32, device="cuda:0")
    flag = torch.tensor([1], dtype=torch.int64, device="cuda:0")
    banner("turbo: skipped step")
    tl.step(dict(H, skip_if_nonzero=flag), 1)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(dp), hp) and not to_host(ds.scalars).any()
    flag.zero_()
    for t in (1, 2):
        banner(f"turbo: scaled step {t}")
        tl.step(dict(H, skip_if_nonzero=flag, grad_scale=scale), t)
        torch.cuda.synchronize()
        sc = oracle.scalars(H["lr"], H["beta1"], H["beta2"], H["eps"], H["weight_decay"], t)
        oracle.turbo_step(hp, oracle.scale_grads(0, to_host(g), np.float32(0.25)), hs, sc,
                          oracle.turbo_scalars(H["beta1"], H["beta2"], t), t)
        _compare_state(ds, hs, f"scaled step {t}")
        assert_params(to_host(dp), hp)


def test_turbo_state_bytes_match_page(pa):
    n = 131072
    ds = pa.TurboState(n, "cuda:0")
    assert ds.nbytes() == pa.pa_turbo_state_bytes(1, 1, 4, n) == oracle.turbo_state_bytes(1, 1, 4, n) == 106508


def _same_f32(got, want):
    got, want = np.asarray(got, np.float32), np.asarray(want, np.float32)
    nan = np.isnan(want)
    return np.array_equal(np.isnan(got), nan) and np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def _same_bf16(got, want):
    wide = lambda a: (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)
    return _same_f32(wide(got), wide(want))


@pytest.mark.parametrize("bits,block,group,general", PATHS, ids=lambda x: str(x))
def test_turbo_nonfinite_gradients(pa, bits, block, group, general):
    """NaN and infinite gradients: the 1Q and UState codes follow the
    readings (NaN and zero to index 0 and code 0, +Inf to the top index)
    exactly; floating results compare by NaN class, since a NaN's sign and
    payload are not part of the result."""
    import torch
    sizes = [4096 + 33, 2000]
    flags = [(True, True), (False, False)]
    r = np.random.default_rng(17)
    hp = [r.normal(0, 0.02, n).astype(np.float32) for n in sizes]
    dp = [to_dev(a) for a in hp]
    hs = [oracle.TurboState(n, cm, cv, bits, block, group) for n, (cm, cv) in zip(sizes, flags)]
    ds = [pa.TurboState(n, "cuda:0", cm, cv, bits, tensor_id=i, block_size=block, m_block_size=group)
          for i, (n, (cm, cv)) in enumerate(zip(sizes, flags))]
    grads = [torch.zeros(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    tl = pa.TurboList(dp, grads, ds, v_bits=bits, block_size=block, m_block_size=group, general=general)
    counter = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    total_bad = 0
    for t in (1, 2, 3):
        hg = [(r.normal(0, 1e-3, n)).astype(np.float32) for n in sizes]
        hg[0][[5, 300, 4100]] = [np.nan, np.inf, -np.inf]
        hg[1][[0, 1999]] = [np.inf, np.nan]
        for gdev, g in zip(grads, hg):
            gdev.copy_(torch.from_numpy(g))
        banner(f"turbo non-finite gradients, step {t}")
        tl.step(dict(H, nonfinite=counter), t)
        torch.cuda.synchronize()
        sc = oracle.scalars(H["lr"], H["beta1"], H["beta2"], H["eps"], H["weight_decay"], t)
        ts = oracle.turbo_scalars(H["beta1"], H["beta2"], t)
        for i in range(len(sizes)):
            total_bad += oracle.turbo_step(hp[i], hg[i], hs[i], sc, ts, t, tensor_id=i)
            assert _same_f32(to_host(dp[i]), hp[i]), f"step {t} tensor {i} params"
            st, ho = ds[i], hs[i]
            if ho.compress_m:
                assert np.array_equal(_host_words(st.m_codes, np.uint32), ho.m_codes)
                assert _same_bf16(_host_words(st.m_means, np.uint16), ho.m_means)
                assert _same_f32(to_host(st.scalars), ho.scal)
                assert np.array_equal(_host_words(st.v_index, np.uint32), ho.v_index)
                assert np.array_equal(_host_words(st.v_ends, np.uint16), ho.v_ends)
            else:
                assert _same_f32(to_host(st.m_fp32), ho.m_fp32) and _same_f32(to_host(st.v_fp32), ho.v_fp32)
    assert int(counter.item()) == total_bad > 0


def test_q1_endpoints_every_float(pa):
    """A block's 1Q endpoints (binary16 of log2 rounded down and up, through
    the hardware log2 with an exact fallback) equal the oracle's on every
    positive finite binary32: one-value blocks over all 2^31 - 2^23 - 1."""
    import torch
    top = 0x7F800000
    chunk = 1 << 27
    bad = 0
    for c in range((top + chunk - 1) // chunk):
        lo_bits, hi_bits = max(1, c * chunk), min(top, (c + 1) * chunk)
        banner(f"1Q endpoints chunk {c}: patterns {lo_bits:#x}..{hi_bits:#x}")
        bits = torch.arange(lo_bits, hi_bits, dtype=torch.int64, device="cuda:0")
        x = bits.to(torch.int32).view(torch.float32)
        out = torch.empty(x.numel(), dtype=torch.int32, device="cuda:0")
        pa.pa_debug_q1_ends(x, out)
        torch.cuda.synchronize()
        got = to_host(out).view(np.uint32)
        lo, hi = oracle.q1_ends(to_host(x))
        want = lo.astype(np.uint32) | (hi.astype(np.uint32) << 16)
        diff = np.nonzero(got != want)[0]
        bad += diff.size
        assert diff.size == 0, (f"{diff.size} endpoint pairs differ, first at pattern "
                                f"{lo_bits + int(diff[0]):#x}: {got[diff[0]]:#010x} vs {want[diff[0]]:#010x}")
        del bits, x, out
    assert bad == 0


TIES = json.load(open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                                   "q1_level_ties.json")))["rows"]


def _f16_code(x):
    return int(np.array([x], np.float16).view(np.uint16)[0])


def _endpoint_words(r, n):
    """n random endpoint words, lower <= upper, over every finite fp16 in [-149, 128]."""
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = codes.view(np.float16).astype(np.float64)
    pool = codes[np.isfinite(vals) & (vals >= -149) & (vals <= 128)]
    a, b = r.choice(pool, n), r.choice(pool, n)
    swap = a.view(np.float16) > b.view(np.float16)
    lo, hi = np.where(swap, b, a), np.where(swap, a, b)
    return lo.astype(np.uint32) | (hi.astype(np.uint32) << 16)


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_q1_levels_match_oracle(pa, bits):
    """1Q grid levels (the exact 2^x rounded once to binary32) equal the
    oracle's bit for bit, through the step's own table builders (the device
    exp2, or the geometric recurrence of 8-bit tables, with the
    double-double evaluation near binary32 midpoints) and through the
    double-double evaluation alone: 16M levels of random blocks across
    the whole endpoint range, the committed near-midpoint blocks, one-level
    blocks, and the range ends (+inf at 128, the smallest subnormal at -149)."""
    import torch
    n = {2: 1 << 22, 3: 1 << 21, 4: 1 << 20, 6: 1 << 18, 8: 1 << 16}[bits]
    words = _endpoint_words(np.random.default_rng(40 + bits), n)
    sel = [t for t in TIES if t["bits"] == bits]
    ties = [int(t["lo16"], 16) | (int(t["hi16"], 16) << 16) for t in sel]
    ends = [_f16_code(e) * 0x10001 for e in (-149, -126, -1, 0, 1, 127, 128)]
    ends += [_f16_code(120) | (_f16_code(128) << 16), _f16_code(-149) | (_f16_code(-100) << 16)]
    words = np.concatenate([np.array(ties + ends, np.uint32), words])
    want = oracle.q1_levels_batch(words, bits)
    d_words = to_dev(words)
    for exact in (False, True):
        banner(f"1Q levels: {bits}-bit, {words.size} blocks, exact={exact}")
        out = torch.empty(words.size << bits, dtype=torch.float32, device="cuda:0")
        pa.pa_debug_q1_levels(d_words, bits, exact, out)
        torch.cuda.synchronize()
        got = to_host(out).reshape(words.size, 1 << bits)
        bad = np.argwhere(got.view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, (f"exact={exact}: {len(bad)} levels differ, first block {words[bad[0][0]]:#010x} "
                               f"level {bad[0][1]}: {got[tuple(bad[0])]!r} vs {want[tuple(bad[0])]!r}")
        for j, t in enumerate(sel):
            assert f"{int(got[j, t['k']:t['k'] + 1].view(np.uint32)[0]):08x}" == t["level_hex"], t
        del out


def test_level_rounding_adversarial_exponents(pa):
    """RN32(2^x) on the device, through the 4-bit tables' route and through
    the double-double evaluation alone, equals the oracle's on x whose
    power lies within 2^-56 (some within 2^-64) of a binary32 midpoint, on
    x around the overflow threshold and the subnormal midpoints, and on
    random x over the whole range and past both ends."""
    import torch
    from exact_pow2 import near_midpoint_exponents
    r = np.random.default_rng(13)
    thr = 128.0 + np.log2(1.0 - 2.0 ** -25)
    edges = [thr, 128.0, -150.0, -149.0 + np.log2(1.5), -126.0]
    xs = np.concatenate([near_midpoint_exponents(14), r.uniform(-152, 130, 200000),
                         np.concatenate([[np.nextafter(e, -np.inf), e, np.nextafter(e, np.inf)] for e in edges])])
    want = oracle.exp2_rn32(xs)
    dx = torch.from_numpy(xs).to("cuda:0")
    for exact in (False, True):
        banner(f"pow2 rounding: {xs.size} exponents, exact={exact}")
        out = torch.empty(xs.size, dtype=torch.float32, device="cuda:0")
        pa.pa_debug_pow2_rn32(dx, exact, out)
        torch.cuda.synchronize()
        got = to_host(out)
        bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
        assert bad.size == 0, f"exact={exact}: {bad.size} differ, first x={xs[bad[0]]!r}: {got[bad[0]]!r} vs {want[bad[0]]!r}"


@pytest.mark.parametrize("general", [False, True], ids=["tuned", "general"])
def test_turbo_residual_tree_past_one_chunk_level(pa, general):
    """A UState tensor of 2^30 + 12,345 values has 4,194,353 tile sums and
    2,049 chunk sums, so the scale's tree takes the chunk pass and two
    levels of the per-tensor pass.  The new scale must equal the perfect
    pairwise tree, computed on the host, over the tile sums the step left in
    its workspace: RN32(1.1 * sqrt(sum / n))."""
    import torch
    n = (1 << 30) + 12345
    banner(f"TurboAdam residual tree: one tensor of {n} values")
    gen = torch.Generator(device="cuda:0").manual_seed(77)
    p = torch.randn(n, generator=gen, device="cuda:0") * 0.02
    g = torch.randn(n, generator=gen, device="cuda:0") * 1e-3
    st = pa.TurboState(n, "cuda:0", True, True, 4, tensor_id=5)
    tl = pa.TurboList([p], [g], [st], general=general)
    try:
        tl.step(H, 1)
        torch.cuda.synchronize()
        tiles = (n + 255) // 256
        assert tl.workspace.numel() >= tiles + (tiles + 2047) // 2048
        a = to_host(tl.workspace[:tiles]).astype(np.float64)
        size = 1 << int(np.ceil(np.log2(tiles)))
        a = np.concatenate([a, np.zeros(size - tiles)])
        while a.size > 1:
            a = a[0::2] + a[1::2]
        scal = to_host(st.scalars)
        want = np.float32(1.1 * np.sqrt(a[0] / n))
        banner(f"residual sum {a[0]!r}, scale {scal[1]!r} vs {want!r}")
        assert scal[0] == 0.0 and scal[2] == 0.0
        assert scal[1].view(np.uint32) == want.view(np.uint32)
    finally:
        del p, g, st, tl
        torch.cuda.empty_cache()


def test_turbo_gpt2_layer_7m_list(pa):
    """TurboAdam over the GPT-2-layer list of the page's own benchmark (as
    read from its memory table; the 768-value vectors keep FP32 moments),
    the benchmark's inputs, three steps against the oracle."""
    import torch
    import workloads
    hp = workloads.host_params(6)
    sizes = [a.size for a in hp]
    dp = [to_dev(a) for a in hp]
    hs = [oracle.TurboState(n, n >= 4096, n >= 4096) for n in sizes]
    ds = [pa.TurboState(n, "cuda:0", n >= 4096, n >= 4096, tensor_id=i) for i, n in enumerate(sizes)]
    assert sum(s.nbytes() for s in ds) == 5769288            # the page's figure for UState + 1Q
    grads = [torch.zeros(n, dtype=torch.float32, device="cuda:0") for n in sizes]
    tl = pa.TurboList(dp, grads, ds)
    for t in range(1, 4):
        hg = workloads.host_grads(6, t)
        for gdev, g in zip(grads, hg):
            gdev.copy_(torch.from_numpy(g))
        banner(f"turbo gpt2-layer-7m step {t}")
        tl.step(H, t)
        torch.cuda.synchronize()
        sc = oracle.scalars(H["lr"], H["beta1"], H["beta2"], H["eps"], H["weight_decay"], t)
        ts = oracle.turbo_scalars(H["beta1"], H["beta2"], t)
        for i in range(len(sizes)):
            oracle.turbo_step(hp[i], hg[i], hs[i], sc, ts, t, tensor_id=i)
            _compare_state(ds[i], hs[i], f"step {t} tensor {i}")
            assert_params(to_host(dp[i]), hp[i], what=f"step {t} tensor {i} params")
