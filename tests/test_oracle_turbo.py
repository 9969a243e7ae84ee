"""Pins of the oracle's TurboAdam state (UState first moment, 1Q second
moment) against what the page prints and what mathematics and independent
libraries fix: Philox4x32-10's published known-answer vectors and Triton's
own philox (run by its CPU interpreter), numpy's binary16, a 60-digit decimal
power of two (the grid levels), torch's bfloat16 cast, math.fsum, the plain FP32 AdamW oracle (the uncompressed
identity), closed forms, and the unbiasedness of stochastic rounding over a
fine grid of draws.

The page leaves the code levels, the endpoint rule, the scale rule and the
hash unprinted; those readings are parity unpinned (the tests below pin the
oracle to them, not them to the page)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from exact_pow2 import grid_x as _grid_x, near_midpoint_exponents, rn32_pow2 as _rn32_pow2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FACTS = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_facts.json")))["turboadam_state"]


KAT = json.load(open(os.path.join(ROOT, "tests", "golden", "philox4x32_10_kat.json")))["vectors"]


@pytest.mark.parametrize("case", KAT, ids=["zeros", "ones", "pi"])
def test_philox_known_answers(oracle_mod, case):
    def words(xs):
        return [int(x, 16) for x in xs]
    assert oracle.philox4x32(words(case["counter"]), words(case["key"])).tolist() == words(case["out"])


_TRITON_PHILOX = r"""
import os, sys, json
os.environ["TRITON_INTERPRET"] = "1"
import numpy as np, torch, triton, triton.language as tl

@triton.jit
def draw(out, seed, c0p, c1p, c2p, c3p, N: tl.constexpr):
    i = tl.arange(0, N)
    a, b, c, d = tl.philox(seed, tl.load(c0p + i), tl.load(c1p + i), tl.load(c2p + i), tl.load(c3p + i), 10)
    tl.store(out + 4 * i, a)
    tl.store(out + 4 * i + 1, b)
    tl.store(out + 4 * i + 2, c)
    tl.store(out + 4 * i + 3, d)

spec = json.loads(sys.argv[1])
ctr = np.array(spec["counters"], np.uint64)
out = torch.zeros(4 * len(ctr), dtype=torch.int64)
cols = [torch.tensor(ctr[:, j].astype(np.int64)).to(torch.uint32) for j in range(4)]
draw[(1,)](out, spec["seed"], *cols, N=len(ctr))
print(json.dumps((out.numpy().astype(np.uint64) & 0xFFFFFFFF).reshape(-1, 4).tolist()))
"""


def test_philox_matches_triton(oracle_mod):
    """The draws are Triton's tl.philox(seed, j, step, tensor id, stream):
    the counter hash a Triton path and a PyTorch path can share."""
    pytest.importorskip("triton")
    import subprocess
    import sys
    seed = 0x9E3779B97F4A7C15
    rng = np.random.default_rng(11)
    ctr = rng.integers(0, 2 ** 32, size=(8, 4), dtype=np.uint64)
    ctr[0] = [0, 1, 0, 0]
    ctr[1] = [0xFFFFFFFF, 0xFFFFFFFF, 7, 1]
    spec = json.dumps({"seed": seed, "counters": ctr.tolist()})
    env = dict(os.environ, TRITON_INTERPRET="1")
    res = subprocess.run([sys.executable, "-c", _TRITON_PHILOX, spec], capture_output=True, text=True, env=env,
                         timeout=600)
    if res.returncode != 0:
        pytest.skip(f"triton interpreter unavailable: {res.stderr.strip().splitlines()[-1:]}")
    got = json.loads(res.stdout.strip().splitlines()[-1])
    key = [seed & 0xFFFFFFFF, seed >> 32]
    for c, w in zip(ctr, got):
        assert oracle.philox4x32(c, key).tolist() == w


def test_state_ledger_matches_page(oracle_mod):
    n = FACTS["values"]
    ustate = oracle.turbo_state_bytes(1, 0, 4, n) - 4 * n
    oneq = oracle.turbo_state_bytes(0, 1, 4, n) - 4 * n
    total = oracle.turbo_state_bytes(1, 1, 4, n)
    assert (ustate, oneq, total) == (FACTS["ustate_bytes"], FACTS["oneq_bytes"], FACTS["total_bytes"])
    assert round(total * 8 / n, 6) == FACTS["bits_per_value"]
    assert round(8 * n / total, 3) == FACTS["vs_two_fp32_moments"]
    assert oracle.turbo_state_bytes(0, 0, 4, n) == 8 * n


@pytest.mark.parametrize("n", [1, 129, 4096, 5003])
def test_uncompressed_is_exact_adamw(oracle_mod, n):
    """Both representations off: the step is the plain FP32 AdamW step, bit for bit."""
    r = np.random.default_rng(n)
    p0 = r.normal(0, 0.02, n).astype(np.float32)
    pa, pb = p0.copy(), p0.copy()
    st = oracle.TurboState(n, compress_m=False, compress_v=False)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    for t in range(1, 6):
        g = r.normal(0, 1e-3, n).astype(np.float32)
        sc = oracle.scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, t)
        oracle.turbo_step(pa, g, st, sc, oracle.turbo_scalars(0.9, 0.999, t), t)
        oracle.step_fp32(pb, g, m, v, sc)
        assert np.array_equal(pa.view(np.uint32), pb.view(np.uint32))
        assert np.array_equal(st.m_fp32.view(np.uint32), m.view(np.uint32))
        assert np.array_equal(st.v_fp32.view(np.uint32), v.view(np.uint32))


def _f16_bits(x):
    return int(np.array([x], np.float16).view(np.uint16)[0])



def test_q1_endpoints_and_levels(oracle_mod):
    r = np.random.default_rng(4)
    for bits in (2, 3, 4, 6, 8):
        for length in (128, 32, 1024):
            if length != 128 and bits in (2, 4, 8):
                continue
            v = (10.0 ** r.uniform(-14, 0, length)).astype(np.float32)
            idx, ends, dec = oracle.q1_block(v, bits, r.random(length).astype(np.float32))
            lo, hi = (float(np.array(ends[k:k + 1]).view(np.float16)[0]) for k in (0, 1))
            l2min, l2max = math.log2(float(v.min())), math.log2(float(v.max()))
            # lo is the largest binary16 at or below log2(min), hi the smallest at or above log2(max)
            assert lo <= l2min and float(np.nextafter(np.float16(lo), np.float16(np.inf))) > l2min
            assert hi >= l2max and float(np.nextafter(np.float16(hi), np.float16(-np.inf))) < l2max
            lev = oracle.q1_levels(ends[0], ends[1], bits)
            L = 1 << bits
            want = [np.float32(0)] + [_rn32_pow2(_grid_x(lo, hi, k, L))[0] for k in range(1, L)]
            assert np.array_equal(lev, np.array(want, np.float32))
            assert lev[1] <= v.min() and lev[-1] >= v.max()
            assert np.all(np.diff(lev[1:]) >= 0)
            assert np.array_equal(dec, lev[idx])
            # each value lands on one of its two bracketing levels
            for x, k in zip(v, idx):
                assert lev[k] == x or (k > 1 and lev[k - 1] < x < lev[k]) or (k < L - 1 and lev[k] < x < lev[k + 1])


TIES = json.load(open(os.path.join(ROOT, "tests", "golden", "q1_level_ties.json")))


def _f16(code):
    return float(np.array([code], np.uint16).view(np.float16)[0])


@pytest.mark.parametrize("row", TIES["rows"], ids=lambda r: f"{r['lo16']}-{r['hi16']}-{r['bits']}-{r['k']}")
def test_q1_level_near_midpoint(oracle_mod, row):
    """Levels whose power of two lies within 2^-47 of a binary32 midpoint: the
    stored oracle level is the exact power rounded once (a double exp2 with a
    one-ulp error may round these to the other side)."""
    lo16, hi16, bits, k = int(row["lo16"], 16), int(row["hi16"], 16), row["bits"], row["k"]
    x = _grid_x(_f16(lo16), _f16(hi16), k, 1 << bits)
    want, dist = _rn32_pow2(x)
    assert dist < 2.0 ** -47
    assert f"{int(np.array([want]).view(np.uint32)[0]):08x}" == row["level_hex"]
    lev = oracle.q1_levels(lo16, hi16, bits)
    assert lev[k] == want


def test_q1_levels_exact_powers_and_range_ends(oracle_mod):
    """Integer exponents give exact powers of two; lo = hi gives one level;
    the grid's top at 128 is +inf and its bottom at -149 the smallest
    subnormal; random endpoint pairs across the whole range match the exact
    power."""
    for e in (-149, -126, -1, 0, 1, 127):
        lev = oracle.q1_levels(_f16_bits(e), _f16_bits(e), 4)
        assert lev[0] == 0 and np.all(lev[1:] == np.float32(2.0 ** e))
    lev = oracle.q1_levels(_f16_bits(120.0), _f16_bits(128.0), 2)
    assert lev[3] == np.inf and lev[2] == np.float32(2.0 ** 124) and lev[1] == np.float32(2.0 ** 120)
    lev = oracle.q1_levels(_f16_bits(-149.0), _f16_bits(-133.0), 4)
    assert lev[1] == np.float32(2.0 ** -149)
    r = np.random.default_rng(12)
    for _ in range(60):
        a, b = np.sort(r.uniform(-149, 128, 2)).astype(np.float16)
        bits = int(r.choice([2, 4, 8]))
        L = 1 << bits
        lev = oracle.q1_levels(_f16_bits(a), _f16_bits(b), bits)
        for k in r.integers(1, L, 4):
            assert lev[k] == _rn32_pow2(_grid_x(float(a), float(b), int(k), L))[0], (a, b, bits, k)


def test_level_rounding_within_2m56_of_midpoints(oracle_mod):
    """The level rounding RN32(2^x) on x whose power lies within 2^-56 of a
    binary32 midpoint, where the 64-bit-significand exp2l cannot decide and
    the oracle takes its binary128 branch: every one equals the decimal
    arbiter (about a thousand, some within 2^-64)."""
    xs = near_midpoint_exponents(11)
    res = [_rn32_pow2(float(x)) for x in xs]
    close = np.array([d < 2.0 ** -56 for _, d in res])
    assert close.sum() > 500 and min(d for _, d in res) < 2.0 ** -64
    want = np.array([v for v, _ in res], np.float32)
    got = oracle.exp2_rn32(xs)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_q1_special_values(oracle_mod):
    v = np.array([0.0, -0.0, np.nan, np.inf, 1e-3, 2e-3, 0.0, 4e-3], np.float32)
    idx, ends, dec = oracle.q1_block(v, 4, np.full(v.size, 0.5, np.float32))
    assert list(idx[[0, 1, 2, 6]]) == [0, 0, 0, 0] and idx[3] == 15
    assert dec[0] == 0.0 and dec[3] == oracle.q1_levels(ends[0], ends[1], 4)[15]
    idx, ends, dec = oracle.q1_block(np.zeros(7, np.float32), 4, np.zeros(7, np.float32))
    assert not idx.any() and not dec.any() and not ends.any()
    # powers of two inside an exact grid: log2 values exact, so the values are levels themselves
    v = np.array([0.25, 1.0, 4.0, 0.5, 2.0], np.float32)
    idx, ends, dec = oracle.q1_block(v, 2, np.full(5, 0.999, np.float32))
    assert ends[0] == _f16_bits(-2.0) and ends[1] == _f16_bits(2.0)
    assert list(idx[:3]) == [1, 2, 3] and np.array_equal(dec[:3], v[:3])


def test_q1_rounding_is_unbiased(oracle_mod):
    """Over a fine, even grid of draws the mean decoded value is the input:
    exact up to the grid's resolution."""
    r = np.random.default_rng(6)
    v = (10.0 ** r.uniform(-10, -4, 100)).astype(np.float32)
    N = 4096
    acc = np.zeros(v.size, np.float64)
    for j in range(N):
        _, _, dec = oracle.q1_block(v, 4, np.full(v.size, (j + 0.5) / N, np.float32))
        acc += dec
    _, ends, _ = oracle.q1_block(v, 4, np.zeros(v.size, np.float32))
    lev = oracle.q1_levels(ends[0], ends[1], 4).astype(np.float64)
    step = np.array([np.diff(lev[1:]).max()] * v.size)
    assert np.all(np.abs(acc / N - v) <= step / N * 2 + 1e-12 * v)


def test_ustate_mean_codes_and_recentering(oracle_mod):
    import torch
    r = np.random.default_rng(8)
    for _ in range(30):
        n = int(r.integers(1, 65))
        q = (r.normal(0, 1, n) * 10.0 ** r.uniform(-2, 1)).astype(np.float32)
        s = np.float32(10.0 ** r.uniform(-2, 1))
        u = r.random((n + 1) // 2).astype(np.float32)
        codes, mean16, r2 = oracle.ustate_group(q, s, u)
        exact_mean = math.fsum(float(x) for x in q) / n
        want16 = int(torch.tensor([float(np.float32(exact_mean))]).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        assert mean16 == want16
        mean = float((np.array([mean16], np.uint32) << 16).view(np.float32)[0])
        res = q - np.float32(mean)
        assert np.array_equal(r2, res.astype(np.float64) ** 2)
        lv = np.array([-1.5, -0.5, 0.5, 1.5])
        x = np.clip(res / s, -1.5, 1.5)
        # each code is one of the two levels around x (or x's own level)
        for xi, c in zip(x, codes):
            assert lv[c] == xi or abs(lv[c] - xi) < 1.0
        dec = oracle.ustate_decode(codes, mean16, s)
        # decoded values: mean + s * (level - mean level); their mean is the stored mean
        lbar = lv[codes].sum() / n
        assert np.allclose(dec, np.float32(mean) + s * (lv[codes] - lbar), rtol=0, atol=4e-7 * (abs(mean) + 2 * s))
        assert abs(dec.astype(np.float64).mean() - mean) <= 4e-7 * (abs(mean) + 2 * s) + 1e-30


def test_ustate_antithetic_pairs(oracle_mod):
    """A pair of equal values with draws u and 1-u moves up by floor(2f) or ceil(2f) steps in total."""
    r = np.random.default_rng(9)
    for _ in range(500):
        x = np.float32(r.uniform(-1.5, 1.5))
        q = np.array([x, x], np.float32)
        codes, mean16, _ = oracle.ustate_group(q, 1.0, np.array([r.random()], np.float32))
        mean = float((np.array([mean16], np.uint32) << 16).view(np.float32)[0])
        xr = float(np.float32(np.float32(x) - np.float32(mean)))
        k = int(xr >= -0.5) + int(xr >= 0.5)
        f = xr - [-1.5, -0.5, 0.5, 1.5][k]
        ups = int(codes[0] > k) + int(codes[1] > k)
        assert math.floor(2 * f) <= ups <= math.ceil(2 * f)


def test_ustate_rounding_is_unbiased(oracle_mod):
    r = np.random.default_rng(10)
    q = r.uniform(-1.2, 1.2, 64).astype(np.float32)
    N = 2048
    acc = np.zeros(64)
    for j in range(N):
        codes, mean16, _ = oracle.ustate_group(q, 1.0, np.full(32, (j + 0.5) / N, np.float32))
        acc += np.array([-1.5, -0.5, 0.5, 1.5])[codes]
    mean = float((np.array([mean16], np.uint32) << 16).view(np.float32)[0])
    x = (q - np.float32(mean)).astype(np.float64)
    assert np.all(np.abs(acc / N - x) <= 2.0 / N)


def test_scale_rotation_and_empty_first_step(oracle_mod):
    r = np.random.default_rng(12)
    n = 3000
    p = r.normal(0, 0.02, n).astype(np.float32)
    st = oracle.TurboState(n)
    g = r.normal(0, 1e-3, n).astype(np.float32)
    oracle.turbo_step(p, g, st, oracle.scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1), oracle.turbo_scalars(0.9, 0.999, 1), 1)
    s1 = float(st.scal[1])
    assert st.scal[0] == 0.0 and s1 > 0 and st.scal[2] == 0.0
    # at step 1 the update is g / (|g| + eps) scaled by lr: the first-moment state is irrelevant
    g2 = r.normal(0, 1e-3, n).astype(np.float32)
    oracle.turbo_step(p, g2, st, oracle.scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 2), oracle.turbo_scalars(0.9, 0.999, 2), 2)
    assert st.scal[0] == np.float32(s1)


def test_rms_sum_is_a_pairwise_double_tree(oracle_mod):
    """The encode scale is 1.1 * sqrt(sum r^2 / n) with the residuals of the
    groups: the tree sum agrees with the exact (fsum) sum to double rounding."""
    r = np.random.default_rng(13)
    n = 1000
    p = r.normal(0, 0.02, n).astype(np.float32)
    st = oracle.TurboState(n, compress_v=False)
    g = r.normal(0, 1e-3, n).astype(np.float32)
    pc = p.copy()
    oracle.turbo_step(pc, g, st, oracle.scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 1), oracle.turbo_scalars(0.9, 0.999, 1), 1)
    # rebuild q and the residuals from the FP32 moments of this step
    m = (np.float32(0.1) * g).astype(np.float32)
    v = (np.float32(0.001) * g * g).astype(np.float32)
    sc = oracle.scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 1)
    q = ((m / np.float32(0.1)) / (np.sqrt(v / sc[4]) + sc[7])).astype(np.float32)
    r2 = []
    for gi in range(0, n, 64):
        _, _, rr = oracle.ustate_group(q[gi:gi + 64], 0.0, np.zeros(32, np.float32))
        r2.extend(rr.tolist())
    want = np.float32(1.1 * math.sqrt(math.fsum(r2) / n))
    assert abs(int(np.float32(st.scal[1]).view(np.int32)) - int(want.view(np.int32))) <= 1


def test_tracks_fp32_adamw(oracle_mod):
    """Twenty compressed steps against plain AdamW on the same gradients.  With
    1Q alone the trajectory stays close element by element; with UState the
    2-bit stochastic codes add per-element noise but the mean movement is
    AdamW's (the page likewise names UState as the source of the remaining
    gap, and 1Q alone as within a fraction of a percent of AdamW)."""
    n = 20000
    p0 = np.random.default_rng(14).normal(0, 0.02, n).astype(np.float32)
    res = {}
    for name, cm, cv in (("1q", False, True), ("both", True, True)):
        pt, pf = p0.copy(), p0.copy()
        st = oracle.TurboState(n, compress_m=cm, compress_v=cv)
        m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
        r = np.random.default_rng(5)
        for t in range(1, 21):
            g = (r.normal(0, 1, n) * 1e-3 + 0.3e-3).astype(np.float32)
            sc = oracle.scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, t)
            assert oracle.turbo_step(pt, g, st, sc, oracle.turbo_scalars(0.9, 0.999, t), t) == 0
            oracle.step_fp32(pf, g, m, v, sc)
        dt, df = (pt - p0).astype(np.float64), (pf - p0).astype(np.float64)
        res[name] = (abs(dt.mean() - df.mean()) / abs(df.mean()), np.corrcoef(dt, df)[0, 1],
                     np.abs(dt - df).mean() / np.abs(df).mean())
    assert res["1q"][0] < 0.03 and res["1q"][1] > 0.98 and res["1q"][2] < 0.12, res
    assert res["both"][0] < 0.06 and res["both"][1] > 0.6, res


def test_deterministic_and_counter_driven(oracle_mod):
    n = 777
    r = np.random.default_rng(15)
    p = r.normal(0, 0.02, n).astype(np.float32)
    g = r.normal(0, 1e-3, n).astype(np.float32)
    outs = []
    for seed, tid in ((1, 0), (1, 0), (2, 0), (1, 3)):
        st = oracle.TurboState(n)
        pc = p.copy()
        oracle.turbo_step(pc, g, st, oracle.scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, 1),
                          oracle.turbo_scalars(0.9, 0.999, 1), 1, tensor_id=tid, seed=seed)
        outs.append(st.v_index.copy())
    assert np.array_equal(outs[0], outs[1])
    assert not np.array_equal(outs[0], outs[2]) and not np.array_equal(outs[0], outs[3])


def test_q1_ends_batch_is_one_value_block(oracle_mod):
    """The batch endpoint routine the GPU test uses gives what a one-value
    block gets from the block encoder, on specials and random floats."""
    rng = np.random.default_rng(21)
    v = np.concatenate([np.array([1.0, 2.0, 0.5, 3.0, 1e-45, 1.1754944e-38, 3.4028235e38], np.float32),
                        (rng.integers(1, 0x7F800000, 300, dtype=np.int64)).astype(np.uint32).view(np.float32)])
    lo, hi = oracle.q1_ends(v)
    for k, x in enumerate(v):
        _, ends, _ = oracle.q1_block(np.array([x], np.float32), 4, np.zeros(1, np.float32))
        assert (int(ends[0]), int(ends[1])) == (int(lo[k]), int(hi[k])), x


# ------------------------------------------------------------- other layouts
# The page's fused path takes power-of-two storage blocks from 32 to 1024
# values, UState mean blocks that divide the storage block, and 2, 3, 4, 6
# or 8 index bits (TurboAdam package page, "Fused CUDA path"; API
# block_size, v_bits, m_block_size).


def test_layouts_taken(oracle_mod):
    for bits in range(0, 10):
        for block in (0, 16, 32, 48, 64, 128, 256, 512, 1024, 2048):
            for group in (0, 1, 2, 3, 4, 48, 64, 128, 1024, 2048):
                want = (bits in (2, 3, 4, 6, 8) and block in (32, 64, 128, 256, 512, 1024)
                        and group >= 1 and group & (group - 1) == 0 and block % group == 0)
                assert oracle.turbo_layout_ok(bits, block, group) == want, (bits, block, group)
                if not want:
                    assert oracle.turbo_state_bytes(1, 1, bits, 4096, block, group) == 0


def test_ledger_other_layouts(oracle_mod):
    """Per value the page's tables give 2 code bits and 16 bits of mean per
    group for UState, b index bits and 32 bits of endpoints per block for
    1Q; per tensor 12 bytes of scales.  At the defaults this is the page's
    6.500732 bits per value."""
    n = FACTS["values"]
    for bits in (2, 3, 4, 6, 8):
        for block in (32, 128, 1024):
            for group in (1, 16, 64, block):
                if group > block:
                    continue
                total = oracle.turbo_state_bytes(1, 1, bits, n, block, group)
                assert total * 8 == n * (2 + bits) + n * 16 // group + n * 32 // block + 96, (bits, block, group)
    assert oracle.turbo_state_bytes(1, 1, 4, n, 128, 64) == FACTS["total_bytes"]


def _unpack(words, bits, n):
    """Field i of the dense little-endian bit stream held in `words`, read
    with numpy's own little-endian bit order."""
    b = np.unpackbits(np.ascontiguousarray(words, "<u4").view(np.uint8), bitorder="little")
    return (b[: n * bits].reshape(n, bits).astype(np.int64) << np.arange(bits)).sum(1), b[n * bits:]


def _f16v(code):
    return float(np.array([code], np.uint16).view(np.float16)[0])


@pytest.mark.parametrize("bits,block", [(3, 32), (3, 1024), (6, 128), (6, 512), (2, 64), (8, 256), (4, 32)])
def test_dense_indices_and_block_endpoints(oracle_mod, bits, block):
    """Step 1 from the empty state, 1Q only: the new second moment is the
    FP32 oracle's.  Unpacked in numpy's little-endian bit order, every index
    decodes, with its own block's endpoints, to one of the two levels around
    that value (0 for a zero); each block's endpoints are the tightest
    binary16 bounds of log2 over its positive values; the bits past the last
    value are zero."""
    r = np.random.default_rng(100 + bits * 7 + block)
    n = 3 * block + 37
    p = r.normal(0, 0.02, n).astype(np.float32)
    g = (r.normal(0, 1, n) * 10.0 ** r.uniform(-5, -1, n)).astype(np.float32)
    g[r.integers(0, n, 5)] = 0.0
    st = oracle.TurboState(n, compress_m=False, compress_v=True, bits=bits, block=block, group=min(64, block))
    sc = oracle.scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    oracle.turbo_step(p.copy(), g, st, sc, oracle.turbo_scalars(0.9, 0.999, 1), 1)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    oracle.step_fp32(p.copy(), g, m, v, sc)
    idx, tail = _unpack(st.v_index, bits, n)
    assert not tail.any()
    L = 1 << bits
    assert idx.min() >= 0 and idx.max() < L
    for b in range((n + block - 1) // block):
        sl = slice(b * block, min(n, (b + 1) * block))
        vb = v[sl]
        pos = vb[vb > 0]
        lo16, hi16 = int(st.v_ends[2 * b]), int(st.v_ends[2 * b + 1])
        lo, hi = _f16v(lo16), _f16v(hi16)
        l2min, l2max = math.log2(float(pos.min())), math.log2(float(pos.max()))
        assert lo <= l2min and float(np.nextafter(np.float16(lo), np.float16(np.inf))) > l2min
        assert hi >= l2max and float(np.nextafter(np.float16(hi), np.float16(-np.inf))) < l2max
        lev = oracle.q1_levels(lo16, hi16, bits)
        for x, k in zip(vb, idx[sl]):
            if x == 0:
                assert k == 0
            else:
                assert k >= 1 and (lev[k] == x or (k > 1 and lev[k - 1] < x < lev[k])
                                   or (k < L - 1 and lev[k] < x < lev[k + 1])), (x, k)


@pytest.mark.parametrize("group", [1, 2, 8, 128, 1024])
def test_group_means_and_scale_other_sizes(oracle_mod, group):
    """Step 1, UState over groups of `group` values with 1Q off, so the
    persisted second moment is v' itself.  q comes from the FP32 oracle's
    moments through numpy's IEEE float32 operations.  Each stored mean is
    torch's bfloat16 of the float32-rounded exact (fsum) group mean; the
    next encode scale is 1.1 x the exact RMS of q minus its group's mean,
    within one binary32 ulp."""
    import torch
    r = np.random.default_rng(200 + group)
    n = 2 * 1024 + 300
    p = r.normal(0, 0.02, n).astype(np.float32)
    g = (r.normal(0, 1e-3, n) + 2e-4).astype(np.float32)
    st = oracle.TurboState(n, compress_m=True, compress_v=False, bits=4, block=1024, group=group)
    sc = oracle.scalars(1e-3, 0.9, 0.999, 1e-8, 0.0, 1)
    oracle.turbo_step(p.copy(), g, st, sc, oracle.turbo_scalars(0.9, 0.999, 1), 1)
    m, v = np.zeros(n, np.float32), np.zeros(n, np.float32)
    oracle.step_fp32(p.copy(), g, m, v, sc)
    bc1 = oracle.turbo_scalars(0.9, 0.999, 1)[0]
    q = ((m / bc1) / (np.sqrt(v / sc[4]) + sc[7])).astype(np.float32)
    assert st.m_means.size == (n + group - 1) // group
    r2 = []
    for gi in range(st.m_means.size):
        qs = q[gi * group:(gi + 1) * group]
        exact = math.fsum(float(x) for x in qs) / qs.size
        want = int(torch.tensor([float(np.float32(exact))]).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF
        assert int(st.m_means[gi]) == want, gi
        mean = np.float32((np.array([want], np.uint32) << 16).view(np.float32)[0])
        r2.extend(((qs - mean).astype(np.float64) ** 2).tolist())
    s_enc = np.float32(1.1 * math.sqrt(math.fsum(r2) / n))
    assert abs(int(np.float32(st.scal[1]).view(np.int32)) - int(s_enc.view(np.int32))) <= 1


@pytest.mark.parametrize("group", [1, 2, 16, 256, 1024])
def test_ustate_recentering_other_group_sizes(oracle_mod, group):
    """Decoding a group of any size keeps the stored mean: mean + s (level -
    mean level) averages to the mean."""
    r = np.random.default_rng(300 + group)
    for _ in range(10):
        n = int(r.integers(1, group + 1))
        q = (r.normal(0, 1, n) * 10.0 ** r.uniform(-2, 1)).astype(np.float32)
        s = np.float32(10.0 ** r.uniform(-2, 1))
        codes, mean16, _ = oracle.ustate_group(q, s, r.random((n + 1) // 2).astype(np.float32), group)
        mean = float((np.array([mean16], np.uint32) << 16).view(np.float32)[0])
        dec = oracle.ustate_decode(codes, mean16, s)
        assert abs(dec.astype(np.float64).mean() - mean) <= 4e-7 * (abs(mean) + 2 * s) + 1e-30


def test_default_layout_is_the_original(oracle_mod):
    """Block 128 and group 64 are the defaults: naming them changes nothing."""
    r = np.random.default_rng(400)
    n = 5003
    p0 = r.normal(0, 0.02, n).astype(np.float32)
    outs = []
    for kw in ({}, dict(block=128, group=64)):
        st = oracle.TurboState(n, **kw)
        p = p0.copy()
        for t in (1, 2, 3):
            g = np.random.default_rng(t).normal(0, 1e-3, n).astype(np.float32)
            oracle.turbo_step(p, g, st, oracle.scalars(1e-3, 0.9, 0.999, 1e-8, 0.01, t),
                              oracle.turbo_scalars(0.9, 0.999, t), t)
        outs.append((p.copy(), st.v_index.copy(), st.m_codes.copy(), st.m_means.copy(), st.scal.copy()))
    for a, b in zip(*outs):
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8))


def test_antithetic_pairs_follow_the_tensor_index(oracle_mod):
    """The pairs are the tensor's values 2j and 2j+1 whatever the group size:
    a one-value group at an odd index takes 1 - u.  With s = 1 a value whose
    residual is almost 0 sits half-way from level -0.5 to level 0.5, so
    u = 0.3 rounds it up and 1 - u = 0.7 does not."""
    q = np.array([0.3], np.float32)             # bf16(0.3) differs from 0.3 by < 2^-9
    u = np.array([0.3], np.float32)
    up, _, _ = oracle.ustate_group(q, 1.0, u, group=1, first=4)
    down, _, _ = oracle.ustate_group(q, 1.0, u, group=1, first=5)
    assert (int(up[0]), int(down[0])) == (2, 1)
    # in a two-value group the second value is the odd one of the pair
    both, _, _ = oracle.ustate_group(np.array([0.3, 0.3], np.float32), 1.0, u, group=2, first=4)
    assert both.tolist() == [2, 1]


def _bf16_rne(x):
    """bfloat16 bits of float32 values, rounded to nearest even by integer
    arithmetic on the bit patterns (finite and infinite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _to_type(x32, dt):
    if dt == oracle.DT_F32:
        return np.ascontiguousarray(x32, np.float32)
    if dt == oracle.DT_BF16:
        return _bf16_rne(x32)
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(x32, np.float32).astype(np.float16).view(np.uint16)


def _widen(a, dt):
    if dt == oracle.DT_F32:
        return a.copy()
    if dt == oracle.DT_BF16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.view(np.float16).astype(np.float32)


@pytest.mark.parametrize("pdt,gdt", [(1, 1), (2, 2), (1, 0), (2, 0)], ids=["bf16", "f16", "bf16-f32g", "f16-f32g"])
@pytest.mark.parametrize("bits,block,group", [(4, 128, 64), (3, 256, 32)])
@pytest.mark.parametrize("lr,wd", [(1e-3, 0.01), (30.0, 0.0)])
def test_typed_parameters_round_only_the_parameter(oracle_mod, pdt, gdt, bits, block, group, lr, wd):
    """16-bit parameters and gradients (the TurboAdam page's Verification runs
    fp16, bf16 and fp32 parameters): over three steps, the new parameter is
    numpy's binary16 rounding, or a round-to-nearest-even on the bfloat16 bit
    pattern, of the FP32 step's result on the widened values, and the state
    and non-finite count are the FP32 step's exactly (the page's update reads
    the parameter only in its own line).  lr = 30 with no decay drives binary16
    parameters near its largest finite value past it, to Inf."""
    n = 3000
    r = np.random.default_rng(61 + 7 * pdt + gdt)
    p32 = r.normal(0, 0.02, n).astype(np.float32)
    p32[:6] = [65504.0, -65504.0, 65000.0, 1.5, -3.0e-8, 6.1e-5]
    pt = _to_type(p32, pdt)
    st_t = oracle.TurboState(n, bits=bits, block=block, group=group)
    st_f = oracle.TurboState(n, bits=bits, block=block, group=group)
    for t in range(1, 4):
        g32 = (r.normal(0, 1e-3, n) - 2e-4).astype(np.float32)
        g32[:6] = [-1e-3, 1e-3, -1e-3, 0.0, 2e-3, -5e-4]
        gt = _to_type(g32, gdt)
        sc = oracle.scalars(lr, 0.9, 0.999, 1e-8, wd, t)
        ts = oracle.turbo_scalars(0.9, 0.999, t)
        pf = _widen(pt, pdt)
        bad_f = oracle.turbo_step(pf, _widen(gt, gdt), st_f, sc, ts, t, tensor_id=5)
        bad_t = oracle.turbo_step_typed(pdt, gdt, pt, gt, st_t, sc, ts, t, tensor_id=5)
        assert bad_t == bad_f
        want = _to_type(pf, pdt)
        assert np.array_equal(pt.view(np.uint16), want.view(np.uint16)), f"step {t}"
        for name, a in st_t.arrays().items():
            b = st_f.arrays()[name]
            assert (a is None) == (b is None)
            if a is not None:
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (t, name)
    if pdt == oracle.DT_F16 and lr == 30.0:
        assert np.isinf(pt[:2].view(np.float16)).all(), pt[:2].view(np.float16)
    # bfloat16 rounding itself: ties go to even, and a value just above a tie up
    x = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20], np.float32)
    assert list(_bf16_rne(x)) == [0x3F80, 0x3F82, 0x3F81]


def test_gpt2_layer_memory_profile(oracle_mod):
    """The page's GPT-2-layer memory table: its four persistent-byte figures
    (AdamW, UState only, 1Q only, both) from the nine-tensor layer that the
    fixture's reading names.  torch's own AdamW on the CPU, an independent
    library, gives the AdamW figure from the same shapes, which pins the
    shape reading; the oracle's ledger then gives the three TurboAdam
    figures, the UState-only and 1Q-only ones included."""
    import torch
    prof = json.load(open(os.path.join(ROOT, "tests", "golden", "pages_facts.json")))["turboadam_gpt2_layer_profile"]
    shapes = [tuple(s) for s in prof["shapes"]]
    want = prof["persistent_bytes"]
    ps = [torch.nn.Parameter(torch.zeros(s)) for s in shapes]
    opt = torch.optim.AdamW(ps, lr=1e-3)
    for p in ps:
        p.grad = torch.ones_like(p)
    opt.step()
    got = sum(t.numel() * t.element_size() for st in opt.state.values() for t in st.values() if torch.is_tensor(t))
    assert got == want["adamw"]
    ns = [math.prod(s) for s in shapes]
    thr = FACTS["defaults"]["min_m_compress_elements"]
    for key, (cm, cv) in (("ustate_and_oneq", (1, 1)), ("ustate_only", (1, 0)), ("oneq_only", (0, 1))):
        total = sum(oracle.turbo_state_bytes(cm and n >= thr, cv and n >= thr, 4, n) for n in ns)
        assert total == want[key], key
