"""The GPU path's double-double decision of a 1Q grid level (the exact 2^x
rounded once to binary32; TurboAdam package page, 1Q), built for the host
from the same header and checked on the CPU against the oracle's levels and
the 60-digit decimal arbiter, over every kind of x it can meet: random grids
across the whole endpoint range, the committed near-midpoint levels, and
x at the overflow threshold, in the subnormal range and at the range ends.
The device runs the same IEEE double operations; the GPU tests compare the
device's own results with the oracle."""
import ctypes
import json
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from exact_pow2 import grid_x, near_midpoint_exponents, rn32_pow2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TIES = json.load(open(os.path.join(ROOT, "tests", "golden", "q1_level_ties.json")))["rows"]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def dd(tmp_path_factory):
    if _hipcc() is None:
        pytest.skip("hipcc not found")
    out = str(tmp_path_factory.mktemp("pow2") / "libpow2_host.so")
    r = subprocess.run([_hipcc(), "-O2", "-std=c++17", "--offload-host-only", "-x", "hip", "-ffp-contract=off",
                        "-fno-fast-math", "-fPIC", "-shared", "-I", os.path.join(ROOT, "adamw_step_amd", "csrc"),
                        os.path.join(ROOT, "tests", "host", "pow2_host.hip"), "-o", out],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    lib = ctypes.CDLL(out)
    lib.pow2_rn32_dd_host.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t]

    def run(x):
        x = np.ascontiguousarray(x, np.float64)
        y = np.empty(x.size, np.float32)
        lib.pow2_rn32_dd_host(x.ctypes.data, y.ctypes.data, x.size)
        return y
    return run


def _f16(code):
    return float(np.array([code], np.uint16).view(np.float16)[0])


def _f16_bits(x):
    return int(np.array([x], np.float16).view(np.uint16)[0])


def test_random_grids_match_oracle(dd):
    r = np.random.default_rng(31)
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = codes.view(np.float16).astype(np.float64)
    pool = codes[np.isfinite(vals) & (vals >= -149) & (vals <= 128)]
    for bits, blocks in ((2, 4000), (4, 1500), (8, 200)):
        L = 1 << bits
        for _ in range(blocks):
            a, b = sorted(float(_f16(c)) for c in r.choice(pool, 2))
            lev = oracle.q1_levels(_f16_bits(a), _f16_bits(b), bits)
            got = dd([grid_x(a, b, k, L) for k in range(1, L)])
            assert np.array_equal(got.view(np.uint32), lev[1:].view(np.uint32)), (a, b, bits)


def test_near_midpoint_levels(dd):
    for row in TIES:
        x = grid_x(_f16(int(row["lo16"], 16)), _f16(int(row["hi16"], 16)), row["k"], 1 << row["bits"])
        assert f"{int(dd([x]).view(np.uint32)[0]):08x}" == row["level_hex"], row


def _around(x, steps):
    out = [x]
    lo = hi = x
    for _ in range(steps):
        lo, hi = np.nextafter(lo, -np.inf), np.nextafter(hi, np.inf)
        out += [lo, hi]
    return out


def test_range_ends_and_thresholds(dd):
    xs = [float("nan"), float("inf"), float("-inf"), 1e300, -1e300, 128.0, -150.0, -149.0, 127.0, 0.0, -0.0]
    xs += list(np.arange(-149, 128, dtype=np.float64))
    # the overflow threshold 2^128 - 2^103 and the top of the range
    xs += _around(128.0 + np.log2(1.0 - 2.0 ** -25), 40) + _around(128.0, 8) + _around(127.99999, 8)
    # 2^-150 (the midpoint between 0 and the smallest subnormal), other
    # subnormal midpoints, and the smallest normal
    xs += _around(-150.0, 8) + _around(-149.0 + np.log2(1.5), 20) + _around(-146.0 + np.log2(1.125), 20)
    xs += _around(-126.0, 8) + _around(-126.0 - 2.0 ** -30, 4)
    # uniform over the range and just past its ends
    xs += list(np.random.default_rng(5).uniform(-151, 129, 20000))
    got = dd(xs)
    for x, g in zip(xs, got):
        want, _ = rn32_pow2(float(x))
        assert (np.isnan(want) and np.isnan(g)) or g.view(np.uint32) == want.view(np.uint32), (x, g, want)


def test_within_2m56_of_midpoints(dd):
    """x whose power lies within 2^-56 of a binary32 midpoint (some within
    2^-64): the double-double decision equals the decimal arbiter."""
    xs = near_midpoint_exponents(12)
    got = dd(xs)
    for x, g in zip(xs, got):
        want, _ = rn32_pow2(float(x))
        assert g.view(np.uint32) == want.view(np.uint32), (x, g, want)
