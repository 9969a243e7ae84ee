"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

Two drivers under tests/sanitize/ are built with the sanitizers on host code
only and run here:
  - oracle_driver.c runs every oracle function on ordinary, boundary and
    non-finite inputs;
  - host_driver.cpp drives the C ABI's argument validation (pa_api.hip's host
    side); its device code is compiled as usual and never launched.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")


def _run(cmd, env=None, timeout=300):
    return subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=timeout, env=env)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    b = _run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
              "-ffp-contract=off", "-o", exe, os.path.join(SAN, "oracle_driver.c"),
              os.path.join(ROOT, "oracle", "pa_oracle.c"), "-lquadmath", "-lm"])
    assert b.returncode == 0, b.stderr[-4000:]
    r = _run([exe], timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "oracle driver ok" in r.stdout


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.mark.skipif(_hipcc() is None, reason="hipcc not found")
def test_host_validation_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_driver")
    b = _run([_hipcc(), "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-ffp-contract=off",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
              "-o", exe, os.path.join(SAN, "host_driver.cpp"),
              os.path.join(ROOT, "adamw_step_amd", "csrc", "pa_api.hip")], timeout=600)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", HIP_VISIBLE_DEVICES="")
    r = _run([exe], env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "host driver ok" in r.stdout
