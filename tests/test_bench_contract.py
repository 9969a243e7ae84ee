"""bench.py's command-line contract that holds without a GPU: a run on more
than one GPU is refused with a message (every box here has one GPU), before
anything touches a device; and a stored counter reading is reported only
with the kernel sources it was taken with."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=e, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    r = _run([], {"WORLD_SIZE": "4", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_stored_counter_readings_are_used_only_with_their_kernel_sources(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, "profiles", "traffic_llama-7b_e4.json")) as f:
        traffic = json.load(f)
    assert bench.kernel_sha("elementwise") != bench.kernel_sha("turbo")
    monkeypatch.setattr(bench, "kernel_sha", lambda family="elementwise": traffic["kernel_sha"])
    assert bench.load_traffic("llama-7b", "e4") == traffic["traffic_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_sha", lambda family="elementwise": "0" * 16)
    assert bench.load_traffic("llama-7b", "e4") is None          # stale: reported as null
    assert bench.load_traffic("llama-7b", "fp32") is None        # never measured


def test_profile_summaries_quote_commands_that_run_committed_files():
    """Every summary under profiles/ gives the command that made it, and the
    program each command runs is a file of this repository (bench.py at its
    root), never one from a working folder."""
    import glob
    import re
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))
    assert files
    for f in files:
        lines = open(f).read().splitlines()
        cmds = [l for l in lines if "rocprofv3 " in l or re.match(r"\s*(timeout .*)?python3? ", l)]
        assert cmds, f"{os.path.basename(f)}: no command"
        for c in cmds:
            assert "_work" not in c, f"{os.path.basename(f)}: {c}"
            for prog in re.findall(r"python3?\s+(?:-u\s+)?(\S+\.py)", c):
                assert os.path.exists(os.path.join(ROOT, prog)), f"{os.path.basename(f)}: {prog} is not in the repository"
