"""The C-ABI library loads, exports every entry point declared in include/pa.h,
and rejects invalid calls before touching the device (no GPU needed)."""
import ctypes
import json
import math
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    if not os.path.exists(pa_mod.LIB_PATH):
        from adamw_step_amd import build as b
        b.build()
    pa_mod.lib()
    return pa_mod


def _declared():
    with open(os.path.join(ROOT, "include", "pa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:[A-Za-z_][\w ]*\*?\s+\**)(pa_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol(pa):
    names = _declared()
    assert set(names) >= {"pa_step", "pa_step_list", "pa_state_bytes", "pa_format_info",
                          "pa_status_string", "pa_last_hip_error", "pa_release_plans", "pa_debug_codec"}
    raw = ctypes.CDLL(pa.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(pa.EXPORTS) == set(names)


def test_ledger_matches_pages(pa):
    with open(os.path.join(ROOT, "tests", "golden", "pages_facts.json")) as f:
        facts = json.load(f)["state_bytes_per_param"]
    n = 11637760
    assert pa.pa_state_bytes(pa.PA_FP32, n) == facts["fp32_adamw"] * n
    assert pa.pa_state_bytes(pa.PA_PACKED_E4, n) == facts["packed_e4"] * n
    assert pa.pa_state_bytes(pa.PA_PACKED_FP16, n) == 4 * n
    assert pa.pa_state_bytes(pa.PA_BLOCKWISE8, 4096) == 2 * 4096 + 2 * 2 * 4
    assert pa.pa_state_bytes(7, 10) == 0


def test_format_info_agrees_with_oracle(pa, oracle_mod):
    f = pa.pa_format_info(pa.PA_PACKED_E4)
    m = oracle_mod.decode(0, np.array([0x7FFF, 0x0800, 0x0001], np.uint16)).astype(np.float64)
    r = oracle_mod.decode(1, np.array([0xFFFF, 0x1000, 0x0001], np.uint16)).astype(np.float64)
    assert (f["m_max"], f["m_min_normal"], f["m_min_subnormal"]) == tuple(m)
    assert (f["r_max"], f["r_min_normal"], f["r_min_subnormal"]) == tuple(r)
    assert f["m_exp_bias"] == f["r_exp_bias"] == oracle_mod.e4_bias()
    assert (f["m_sign_bits"], f["m_exp_bits"], f["m_mant_bits"]) == (1, 4, 11)
    assert (f["r_sign_bits"], f["r_exp_bits"], f["r_mant_bits"]) == (0, 4, 12)
    h = pa.pa_format_info(pa.PA_PACKED_FP16)
    assert h["m_max"] == 65504.0 and h["m_min_subnormal"] == 2.0 ** -24
    assert pa.pa_format_info(pa.PA_BLOCKWISE8)["block"] == 2048


def test_status_strings(pa):
    for rc in range(0, -8, -1):
        assert pa.pa_status_string(rc) != "unknown status"
    assert pa.pa_status_string(-99) == "unknown status"


def _hyper(pa, **kw):
    h = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    h.update(kw)
    return pa.Hyper(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], None)


def _raw_step(pa, mode, p, g, s, n, h, step=1):
    return pa.lib().pa_step(mode, p, g, s, n, ctypes.byref(h), step, None)


FAKE = 0x7F0000000000   # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("kw,step,want", [
    (dict(), 0, -1),
    (dict(beta1=1.0), 1, -1),
    (dict(beta2=-0.1), 1, -1),
    (dict(lr=float("nan")), 1, -1),
    (dict(eps=-1.0), 1, -1),
    (dict(weight_decay=float("inf")), 1, -1),
])
def test_bad_hyper_rejected(pa, kw, step, want):
    h = _hyper(pa, **kw)
    assert _raw_step(pa, 1, FAKE, FAKE + 4096, FAKE + 8192, 16, h, step) == want


def test_argument_rules(pa):
    h = _hyper(pa)
    n = 1024
    L = pa.lib()
    assert L.pa_step(9, FAKE, FAKE, FAKE, n, ctypes.byref(h), 1, None) == pa.PA_ERR_ARG
    assert _raw_step(pa, 1, None, FAKE, FAKE, n, h) == pa.PA_ERR_ARG
    assert _raw_step(pa, 1, None, None, None, 0, h) == pa.PA_OK           # n == 0 is a no-op
    assert L.pa_step(1, FAKE, FAKE, FAKE, n, None, 1, None) == pa.PA_ERR_ARG
    # alignment: 2-byte offset, and a different 16-byte phase
    assert _raw_step(pa, 1, FAKE + 2, FAKE + 8192, FAKE + 16384, n, h) == pa.PA_ERR_ALIGN
    assert _raw_step(pa, 1, FAKE + 4, FAKE + 8192, FAKE + 16384, n, h) == pa.PA_ERR_ALIGN
    # overlap of params and state words
    assert _raw_step(pa, 1, FAKE, FAKE + 65536, FAKE + 1024, n, h) == pa.PA_ERR_ALIAS
    # FP32 mode reads its host descriptor
    st = pa.Fp32State(FAKE + 65536, None)
    assert _raw_step(pa, 0, FAKE, FAKE + 16384, ctypes.addressof(st), n, h) == pa.PA_ERR_ARG
    st = pa.Fp32State(FAKE + 65536, FAKE + 65536 + 2048)
    assert _raw_step(pa, 0, FAKE, FAKE + 16384, ctypes.addressof(st), n, h) == pa.PA_ERR_ALIAS
    # blockwise: the length rule, then alignment
    bw = pa.BlockwiseState(FAKE + 2 ** 20, FAKE + 2 ** 21, FAKE + 2 ** 22, FAKE + 2 ** 23,
                           FAKE + 2 ** 24, FAKE + 2 ** 25, FAKE + 2 ** 26)
    assert _raw_step(pa, 3, FAKE, FAKE + 2 ** 18, ctypes.addressof(bw), 2048 + 16, h) == pa.PA_ERR_SHAPE
    assert _raw_step(pa, 3, FAKE + 4, FAKE + 2 ** 18, ctypes.addressof(bw), 2048, h) == pa.PA_ERR_ALIGN
    bw2 = pa.BlockwiseState(FAKE + 2 ** 20, FAKE + 2 ** 21, FAKE + 2 ** 20 + 1024, FAKE + 2 ** 23,
                            FAKE + 2 ** 24, FAKE + 2 ** 25, FAKE + 2 ** 26)
    assert _raw_step(pa, 3, FAKE, FAKE + 2 ** 18, ctypes.addressof(bw2), 2048, h) == pa.PA_ERR_ALIAS


def test_list_argument_rules(pa):
    h = _hyper(pa)
    L = pa.lib()
    assert L.pa_step_list(1, 0, None, None, None, None, ctypes.byref(h), 1, None) == pa.PA_OK
    assert L.pa_step_list(1, 2, None, None, None, None, ctypes.byref(h), 1, None) == pa.PA_ERR_ARG
    assert L.pa_step_list(5, 1, None, None, None, None, ctypes.byref(h), 1, None) == pa.PA_ERR_ARG
    assert L.pa_step_list(1, 1, None, None, None, None, ctypes.byref(h), 0, None) == pa.PA_ERR_ARG


def test_debug_codec_rules(pa):
    L = pa.lib()
    assert L.pa_debug_codec(4, 0, FAKE, FAKE + 4096, 4, None) == pa.PA_ERR_ARG
    assert L.pa_debug_codec(-1, 0, FAKE, FAKE + 4096, 4, None) == pa.PA_ERR_ARG
    assert L.pa_debug_codec(0, 2, FAKE, FAKE + 4096, 4, None) == pa.PA_ERR_ARG
    assert L.pa_debug_codec(0, 0, FAKE + 2, FAKE + 4096, 4, None) == pa.PA_ERR_ALIGN
    assert L.pa_debug_codec(0, 0, None, None, 0, None) == pa.PA_OK
    assert L.pa_debug_q1_ends(None, None, 0, None) == pa.PA_OK
    assert L.pa_debug_q1_ends(None, FAKE, 4, None) == pa.PA_ERR_ARG
    assert L.pa_debug_q1_ends(FAKE + 2, FAKE + 4096, 4, None) == pa.PA_ERR_ALIGN
    assert L.pa_debug_q1_levels(None, 4, 0, None, 0, None) == pa.PA_OK
    for bits in (0, 1, 5, 7, 9):
        assert L.pa_debug_q1_levels(FAKE, bits, 0, FAKE + 4096, 4, None) == pa.PA_ERR_ARG
    assert L.pa_debug_q1_levels(None, 4, 0, FAKE, 4, None) == pa.PA_ERR_ARG
    assert L.pa_debug_q1_levels(FAKE, 4, 1, FAKE + 4096, (1 << 40) + 1, None) == pa.PA_ERR_ARG
    assert L.pa_debug_q1_levels(FAKE + 2, 4, 0, FAKE + 4096, 4, None) == pa.PA_ERR_ALIGN
    assert L.pa_debug_pow2_rn32(None, 0, None, 0, None) == pa.PA_OK
    assert L.pa_debug_pow2_rn32(None, 0, FAKE, 4, None) == pa.PA_ERR_ARG
    assert L.pa_debug_pow2_rn32(FAKE + 4, 0, FAKE + 4096, 4, None) == pa.PA_ERR_ALIGN


def test_debug_blockwise_path_rules(pa):
    """The blockwise launch switch takes -1 (persistent), 0 (by size) and
    1..2^20 blocks per workgroup; it only sets a flag (no device work)."""
    L = pa.lib()
    for bad in (-2, -(1 << 40), (1 << 20) + 1):
        assert L.pa_debug_blockwise_path(bad) == pa.PA_ERR_ARG
    for ok in (-1, 1, 12, 1 << 20, 0):
        assert L.pa_debug_blockwise_path(ok) == pa.PA_OK


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import adamw_step_amd as pa_mod
    monkeypatch.setattr(pa_mod, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(pa_mod, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        pa_mod.lib()


def test_product_path_never_imports_oracle():
    pkg = os.path.join(ROOT, "adamw_step_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                with open(os.path.join(dirpath, fn)) as f:
                    text = f.read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "pa_oracle" not in text and "libpa_oracle" not in text, fn
    with open(os.path.join(ROOT, "oracle", "pa_oracle.c")) as f:
        text = f.read()
    assert "codec.hpp" not in text and "kernels.hpp" not in text and "pa.h" not in text
    assert not math.isnan(0.0)


def test_inspect_formats_runs_without_torch(pa):
    """The inspection command imports no torch and agrees with the ledger."""
    import subprocess
    import sys as _sys
    code = ("import sys; from adamw_step_amd import inspect_formats as f; "
            "t = f.render(markdown=True); assert 'torch' not in sys.modules, 'torch imported'; print(t)")
    r = subprocess.run([_sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "bias 15" in r.stdout and "| 4 |" in r.stdout and "| 8 |" in r.stdout
    if not __import__("torch").cuda.is_available():   # without a GPU the examples say so and exit 2
        r = subprocess.run([_sys.executable, "-m", "adamw_step_amd.inspect_formats", "--examples"], cwd=ROOT,
                           capture_output=True, text=True, timeout=300)
        assert r.returncode == 2 and "GPU" in r.stderr and "Traceback" not in r.stderr, r.stderr
        assert "bias 15" in r.stdout


def test_typed_argument_rules(pa):
    h = _hyper(pa)
    L = pa.lib()
    L.pa_step_typed.argtypes = None
    f = lambda mode, pdt, gdt, p, g, s, n: L.pa_step_typed(mode, pdt, gdt, ctypes.c_void_p(p), ctypes.c_void_p(g),
                                                             ctypes.c_void_p(s), ctypes.c_size_t(n), ctypes.byref(h),
                                                             ctypes.c_longlong(1), None)
    assert f(1, 1, 2, FAKE, FAKE + 8192, FAKE + 16384, 64) == pa.PA_ERR_ARG      # bf16 params, f16 grads
    assert f(1, 0, 1, FAKE, FAKE + 8192, FAKE + 16384, 64) == pa.PA_ERR_ARG      # f32 params, bf16 grads
    assert f(1, 3, 3, FAKE, FAKE + 8192, FAKE + 16384, 64) == pa.PA_ERR_ARG      # unknown dtype
    bw = pa.BlockwiseState(FAKE + 2 ** 20, FAKE + 2 ** 21, FAKE + 2 ** 22, FAKE + 2 ** 23,
                           FAKE + 2 ** 24, FAKE + 2 ** 25, FAKE + 2 ** 26)
    assert f(3, 1, 1, FAKE, FAKE + 2 ** 18, ctypes.addressof(bw), 2048) == pa.PA_ERR_ARG   # blockwise 16-bit
    assert f(1, 1, 1, FAKE + 1, FAKE + 8193, FAKE + 16384, 64) == pa.PA_ERR_ALIGN           # odd address
    # bf16 params and grads at element phase 1, words at element phase 2
    assert f(1, 1, 1, FAKE + 2, FAKE + 8194, FAKE + 16392, 64) == pa.PA_ERR_ALIGN
    # bf16 params at phase 1, f32 grads at phase 0
    assert f(1, 1, 0, FAKE + 2, FAKE + 8192, FAKE + 16388, 64) == pa.PA_ERR_ALIGN
    # overlapping bf16 params and words
    assert f(1, 1, 1, FAKE, FAKE + 65536, FAKE + 64, 64) == pa.PA_ERR_ALIAS


def test_grad_stats_argument_rules(pa):
    L = pa.lib()
    G = (ctypes.c_void_p * 1)(FAKE)
    N = (ctypes.c_size_t * 1)(64)
    f = lambda gdt, cnt, g, n, mx, s, nf, cl: L.pa_grad_stats_list(gdt, cnt, g, n, mx, s, nf, cl, None)
    assert f(3, 1, G, N, 0.0, FAKE + 4096, None, None) == pa.PA_ERR_ARG            # unknown dtype
    assert f(0, 1, G, N, 0.0, None, None, None) == pa.PA_ERR_ARG                    # no sumsq output
    assert f(0, 1, None, N, 0.0, FAKE + 4096, None, None) == pa.PA_ERR_ARG          # no gradient list
    assert f(0, 1, G, N, 0.0, FAKE + 4096, None, FAKE + 4104) == pa.PA_ERR_ARG      # clip without max_norm
    assert f(0, 1, G, N, float("nan"), FAKE + 4096, None, FAKE + 4104) == pa.PA_ERR_ARG
    assert f(0, 1, G, N, 1.0, FAKE + 4100, None, None) == pa.PA_ERR_ALIGN           # sumsq not 8-aligned
    assert f(0, 1, G, N, 1.0, FAKE + 4096, FAKE + 4108, None) == pa.PA_ERR_ALIGN    # counter not 8-aligned
    assert f(0, 1, G, N, 1.0, FAKE + 4096, FAKE + 4096, None) == pa.PA_ERR_ALIAS    # outputs overlap
    assert f(0, 1, G, N, 1.0, FAKE + 4096, FAKE + 4104, FAKE + 4100) == pa.PA_ERR_ALIAS


def test_hyper_device_inputs_rules(pa):
    n = 1024
    h = _hyper(pa)
    h.grad_scale = FAKE + 2 ** 20 + 2                       # not 4-aligned
    assert _raw_step(pa, 1, FAKE, FAKE + 8192, FAKE + 16384, n, h) == pa.PA_ERR_ALIGN
    h = _hyper(pa)
    h.skip_if_nonzero = FAKE + 2 ** 20 + 4                  # not 8-aligned
    assert _raw_step(pa, 1, FAKE, FAKE + 8192, FAKE + 16384, n, h) == pa.PA_ERR_ALIGN
    h = _hyper(pa)
    h.skip_if_nonzero = FAKE + 64                           # inside the params
    assert _raw_step(pa, 1, FAKE, FAKE + 8192, FAKE + 16384, n, h) == pa.PA_ERR_ALIAS
    h = _hyper(pa)
    h.grad_scale = FAKE + 16384 + 128                       # inside the state words
    assert _raw_step(pa, 1, FAKE, FAKE + 8192, FAKE + 16384, n, h) == pa.PA_ERR_ALIAS
    h = _hyper(pa)
    h.nonfinite = FAKE + 2 ** 20
    h.skip_if_nonzero = FAKE + 2 ** 20                      # one counter as both: would race
    assert _raw_step(pa, 1, FAKE, FAKE + 8192, FAKE + 16384, n, h) == pa.PA_ERR_ALIAS
    bw = pa.BlockwiseState(FAKE + 2 ** 20, FAKE + 2 ** 21, FAKE + 2 ** 22, FAKE + 2 ** 23,
                           FAKE + 2 ** 24, FAKE + 2 ** 25, FAKE + 2 ** 26)
    h = _hyper(pa)
    h.grad_scale = FAKE + 2 ** 22 + 8                       # inside the v codes
    assert _raw_step(pa, 3, FAKE, FAKE + 2 ** 18, ctypes.addressof(bw), 2048, h) == pa.PA_ERR_ALIAS


def test_turbo_argument_rules(pa):
    L = pa.lib()
    h = _hyper(pa)
    cfg = pa.TurboConfig(4, 1.1, 0x12345678)
    P = (ctypes.c_void_p * 1)(FAKE)
    G = (ctypes.c_void_p * 1)(FAKE + 2 ** 20)
    N = (ctypes.c_size_t * 1)(4096)
    S = (pa.TurboStateDesc * 1)(pa.TurboStateDesc(1, 1, 0, FAKE + 2 ** 21, FAKE + 2 ** 22, None,
                                                  FAKE + 2 ** 23, FAKE + 2 ** 24, None, FAKE + 2 ** 25))
    call = lambda h_, c_, step=1: L.pa_turbo_step_list(1, P, G, S, N, ctypes.byref(h_), ctypes.byref(c_), step,
                                                        FAKE + 2 ** 26, 1 << 20, None)
    for bits in (0, 1, 5, 7, 9):                                          # index width
        assert call(h, pa.TurboConfig(bits, 1.1, 1)) == pa.PA_ERR_ARG
    for block, group in ((16, 8), (2048, 64), (96, 32), (64, 128), (128, 3), (128, -4), (-128, 64)):
        assert call(h, pa.TurboConfig(4, 1.1, 1, block, group)) == pa.PA_ERR_ARG, (block, group)
    assert call(h, pa.TurboConfig(4, 1.1, 1, 0, 0, 2)) == pa.PA_ERR_ARG   # kernel choice
    assert call(h, pa.TurboConfig(4, 0.0, 1)) == pa.PA_ERR_ARG            # scale factor
    assert call(h, cfg, step=0) == pa.PA_ERR_ARG
    assert call(h, cfg, step=2 ** 32) == pa.PA_ERR_ARG                    # the draws' 32-bit step word
    N[0] = 2 ** 34 + 4                                                    # the draws' 32-bit index word
    assert call(h, cfg) == pa.PA_ERR_ARG
    N[0] = 4096
    hb = _hyper(pa, beta1=0.99, beta2=0.98)                               # beta1^2 >= beta2 with UState
    assert call(hb, cfg) == pa.PA_ERR_ARG
    # the typed entry: the type pairs of pa_step_typed, checked before anything else
    typed = lambda pdt, gdt: L.pa_turbo_step_list_typed(pdt, gdt, 1, P, G, S, N, ctypes.byref(hb), ctypes.byref(cfg),
                                                         1, FAKE + 2 ** 26, 1 << 20, None)
    for pdt, gdt in ((0, 1), (0, 2), (1, 2), (2, 1), (3, 0), (0, -1)):
        assert typed(pdt, gdt) == pa.PA_ERR_ARG, (pdt, gdt)
    for pdt, gdt in ((0, 0), (1, 1), (2, 2), (1, 0), (2, 0)):   # valid pairs reach the beta rule
        assert typed(pdt, gdt) == pa.PA_ERR_ARG, (pdt, gdt)
    assert pa.pa_turbo_state_bytes(1, 1, 4, 131072) == 106508
    assert pa.pa_turbo_state_bytes(0, 0, 4, 10) == 80
    assert pa.pa_turbo_state_bytes(1, 1, 5, 10) == 0
    import oracle
    for bits in (2, 3, 4, 6, 8):
        for block, group in ((32, 1), (32, 32), (128, 64), (256, 2), (1024, 1024), (1024, 16)):
            for cm, cv in ((1, 1), (1, 0), (0, 1)):
                for n in (1, 31, 4096, 100003):
                    got = pa.pa_turbo_layout_bytes(cm, cv, bits, block, group, n)
                    assert got == oracle.turbo_state_bytes(cm, cv, bits, n, block, group), (bits, block, group, n)
                    if (block, group) == (128, 64):
                        assert got == pa.pa_turbo_state_bytes(cm, cv, bits, n)
    assert pa.pa_turbo_layout_bytes(1, 1, 4, 64, 128, 10) == 0
    assert L.pa_turbo_workspace_bytes(1, S, N) == 8 * (16 + 1)           # 16 tile sums, 1 chunk sum
    N[0] = 2048 * 256 + 1                                                 # 2049 tile sums, 2 chunk sums
    assert L.pa_turbo_workspace_bytes(1, S, N) == 8 * (2049 + 2)
    N[0] = 4096


def test_noalloc_refuses_a_list_over_capacity_before_any_device_call(pa):
    """pa_step_list_noalloc checks the list against the capacity of its
    static table on the host (fake device addresses are never touched), and
    the binding's constant is the header's."""
    import re
    with open(os.path.join(ROOT, "include", "pa.h")) as f:
        cap = int(re.search(r"#define PA_NOALLOC_MAX_TENSORS (\d+)", f.read()).group(1))
    assert cap == pa.PA_NOALLOC_MAX_TENSORS
    L = pa.lib()
    k = cap + 1
    P = (ctypes.c_void_p * k)(*[FAKE + 64 * i for i in range(k)])
    G = (ctypes.c_void_p * k)(*[FAKE + (1 << 24) + 64 * i for i in range(k)])
    S = (ctypes.c_void_p * k)(*[FAKE + (1 << 25) + 64 * i for i in range(k)])
    N = (ctypes.c_size_t * k)(*([4] * k))
    h = pa._hyper(dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0))
    assert L.pa_step_list_noalloc(1, 0, 0, k, P, G, S, N, ctypes.byref(h), 1, None) == pa.PA_ERR_CAPACITY
    assert L.pa_step_list_noalloc(1, 0, 0, 2, P, G, S, N, ctypes.byref(h), 0, None) == pa.PA_ERR_ARG


def test_turbo_ledger_matches_gpt2_layer_profile(pa):
    """The library's ledger gives the page's GPT-2-layer figures for the three
    TurboAdam configurations (the shape reading is pinned in the oracle's
    tests by torch's own AdamW)."""
    with open(os.path.join(ROOT, "tests", "golden", "pages_facts.json")) as f:
        prof = json.load(f)["turboadam_gpt2_layer_profile"]
    ns = [math.prod(s) for s in prof["shapes"]]
    for key, (cm, cv) in (("ustate_and_oneq", (1, 1)), ("ustate_only", (1, 0)), ("oneq_only", (0, 1))):
        total = sum(pa.pa_turbo_state_bytes(int(cm and n >= 4096), int(cv and n >= 4096), 4, n) for n in ns)
        assert total == prof["persistent_bytes"][key], key
