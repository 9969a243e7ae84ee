"""GPU lane codecs against the oracle's, through the C ABI (pa_debug_codec):
every code of every lane decoded, every rounding boundary (with its FP32
neighbours), whole FP32 binades and random bit patterns encoded, and then
every one of the 2^32 binary32 bit patterns encoded."""
import numpy as np
import pytest

import oracle
from gpu_util import banner, to_dev, to_host
from pins import boundary_set, random_patterns, specials

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pa():
    import adamw_step_amd as pa_mod
    pa_mod.lib()
    return pa_mod


def _decode_gpu(pa, lane, codes):
    import torch
    inp = to_dev(codes.astype(np.uint16))
    out = torch.empty(codes.size, dtype=torch.float32, device=inp.device)
    pa.pa_debug_codec(lane, 1, inp, out)
    torch.cuda.synchronize()
    return to_host(out)


def _encode_gpu(pa, lane, x):
    import torch
    inp = to_dev(x.astype(np.float32))
    out = torch.empty(x.size, dtype=torch.int16, device=inp.device)
    pa.pa_debug_codec(lane, 0, inp, out)
    torch.cuda.synchronize()
    return to_host(out, np.uint16)


def _binade(e):
    return ((np.uint32((e + 127) << 23)) + np.arange(1 << 23, dtype=np.uint32)).view(np.float32)


@pytest.mark.parametrize("lane", [0, 1, 2, 3])
def test_decode_every_code(pa, lane):
    banner(f"decode all codes lane {lane}")
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = _decode_gpu(pa, lane, codes)
    want = oracle.decode(lane, codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


@pytest.mark.parametrize("lane", [0, 1, 2])
def test_encode_boundaries_and_random(pa, lane):
    banner(f"encode boundary sets lane {lane}")
    if lane == 0:
        table = oracle.decode(0, np.arange(0x8000, dtype=np.uint16)).astype(np.float64)
        extra = [2.0]
    elif lane == 1:
        table = oracle.decode(1, np.arange(0x10000, dtype=np.uint16)).astype(np.float64)
        extra = [2.0]
    else:
        table = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
        extra = [65536.0]
    x = np.concatenate([boundary_set(np.append(table, extra)), random_patterns(1 << 24, 100 + lane),
                        specials(), _binade(-15), _binade(-27), _binade(0), -_binade(-20)])
    got = _encode_gpu(pa, lane, x)
    want = oracle.encode(lane, x)
    if lane == 2:
        nan = np.isnan(x)
        np.testing.assert_array_equal(got[~nan], want[~nan])
        assert np.all(((got[nan] & 0x7C00) == 0x7C00) & ((got[nan] & 0x3FF) != 0))
    else:
        np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("lane", [0, 1])
def test_decode_encode_identity_on_device(pa, lane):
    banner(f"identity lane {lane}")
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    back = _encode_gpu(pa, lane, _decode_gpu(pa, lane, codes))
    np.testing.assert_array_equal(back, codes)


@pytest.mark.parametrize("lane", [0, 1, 2])
def test_encode_every_float(pa, lane):
    """Each lane's GPU encoder equals the oracle's nearest-in-table encoder on
    all 2^32 binary32 bit patterns (binary16 NaNs by class and sign)."""
    import torch
    chunk = 1 << 28
    bad = 0
    for c in range(1 << 4):
        banner(f"encode lane {lane} chunk {c}/16")
        bits = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device="cuda:0")
        x = bits.to(torch.int32).view(torch.float32)        # wraps to the bit pattern
        out = torch.empty(chunk, dtype=torch.int16, device="cuda:0")
        pa.pa_debug_codec(lane, 0, x, out)
        torch.cuda.synchronize()
        hx = to_host(x)
        got = to_host(out, np.uint16)
        want = oracle.encode(lane, hx)
        if lane == 2:
            nan = np.isnan(hx)
            bad += int((got[~nan] != want[~nan]).sum())
            assert np.all(((got[nan] & 0x7C00) == 0x7C00) & ((got[nan] & 0x3FF) != 0))
            assert np.array_equal(got[nan] >> 15, want[nan] >> 15)
        else:
            bad += int((got != want).sum())
        del bits, x, out
    assert bad == 0, f"lane {lane}: {bad} codes differ from the oracle"


def test_bf16_encode_every_float(pa):
    """The GPU's bfloat16 rounding (gfx950's conversion instruction, used for
    16-bit parameters, the blockwise output and TurboAdam's group means)
    equals the oracle's nearest-even bfloat16 on all 2^32 bit patterns; NaN
    stays NaN with its sign."""
    import torch
    chunk = 1 << 28
    bad = 0
    for c in range(1 << 4):
        banner(f"bf16 encode chunk {c}/16")
        bits = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device="cuda:0")
        x = bits.to(torch.int32).view(torch.float32)        # wraps to the bit pattern
        out = torch.empty(chunk, dtype=torch.int16, device="cuda:0")
        pa.pa_debug_codec(3, 0, x, out)
        torch.cuda.synchronize()
        hx = to_host(x)
        got = to_host(out, np.uint16)
        want = oracle.encode(3, hx)
        nan = np.isnan(hx)
        bad += int((got[~nan] != want[~nan]).sum())
        assert np.all(((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0))
        assert np.array_equal(got[nan] >> 15, want[nan] >> 15)
        del bits, x, out
    assert bad == 0, f"{bad} bfloat16 roundings differ from the oracle"


def test_sqrt_every_float(pa):
    """The GPU path's square root equals the host's IEEE square root
    (numpy, correctly rounded) on all 2^32 bit patterns; NaN by class."""
    import torch
    chunk = 1 << 28
    bad = 0
    for c in range(1 << 4):
        banner(f"sqrt chunk {c}/16")
        bits = torch.arange(c * chunk, (c + 1) * chunk, dtype=torch.int64, device="cuda:0")
        x = bits.to(torch.int32).view(torch.float32)        # wraps to the bit pattern
        out = torch.empty_like(x)
        pa.pa_debug_sqrt(x, out)
        torch.cuda.synchronize()
        hx = to_host(x)
        got = to_host(out)
        with np.errstate(invalid="ignore"):
            want = np.sqrt(hx)
        nan = np.isnan(want)
        assert np.array_equal(np.isnan(got), nan)
        bad += int((got[~nan].view(np.uint32) != want[~nan].view(np.uint32)).sum())
        del bits, x, out
    assert bad == 0, f"{bad} square roots differ from IEEE"


def test_inspect_formats_examples(pa):
    """The inspection command's GPU examples: 1.5 is E4M11 0x7c00 (exponent 15,
    mantissa 1024) and E4M12 0xf800; 2.0 saturates to 0x7fff / 0xffff."""
    from adamw_step_amd.inspect_formats import examples
    banner("inspect_formats --examples")
    text = examples()
    line15 = [l for l in text.splitlines() if l.strip().startswith("1.5 ")][0]
    assert "0x7c00" in line15 and "0xf800" in line15
    line2 = [l for l in text.splitlines() if l.strip().startswith("2 ")][0]
    assert "0x7fff" in line2 and "0xffff" in line2


def test_inspect_formats_update_example(pa):
    """The inspection command's one-update example against the oracle: the
    prior words it builds decode to its stated moments' codes, and the new
    parameters and words equal the oracle's packed E4 step on the same
    inputs, bit for bit."""
    from adamw_step_amd.inspect_formats import EXAMPLE_HYPER, EXAMPLE_STEP, run_update_example
    banner("inspect_formats update example")
    r = run_update_example()
    p = np.array(r["param"], np.float32)
    g = np.array(r["grad"], np.float32)
    words = np.array(r["word"], np.uint32)
    h = EXAMPLE_HYPER
    sc = oracle.scalars(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], EXAMPLE_STEP)
    oracle.step_packed(1, p, g, words, sc)
    assert np.array_equal(np.array(r["new_word"], np.uint32), words)
    assert np.array_equal(np.array(r["new_param"], np.float32).view(np.uint32), p.view(np.uint32))
    assert r["new_word"] != r["word"]
