"""Print the packed state formats, from the library's own description.

    python -m adamw_step_amd.inspect_formats [--markdown] [--examples]

The table comes from pa_format_info (host code, no device needed) and, like
the reference's format inspection command (Packed AdamW Reference README,
Dependency-light inspection), imports neither torch nor any kernel
framework.  --examples additionally runs a few values through the GPU
codecs (pa_debug_codec) and one packed E4 update of a few parameters
through pa_step, and so needs a GPU and torch (without one it says so and
exits with status 2).
"""
import argparse
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))

MODE_NAMES = {0: "fp32 (two FP32 moments)", 1: "packed E4 (E4M11 m, E4M12 RMS in one word)",
              2: "packed FP16 (binary16 m, binary16 RMS in one word)", 3: "blockwise 8-bit (codes + absmax per 2048)"}


class _Format(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("lanes", ctypes.c_int),
                ("m_sign_bits", ctypes.c_int), ("m_exp_bits", ctypes.c_int),
                ("m_mant_bits", ctypes.c_int), ("m_exp_bias", ctypes.c_int),
                ("r_sign_bits", ctypes.c_int), ("r_exp_bits", ctypes.c_int),
                ("r_mant_bits", ctypes.c_int), ("r_exp_bias", ctypes.c_int),
                ("m_max", ctypes.c_double), ("m_min_normal", ctypes.c_double),
                ("m_min_subnormal", ctypes.c_double), ("r_max", ctypes.c_double),
                ("r_min_normal", ctypes.c_double), ("r_min_subnormal", ctypes.c_double),
                ("block", ctypes.c_int)]


def formats():
    """[(mode, dict), ...] straight from the library, without torch."""
    lib = ctypes.CDLL(os.path.join(HERE, "libpa.so"))
    lib.pa_format_info.argtypes = [ctypes.c_int, ctypes.POINTER(_Format)]
    lib.pa_state_bytes.argtypes = [ctypes.c_int, ctypes.c_size_t]
    lib.pa_state_bytes.restype = ctypes.c_size_t
    out = []
    for mode in range(4):
        f = _Format()
        if lib.pa_format_info(mode, ctypes.byref(f)) != 0:
            raise RuntimeError(f"pa_format_info({mode}) failed")
        d = {name: getattr(f, name) for name, _ in _Format._fields_}
        d["state_bytes_per_2048_params"] = lib.pa_state_bytes(mode, 2048)
        out.append((mode, d))
    return out


def render(markdown=False):
    rows = []
    for mode, d in formats():
        if mode == 3:
            lane = "8-bit code into a 256-entry ascending map; one FP32 absmax per 2048 values"
            rows.append((MODE_NAMES[mode], lane, lane, d["state_bytes_per_2048_params"] / 2048))
            continue
        m = (f"s{d['m_sign_bits']} e{d['m_exp_bits']} m{d['m_mant_bits']}, bias {d['m_exp_bias']}; "
             f"max {d['m_max']:.9g}, min normal {d['m_min_normal']:.6g}, min subnormal {d['m_min_subnormal']:.6g}")
        r = (f"s{d['r_sign_bits']} e{d['r_exp_bits']} m{d['r_mant_bits']}, bias {d['r_exp_bias']}; "
             f"max {d['r_max']:.9g}, min normal {d['r_min_normal']:.6g}, min subnormal {d['r_min_subnormal']:.6g}")
        rows.append((MODE_NAMES[mode], m, r, d["state_bytes_per_2048_params"] / 2048))
    lines = []
    if markdown:
        lines.append("| Mode | First moment lane | Second-moment lane | State bytes / param |")
        lines.append("|---|---|---|---|")
        for name, m, r, b in rows:
            lines.append(f"| {name} | {m} | {r} | {b:g} |")
    else:
        for name, m, r, b in rows:
            lines += [name, f"  first moment : {m}", f"  second lane  : {r}", f"  state bytes  : {b:g} per parameter", ""]
    return "\n".join(lines)


def examples():
    import torch
    import adamw_step_amd as pa
    vals = torch.tensor([0.0, -0.0, 1e-9, 3e-8, 6.1035156e-05, 1e-3, -1e-3, 0.1, 1.5, 1.99951171875, 2.0, 1e9,
                         float("inf"), float("nan")], dtype=torch.float32, device="cuda:0")
    lines = ["value -> E4M11 code (decoded) | E4M12 code (decoded)"]
    out = []
    for lane in (0, 1):
        codes = torch.empty(vals.numel(), dtype=torch.int16, device="cuda:0")
        pa.pa_debug_codec(lane, 0, vals, codes)
        back = torch.empty(vals.numel(), dtype=torch.float32, device="cuda:0")
        pa.pa_debug_codec(lane, 1, codes, back)
        torch.cuda.synchronize()
        out.append((codes.cpu().numpy().view("uint16"), back.cpu().numpy()))
    for i, v in enumerate(vals.cpu().tolist()):
        (cm, dm), (cr, dr) = out[0], out[1]
        lines.append(f"{v:>14.9g} -> 0x{cm[i]:04x} ({dm[i]:.9g}) | 0x{cr[i]:04x} ({dr[i]:.9g})")
    return "\n".join(lines)


def _decode_words(pa, torch, words):
    """(m, r) decoded from packed E4 words on the device."""
    halves = words.view(torch.int16)            # little-endian: low lane first
    lo, hi = halves[0::2].contiguous(), halves[1::2].contiguous()
    out = []
    for lane, codes in ((0, lo), (1, hi)):
        back = torch.empty(codes.numel(), dtype=torch.float32, device=codes.device)
        pa.pa_debug_codec(lane, 1, codes, back)
        out.append(back)
    torch.cuda.synchronize()
    return out[0].cpu().tolist(), out[1].cpu().tolist()


EXAMPLE_HYPER = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
EXAMPLE_STEP = 10


def run_update_example():
    """One packed E4 update of four parameters through the library's step
    (pa_step): the step decodes the prior moments, reconstructs v as RMS
    squared, updates in FP32 and packs afterwards.  Returns host lists: the
    parameters, gradients and prior words, then the new parameters and
    words, and the decoded (m, RMS) of the prior and new words."""
    import torch
    import adamw_step_amd as pa
    dev = "cuda:0"
    p = torch.tensor([0.5, -0.25, 1e-3, 0.0], dtype=torch.float32, device=dev)
    g = torch.tensor([0.01, -0.003, 1e-7, 0.2], dtype=torch.float32, device=dev)
    m0 = torch.tensor([0.004, -0.001, 0.0, 0.01], dtype=torch.float32, device=dev)
    r0 = torch.tensor([0.02, 0.005, 1e-6, 0.05], dtype=torch.float32, device=dev)
    halves = torch.empty(2 * p.numel(), dtype=torch.int16, device=dev)
    for lane, x in ((0, m0), (1, r0)):
        codes = torch.empty(p.numel(), dtype=torch.int16, device=dev)
        pa.pa_debug_codec(lane, 0, x, codes)
        halves[lane::2] = codes
    w = halves.view(torch.int32)
    out = {"param": p.cpu().tolist(), "grad": g.cpu().tolist(),
           "word": [int(x) & 0xFFFFFFFF for x in w.cpu().tolist()]}
    out["m"], out["rms"] = _decode_words(pa, torch, w)
    pa.pa_step(pa.PA_PACKED_E4, p, g, w, EXAMPLE_HYPER, EXAMPLE_STEP)
    torch.cuda.synchronize()
    out["new_param"] = p.cpu().tolist()
    out["new_word"] = [int(x) & 0xFFFFFFFF for x in w.cpu().tolist()]
    out["new_m"], out["new_rms"] = _decode_words(pa, torch, w)
    return out


def update_example():
    """The update inspection as text (Packed AdamW Reference README,
    Dependency-light inspection)."""
    r = run_update_example()
    h = EXAMPLE_HYPER
    lines = [f"one packed E4 update, step {EXAMPLE_STEP}, lr {h['lr']}, betas ({h['beta1']}, {h['beta2']}), "
             f"eps {h['eps']}, weight decay {h['weight_decay']}",
             "param, grad, prior word (m, rms) -> new param, new word (m, rms)"]
    for i in range(len(r["param"])):
        lines.append(f"{r['param'][i]:>10.6g} {r['grad'][i]:>10.3g}  0x{r['word'][i]:08x} "
                     f"({r['m'][i]:.6g}, {r['rms'][i]:.6g}) -> {r['new_param'][i]:>13.9g}  "
                     f"0x{r['new_word'][i]:08x} ({r['new_m'][i]:.6g}, {r['new_rms'][i]:.6g})")
    return "\n".join(lines)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--markdown", action="store_true")
    ap.add_argument("--examples", action="store_true",
                    help="also encode sample values and run one update on the GPU")
    a = ap.parse_args(argv)
    have_gpu = False
    if a.examples:
        # torch first: the library must bind to the HIP runtime torch loads,
        # so it is imported before the table below loads the library.
        try:
            import torch
            have_gpu = torch.cuda.is_available()
        except ImportError:
            pass
    print(render(markdown=a.markdown))
    if a.examples:
        if not have_gpu:
            print("--examples runs the library's codec and step on a GPU; none is available here", file=sys.stderr)
            return 2
        print(examples())
        print()
        print(update_example())
    return 0


if __name__ == "__main__":
    sys.exit(main())
