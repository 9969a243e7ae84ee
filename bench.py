"""Benchmark of the packed-AdamW step on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload llama-7b] [--mode e4]

A step is one pa_step_list call (one persistent launch) over the whole
parameter list of the workload, made through a StepList (the list is
validated and marshalled once, as an optimizer object would hold it), with parameters, gradients and state already
resident in HBM.  Default workload: the 291-tensor Llama-7B list
(6,738,415,616 FP32 parameters, packed E4 state), gradients drawn once on the
device and reused, 3 warm-up and 20 timed steps.

Prints one JSON line: params/s over the timed steps (whole job), the
roofline of the step kernel (algorithmic bytes per launch over the mean
launch time from HIP events on the launch stream, against 8 TB/s), and the
CPU oracle's throughput on a bounded sample of the same workload.

Other flags:
  --no-cpu-baseline       skip the oracle timing
  --probe                 after the step, time the step-layout probes and
                          references (see step_layout_ceilings) in any mode
  --calibrate-copy BYTES  only run the plain copy probe (for counter calibration)
  --train-gpt             instead: time a synthetic-token training step of the
                          gpt-11m model (trainer/) with each optimizer and
                          report the optimizer's share of the step
  --layout plain          allocate parameters, gradients and state back to
                          back, as PackedAdamW does (default: state one HBM
                          region below the parameters, see build_workload)
  --mode turbo            the TurboAdam compressed-state step (UState first
                          moment, 4-bit 1Q second moment; tensors below 4096
                          values keep FP32 moments, as the page's thresholds)
  --turbo-bits B          with --mode turbo: 1Q index width, 2, 3, 4, 6 or 8
  --turbo-block B, --turbo-group G
                          with --mode turbo: 1Q block (32 to 1024) and UState
                          group (dividing it); defaults 128 and 64
  --turbo-general         with --mode turbo: run the general kernel even at
                          the default layout
  --count-nonfinite       count non-finite values, as the optimizers do by
                          default (the counting kernel variant)
  --mode gradstats        instead of the step: time the gradient pre-pass
                          (pa_grad_stats_list: sum of squares, non-finite
                          count and clip coefficient) over the workload's
                          gradients
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "packed-AdamW step: params/s and achieved HBM GB/s (% of 8 TB/s) at 7B"
PEAK_GBPS = 8000.0
# Vector ALU peak of MI355X in G lane-operations per second: its FP32
# vector rate, 157.3 TFLOP/s (256 CUs x 2.4 GHz x 256 flops), counting a
# lane's FMA as two flops, so 128 lane-operations per CU per clock.  One
# wave64 instruction per SIMD every four cycles (half of this) is not a
# ceiling on gfx950: the general TurboAdam kernel's counters exceed it.
PEAK_VALU_GLANE = 256 * 128 * 2.4
BYTES_PER_PARAM = {"e4": 20, "fp16": 20, "fp32": 28, "blockwise8": 14, "gradstats": 4, "turbo": None}
WORKLOADS = {"single-262k": 1, "gpt-11m": 2, "gpt2-small-124m": 3, "llama-7b": 4, "blockwise-268m": 5,
             "gpt2-layer-7m": 6}
# Device sources each kernel family is compiled from: a stored counter
# reading stays valid while these bytes are unchanged.
KERNEL_SOURCES = {
    "elementwise": ("adamw_step_amd/csrc/kernels.hpp", "adamw_step_amd/csrc/codec.hpp",
                    "adamw_step_amd/csrc/pa_api.hip", "adamw_step_amd/build.py"),
    "turbo": ("adamw_step_amd/csrc/kernels.hpp", "adamw_step_amd/csrc/codec.hpp", "adamw_step_amd/csrc/turbo.hpp",
              "adamw_step_amd/csrc/pow2.hpp", "adamw_step_amd/csrc/pa_api.hip", "adamw_step_amd/build.py"),
}


def kernel_sha(family="elementwise"):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def probe_lib():
    import ctypes
    import adamw_step_amd as pa
    pa.lib()
    path = os.path.join(ROOT, "adamw_step_amd", "libpa_probe.so")
    L = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.pa_probe_copy.argtypes = [vp, vp, sz, ctypes.c_int, vp]
    L.pa_probe_read.argtypes = [vp, sz, vp, vp]
    L.pa_probe_write.argtypes = [vp, sz, vp]
    L.pa_probe_mix.argtypes = [vp, vp, vp, sz, ctypes.c_int, vp]
    L.pa_probe_runtime_copy.argtypes = [vp, vp, sz, vp]
    return L


def time_probe(fn, reps):
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        s.record()
        fn()
        e.record()
        e.synchronize()
        ts.append(s.elapsed_time(e))
    return sorted(ts)[len(ts) // 2]


def step_layout_ceilings(L, stream_bytes, layout="regions"):
    """Ceilings of the packed step's traffic on this HBM, in the benchmark's
    layout: three streams of `stream_bytes` (the step's p, g and w), the
    first two at the start of device memory and the third one HBM region
    further on in allocation order (layout "regions"), or all three back to
    back (layout "plain").

    This library's probes (libpa_probe.so, one tile per workgroup in tile
    order, as the step): a nontemporal read of one stream, a write of one
    stream, and the step's 3-read/2-write mix in place with no arithmetic
    and with 80 binary32 instructions per value (the step issues about
    78).  References that are not code of this library, on the same
    streams: torch's fill_ (one write stream), the HIP runtime's
    device-to-device copy (one read and one write stream), torch's add of
    two streams into a third (two reads, one write), and torch's sum (one
    read).  `read_then_write_bound_gbps` is the rate of the step's bytes if
    its reads ran at the best read rate measured here and its writes, one
    after the other, at the best write rate: 5 / (3 / read + 2 / write)."""
    import torch
    st = torch.cuda.current_stream().cuda_stream
    stream_bytes -= stream_bytes % 16
    n16 = stream_bytes // 16
    a = torch.zeros(stream_bytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.zeros_like(a)
    spacer = None
    if layout == "regions":
        spacer = torch.empty(max(region_bytes() - 2 * stream_bytes, 0), dtype=torch.uint8, device="cuda:0")
    c = torch.zeros_like(a)
    del spacer
    torch.cuda.empty_cache()
    sink = torch.zeros(4, dtype=torch.float32, device="cuda:0")

    def gbps(moved, fn):
        return round(moved / time_probe(fn, 5) / 1e6, 1)

    def ok(rc):
        assert rc == 0, "probe launch failed"

    S = stream_bytes
    res = {"stream_bytes": S,
           "read_nt_gbps": gbps(S, lambda: ok(L.pa_probe_read(a.data_ptr(), n16, sink.data_ptr(), st))),
           "write_gbps": gbps(S, lambda: ok(L.pa_probe_write(c.data_ptr(), n16, st))),
           "mix_3r2w_gbps": gbps(5 * S, lambda: ok(L.pa_probe_mix(a.data_ptr(), b.data_ptr(), c.data_ptr(), n16, 0,
                                                                  st))),
           "mix_3r2w_80valu_gbps": gbps(5 * S, lambda: ok(L.pa_probe_mix(a.data_ptr(), b.data_ptr(), c.data_ptr(),
                                                                         n16, 80, st)))}
    refs = {"torch_fill_gbps": gbps(S, lambda: c.fill_(1.0)),
            "hip_memcpy_d2d_gbps": gbps(2 * S, lambda: ok(L.pa_probe_runtime_copy(a.data_ptr(), c.data_ptr(), S, st))),
            "torch_add_2r1w_gbps": gbps(3 * S, lambda: torch.add(a, b, out=c)),
            "torch_sum_gbps": gbps(S, lambda: a.sum())}
    res["references"] = refs
    best_read = max(res["read_nt_gbps"], refs["torch_sum_gbps"])
    best_write = max(res["write_gbps"], refs["torch_fill_gbps"])
    res["read_then_write_bound_gbps"] = round(5.0 / (3.0 / best_read + 2.0 / best_write), 1)
    del a, b, c, sink
    torch.cuda.empty_cache()
    return res


def calibrate_copy(nbytes):
    import torch
    L = probe_lib()
    st = torch.cuda.current_stream().cuda_stream
    a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        assert L.pa_probe_copy(a.data_ptr(), b.data_ptr(), nbytes, 2048, st) == 0
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 3}), flush=True)


def build_blockwise(cfg, layout="regions"):
    """The blockwise workload.  layout "regions" puts the state the step
    writes (codes, absmax values, BF16 output) one HBM region below the
    parameters and gradients in allocation order."""
    import torch
    import workloads
    n = workloads.total(cfg)
    nb = n // 2048
    qm, qv = workloads.code_maps()
    zero_m = int((torch.from_numpy(qm) == 0).nonzero()[0])
    p = torch.empty(n, dtype=torch.float32, device="cuda:0")
    g = torch.empty(n, dtype=torch.float32, device="cuda:0")
    spacer = None
    if layout == "regions":
        spacer = torch.empty(max(region_bytes() - 8 * n, 0), dtype=torch.uint8, device="cuda:0")
    state = (torch.full((n,), zero_m, dtype=torch.uint8, device="cuda:0"),
             torch.zeros(nb, dtype=torch.float32, device="cuda:0"),
             torch.zeros(n, dtype=torch.uint8, device="cuda:0"),
             torch.zeros(nb, dtype=torch.float32, device="cuda:0"),
             torch.from_numpy(qm).to("cuda:0"), torch.from_numpy(qv).to("cuda:0"),
             torch.empty(n, dtype=torch.int16, device="cuda:0"))
    del spacer
    torch.cuda.empty_cache()
    workloads.device_fill_params(cfg, [p])
    workloads.device_fill_grads(cfg, 1, [g])
    torch.cuda.synchronize()
    return [n], [p], [g], [state]


def region_bytes():
    """One HBM region: a third of the device memory.  Measured on MI355X
    (288 GB of HBM3E): in allocation order the device memory falls into three
    equal regions; with a persistent launch the step ran about 13% faster
    when its written streams (parameters and state) lay in different
    regions.  With one tile per workgroup the layouts converge after a few
    processes on a box, but in the first ones the back-to-back layout still
    runs up to 10% slower."""
    import torch
    return torch.cuda.get_device_properties(0).total_memory // 3


def build_workload(cfg, mode, param_dtype="fp32", layout="regions"):
    """Parameters, gradients and state of the workload in HBM.  layout
    "regions" allocates the streams the step writes one HBM region apart in
    allocation order (parameters, gradients, then each state stream one
    region below the parameters, with a temporary spacer allocation in
    between); "plain" allocates them back to back."""
    import torch
    import workloads
    if mode == "blockwise8":
        return build_blockwise(cfg, layout)
    sizes = workloads.sizes(cfg)
    log(f"allocating {workloads.NAMES[cfg]}: {len(sizes)} tensors, {sum(sizes)} params, layout {layout}")
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[param_dtype]
    esz = torch.empty(0, dtype=dt).element_size()
    ps = [torch.empty(n, dtype=dt, device="cuda:0") for n in sizes]
    gs = [torch.empty(n, dtype=dt, device="cuda:0") for n in sizes]
    spacers, placed = [], 2 * esz * sum(sizes)

    def state_stream():
        nonlocal placed
        if layout == "regions":
            region = region_bytes()
            gap = region * (len(spacers) + 1) - placed
            if gap > 0:
                spacers.append(torch.empty(gap, dtype=torch.uint8, device="cuda:0"))
                placed += gap
        out = [torch.zeros(n, dtype=torch.int32 if mode != "fp32" else torch.float32, device="cuda:0")
               for n in sizes]
        placed += 4 * sum(sizes)
        return out

    if mode == "fp32":
        ms = state_stream()
        vs = state_stream()
        states = list(zip(ms, vs))
    else:
        states = state_stream()
    del spacers
    torch.cuda.empty_cache()
    workloads.device_fill_params(cfg, ps)
    workloads.device_fill_grads(cfg, 1, gs)
    torch.cuda.synchronize()
    return sizes, ps, gs, states


def cpu_baseline(cfg, mode, ps, gs, states, budget_params, one_core_params=64 << 20):
    """Time the oracle (as it stands) on the host cores: one step over the
    workload's whole list when it holds at most `budget_params` parameters
    (single-262k, gpt-11m, gpt2-small-124m, blockwise-268m), else over the
    leading tensors of the list up to that many; then the same oracle on one
    core over the first `one_core_params` values of that sample (the whole
    sample if smaller).  Inputs are the device buffers as the benchmark left
    them (any valid state will do for timing)."""
    import numpy as np
    import oracle
    import workloads
    h = workloads.HYPER
    sc = oracle.scalars(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], 1)
    picked, total = [], 0
    for k in range(len(ps)):
        n = ps[k].numel()
        if total + n > budget_params and picked:
            break
        picked.append(k)
        total += n
    whole = len(picked) == len(ps)
    names = [workloads.shapes(cfg)[k][0] for k in picked]
    hp = [ps[k].cpu().numpy() for k in picked]
    hg = [gs[k].cpu().numpy() for k in picked]
    if mode == "blockwise8":
        mc, ma, vc, va, qm, qv, _ = states[0]
        hs = [(mc.cpu().numpy(), ma.cpu().numpy(), vc.cpu().numpy(), va.cpu().numpy(), qm.cpu().numpy(),
               qv.cpu().numpy())]
    elif mode == "fp32":
        hs = [(states[k][0].cpu().numpy(), states[k][1].cpu().numpy()) for k in picked]
    else:
        hs = [states[k].cpu().numpy().view(np.uint32) for k in picked]

    def step(p, g, st, lo, hi):
        # contiguous views: the oracle updates the host copies in place
        if mode == "blockwise8":
            mc, ma, vc, va, qm, qv = st
            nb0, nb1 = lo // 2048, hi // 2048
            out = np.empty(hi - lo, np.uint16)
            oracle.step_blockwise(p[lo:hi], g[lo:hi], mc[lo:hi], ma[nb0:nb1], vc[lo:hi], va[nb0:nb1], qm, qv, out, sc)
        elif mode == "fp32":
            oracle.step_fp32(p[lo:hi], g[lo:hi], st[0][lo:hi], st[1][lo:hi], sc)
        else:
            oracle.step_packed(oracle.PACKED_E4 if mode == "e4" else oracle.PACKED_F16, p[lo:hi], g[lo:hi],
                               st[lo:hi], sc)

    t0 = time.perf_counter()
    for i in range(len(picked)):
        step(hp[i], hg[i], hs[i], 0, hp[i].size)
    dt = time.perf_counter() - t0
    cores = oracle.num_threads()
    k = min(hp[0].size, one_core_params)
    if mode == "blockwise8":
        k -= k % 2048
    oracle.set_num_threads(1)
    try:
        t1 = time.perf_counter()
        step(hp[0], hg[0], hs[0], 0, k)
        dt1 = time.perf_counter() - t1
    finally:
        oracle.set_num_threads(cores)
    what = (f"one step over the whole list ({len(picked)} tensors, {total} params)" if whole else
            f"one step over the first {len(picked)} tensors of the list ({names[0]}..{names[-1]}, {total} params)")
    return {"value": round(total / dt, 1), "unit": "params/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{what}, {dt:.1f} s wall",
            "one_core": {"value": round(k / dt1, 1), "unit": "params/s",
                         "sample": f"one step over the first {k} values of {names[0]}, {dt1:.1f} s wall"}}


def run_gradstats(args, cfg):
    """Time the gradient pre-pass over the workload's gradient list."""
    import torch
    import adamw_step_amd as pa
    import workloads
    sizes = workloads.sizes(cfg)
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[args.param_dtype]
    log(f"allocating {workloads.NAMES[cfg]} gradients: {len(sizes)} tensors, {sum(sizes)} values")
    gs = [torch.empty(n, dtype=dt, device="cuda:0") for n in sizes]
    workloads.device_fill_grads(cfg, 1, gs)
    s = torch.zeros(1, dtype=torch.float64, device="cuda:0")
    nf = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    clip = torch.zeros(1, dtype=torch.float32, device="cuda:0")
    stats = pa.GradStats(gs)
    for _ in range(args.warmup):
        stats.run(s, nf, clip, max_norm=1.0)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        evs[k][0].record(stream)
        stats.run(s, nf, clip, max_norm=1.0)
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    mean_ms = sum(launch_ms) / len(launch_ms)
    n = sum(sizes)
    algo = n * (4 if args.param_dtype == "fp32" else 2)
    achieved = algo / (mean_ms / 1e3) / 1e9
    log(f"timed {args.steps} pre-passes: {mean_ms:.3f} ms/call (events), sumsq {s.item():.6g}, "
        f"nonfinite {int(nf.item())}, clip {clip.item():.6g}")
    out = {"metric": "gradient pre-pass (sum of squares, non-finite count, clip coefficient): params/s",
           "value": round(n * args.steps / elapsed, 1), "unit": "params/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f64 accumulation of " + args.param_dtype + " grads",
           "data": "synthetic",
           "config": {"workload": args.workload, "params": n, "tensors": len(sizes), "mode": "gradstats",
                      "grad_dtype": args.param_dtype},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                        "frac": round(achieved / PEAK_GBPS, 4), "traffic": None,
                        "kernel": "grad_stats_list + grad_stats_finalize", "algorithmic_bytes_per_launch": algo,
                        "mean_launch_ms": round(mean_ms, 4), "kernel_sha": kernel_sha()}}
    if not args.no_cpu_baseline and args.param_dtype == "fp32":
        import oracle
        picked, total = [], 0
        for g in gs:
            if total + g.numel() > args.cpu_sample_params and picked:
                break
            picked.append(g)
            total += g.numel()
        host = [g.cpu().numpy() for g in picked]
        t1 = time.perf_counter()
        oracle.grad_stats(0, host)
        dt_cpu = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": round(total / dt_cpu, 1), "unit": "params/s", "cores": oracle.num_threads(),
                               "kind": "oracle", "sample": f"the first {len(picked)} gradient tensors "
                               f"({total} values), exact accumulation, {dt_cpu:.1f} s wall"}
    print(json.dumps(out), flush=True)


def run_turbo(args, cfg):
    """Time the TurboAdam step over the workload's tensor list."""
    import torch
    import adamw_step_amd as pa
    import workloads
    sizes = workloads.sizes(cfg)
    log(f"allocating {workloads.NAMES[cfg]} with TurboAdam state: {len(sizes)} tensors, {sum(sizes)} params")
    dt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[args.param_dtype]
    esz = 4 if args.param_dtype == "fp32" else 2
    ps = [torch.empty(n, dtype=dt, device="cuda:0") for n in sizes]
    gs = [torch.empty(n, dtype=dt, device="cuda:0") for n in sizes]
    spacer = None
    if args.layout == "regions":
        spacer = torch.empty(max(region_bytes() - 2 * esz * sum(sizes), 0), dtype=torch.uint8, device="cuda:0")
    B, G = args.turbo_block, args.turbo_group
    general = args.turbo_general or (B, G) != (128, 64)
    states = [pa.TurboState(n, "cuda:0", compress_m=n >= 4096, compress_v=n >= 4096, v_bits=args.turbo_bits,
                            tensor_id=i, block_size=B, m_block_size=G)
              for i, n in enumerate(sizes)]
    del spacer
    torch.cuda.empty_cache()
    workloads.device_fill_params(cfg, ps)
    workloads.device_fill_grads(cfg, 1, gs)
    tl = pa.TurboList(ps, gs, states, v_bits=args.turbo_bits, block_size=B, m_block_size=G,
                      general=args.turbo_general)
    h = dict(workloads.HYPER)
    if args.count_nonfinite:   # the optimizers' default: the kernel variant that counts
        h["nonfinite"] = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    torch.cuda.synchronize()
    t = 0
    for _ in range(args.warmup):
        t += 1
        tl.step(h, t)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for k in range(args.steps):
        t += 1
        evs[k][0].record(stream)
        tl.step(h, t)
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    mean_ms = sum(launch_ms) / len(launch_ms)
    n = sum(sizes)
    state = sum(st.nbytes() for st in states)
    tiles = sum((k + 255) // 256 for k in sizes if k >= 4096)   # residual partial sums, either kernel
    algo = 3 * esz * n + 2 * state + 16 * tiles   # p, g read; p written; state read and written; residual sums
    achieved = algo / (mean_ms / 1e3) / 1e9
    log(f"timed {args.steps} TurboAdam steps: {mean_ms:.3f} ms/step (events), state {state / n:.4f} B/param")
    # The step is bound by vector ALU issue, not HBM: its roofline is the
    # VALU lane-instruction rate, from the instructions per parameter that
    # the counters measured for this kernel source (profiles/), if current.
    valu = None
    vpath = os.path.join(ROOT, "profiles", f"valu_{args.workload}_turbo.json")
    if (os.path.exists(vpath) and args.turbo_bits == 4 and not args.count_nonfinite and not general
            and args.param_dtype == "fp32"):
        with open(vpath) as f:
            vj = json.load(f)
        if vj.get("kernel_sha") == kernel_sha("turbo"):
            valu = vj["valu_lane_instr_per_param"]
    out = {"metric": f"TurboAdam step (UState + {args.turbo_bits}-bit 1Q state): params/s", "value": round(n * args.steps / elapsed, 1),
           "unit": "params/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(elapsed * 1e3 / args.steps, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None,
           "dtype": "f32" if args.param_dtype == "fp32" else f"f32 math, {args.param_dtype} params and grads",
           "data": "synthetic",
           "config": {"workload": args.workload, "params": n, "tensors": len(sizes), "mode": f"turbo-ustate-1q{args.turbo_bits}",
                      "param_dtype": args.param_dtype,
                      "block_size": B, "m_block_size": G,
                      "state_bytes": state, "state_bits_per_param": round(8 * state / n, 4),
                      "layout": args.layout, "count_nonfinite": bool(args.count_nonfinite)},
           "roofline": ({"bound": "alu", "achieved": round(valu * n / (mean_ms / 1e3) / 1e9, 1),
                         "peak": PEAK_VALU_GLANE, "unit": "G VALU lane-instr/s",
                         "frac": round(valu * n / (mean_ms / 1e3) / 1e9 / PEAK_VALU_GLANE, 4),
                         "valu_lane_instr_per_param": valu} if valu is not None else
                        {"bound": "alu", "achieved": None, "peak": PEAK_VALU_GLANE, "unit": "G VALU lane-instr/s",
                         "frac": None}) | {
                        "hbm_achieved_gbps": round(achieved, 1), "hbm_frac": round(achieved / PEAK_GBPS, 4),
                        "traffic": None,
                        "kernel": f"{'turbo_general' if general else 'turbo_list'}<{args.turbo_bits}, "
                                  f"{'true' if args.count_nonfinite else 'false'}, "
                                  f"{'false' if args.param_dtype == 'fp32' else 'true'}> + turbo_chunks + turbo_reduce",
                        "algorithmic_bytes_per_launch": algo, "mean_launch_ms": round(mean_ms, 4),
                        "kernel_sha": kernel_sha("turbo")}}
    if not args.no_cpu_baseline and args.param_dtype == "fp32":
        import numpy as np
        import oracle
        picked, total = [], 0
        for i, k in enumerate(sizes):
            if total + k > args.cpu_sample_params // 8 and picked:
                break
            picked.append(i)
            total += k
        hp = [ps[i].cpu().numpy() for i in picked]
        hg = [gs[i].cpu().numpy() for i in picked]
        hs = [oracle.TurboState(sizes[i], sizes[i] >= 4096, sizes[i] >= 4096, args.turbo_bits, B, G) for i in picked]
        sc = oracle.scalars(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], 1)
        ts = oracle.turbo_scalars(h["beta1"], h["beta2"], 1)
        t1 = time.perf_counter()
        for j, i in enumerate(picked):
            oracle.turbo_step(hp[j], hg[j], hs[j], sc, ts, 1, tensor_id=i)
        dt_cpu = time.perf_counter() - t1
        out["cpu_baseline"] = {"value": round(total / dt_cpu, 1), "unit": "params/s", "cores": 1, "kind": "oracle",
                               "sample": f"one step over the first {len(picked)} tensors ({total} params), "
                                         f"{dt_cpu:.1f} s wall, single-threaded"}
    print(json.dumps(out), flush=True)


def load_traffic(workload, mode):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}_{mode}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != kernel_sha():
        return None
    return t.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama-7b", choices=sorted(WORKLOADS))
    ap.add_argument("--mode", default="e4", choices=sorted(BYTES_PER_PARAM))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the step-layout bandwidth probes after the timed region (E4 mode)")
    ap.add_argument("--cpu-sample-params", type=int, default=1_300_000_000)
    ap.add_argument("--probe", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0)
    ap.add_argument("--train-gpt", action="store_true")
    ap.add_argument("--param-dtype", default="fp32", choices=["fp32", "bf16", "fp16"],
                    help="element type of parameters and gradients (state unchanged)")
    ap.add_argument("--turbo-bits", type=int, default=4, choices=[2, 3, 4, 6, 8],
                    help="1Q index width of the TurboAdam mode (the page's default is 4)")
    ap.add_argument("--turbo-block", type=int, default=128, help="1Q block of the TurboAdam mode (32 to 1024)")
    ap.add_argument("--turbo-group", type=int, default=64, help="UState group of the TurboAdam mode (divides the block)")
    ap.add_argument("--turbo-general", action="store_true",
                    help="run the general TurboAdam kernel even at the default layout")
    ap.add_argument("--count-nonfinite", action="store_true",
                    help="count non-finite values, as the optimizers do by default (the counting kernel)")
    ap.add_argument("--layout", default="regions", choices=["regions", "plain"],
                    help="HBM placement of the state streams (see build_workload)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this benchmark runs on one GPU only (one process, one device), "
              "so --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import adamw_step_amd as pa
    import workloads

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.train_gpt:
        from trainer.loop import measure
        rows = [measure(kind, steps=args.steps, warmup=args.warmup) for kind in ("e4", "fp32", "turbo", "torch-fused")]
        for r in rows:
            r["opt_share"] = round(r["opt_ms"] / r["step_ms"], 4)
            log(f"train {r['optimizer']}: {r['step_ms']:.3f} ms/step, optimizer {r['opt_ms']:.3f} ms")
        print(json.dumps({"metric": "gpt-11m synthetic training step: optimizer share", "unit": "ms",
                          "n_gpus": 1, "data": "synthetic", "rows": rows}), flush=True)
        return

    cfg = WORKLOADS[args.workload]
    mode = args.mode
    if mode == "turbo":
        if cfg == 5:
            print("bench.py: the turbo mode runs on the list workloads", file=sys.stderr)
            sys.exit(2)
        run_turbo(args, cfg)
        return
    if mode == "gradstats":
        if cfg == 5:
            print("bench.py: the gradstats mode runs on the list workloads", file=sys.stderr)
            sys.exit(2)
        run_gradstats(args, cfg)
        return
    if (mode == "blockwise8") != (cfg == 5):
        print("bench.py: the blockwise8 mode runs on the blockwise-268m workload and only there", file=sys.stderr)
        sys.exit(2)
    if mode == "blockwise8" and args.param_dtype != "fp32":
        print("bench.py: the blockwise8 mode takes FP32 parameters", file=sys.stderr)
        sys.exit(2)
    sizes, ps, gs, states = build_workload(cfg, mode, args.param_dtype, args.layout)
    n_params = sum(sizes)
    h = dict(workloads.HYPER)
    if args.count_nonfinite:   # the optimizers' default: the kernel variant that counts
        h["nonfinite"] = torch.zeros(1, dtype=torch.int64, device="cuda:0")
    t = 0
    prepared = None if mode == "blockwise8" else pa.StepList(mode, ps, gs, states)

    def step():
        nonlocal t
        t += 1
        if mode == "blockwise8":
            pa.pa_step(mode, ps[0], gs[0], states[0], h, t)
        else:
            prepared.step(h, t)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        evs[k][0].record(stream)
        step()
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    launch_ms = [a.elapsed_time(b) for a, b in evs]
    mean_launch_ms = sum(launch_ms) / len(launch_ms)
    log(f"timed {args.steps} steps: {elapsed * 1e3 / args.steps:.3f} ms/step wall, "
        f"{mean_launch_ms:.3f} ms/launch (events), min {min(launch_ms):.3f}")

    algo_bytes = BYTES_PER_PARAM[mode] * n_params
    if args.param_dtype != "fp32":
        algo_bytes -= 6 * n_params      # 16-bit params (read + write) and grads: 2 bytes each instead of 4
    if mode == "blockwise8":
        algo_bytes += 16 * (n_params // 2048)     # absmax read and write, both moments
    achieved = algo_bytes / (mean_launch_ms / 1e3) / 1e9
    # The stored counters are those of the plain kernel (FP32 parameters, no count).
    traffic = None if (args.count_nonfinite or args.param_dtype != "fp32") else load_traffic(args.workload, mode)
    out = {
        "metric": METRIC,
        "value": round(n_params * args.steps / elapsed, 1),
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if args.param_dtype == "fp32" else f"f32 math, {args.param_dtype} params and grads",
        "data": "synthetic",
        "config": {"workload": args.workload, "params": n_params, "tensors": len(sizes),
                   "mode": {"e4": "packed-e4m11-e4m12", "fp16": "packed-fp16", "fp32": "fp32-adamw",
                            "blockwise8": "blockwise-8bit-2048"}[mode],
                   "state_bytes_per_param": pa.pa_state_bytes(mode, 1),
                   "param_dtype": args.param_dtype,
                   "count_nonfinite": bool(args.count_nonfinite),
                   "layout": ("state one HBM region (a third of device memory) below the parameters "
                              "in allocation order" if args.layout == "regions" else "back to back"),
                   "grads": "drawn once on the device, reused every step"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": ("blockwise_tables + blockwise_kernel (the events span both launches of the step)"
                                if mode == "blockwise8" else f"elementwise_list<{mode}>"),
                     "algorithmic_bytes_per_launch": algo_bytes,
                     "mean_launch_ms": round(mean_launch_ms, 4),
                     "median_launch_ms": round(sorted(launch_ms)[len(launch_ms) // 2], 4),
                     "kernel_sha": kernel_sha()},
    }
    if args.probe:
        del ps, gs, states
        prepared = None              # it holds the tensors too
        torch.cuda.empty_cache()
        out["probes"] = step_layout_ceilings(probe_lib(), 4 * n_params, args.layout)
        log(f"probes: {out['probes']}")
    if not args.no_cpu_baseline and not args.probe and args.param_dtype == "fp32":
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(cfg, mode, ps, gs, states, args.cpu_sample_params)
    # The ceilings are HBM figures: only the 7B list's 27 GB streams are far
    # past the 256 MB last-level cache (the smaller workloads stay partly or
    # wholly in it).
    if mode == "e4" and cfg == 4 and args.param_dtype == "fp32" and not args.probe and not args.no_ceiling:
        # What this HBM delivers for the step's own traffic and access forms,
        # measured after the step's buffers are freed (context for `frac`).
        del ps, gs, states
        prepared = None
        torch.cuda.empty_cache()
        try:
            import adamw_step_amd as _p  # noqa: F401
            ceil = step_layout_ceilings(probe_lib(), 4 * n_params, args.layout)
            ceil["frac_of_traffic_probe"] = round(achieved / ceil["mix_3r2w_gbps"], 4)
            ceil["frac_of_traffic_and_valu_probe"] = round(achieved / ceil["mix_3r2w_80valu_gbps"], 4)
            ceil["frac_of_read_then_write_bound"] = round(achieved / ceil["read_then_write_bound_gbps"], 4)
            out["roofline"]["measured_ceilings"] = ceil
            log(f"measured ceilings: {ceil}")
        except Exception as ex:      # a probe problem must not cost the result line
            out["roofline"]["measured_ceilings"] = None
            log(f"ceiling probes failed: {ex!r}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
