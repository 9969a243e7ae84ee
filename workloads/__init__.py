"""Seeded synthetic inputs for the packed-AdamW step.

This module is the only thing the HIP path's tests and the oracle's tests
share: tensor-list shapes and seeded random inputs.  It holds none of the
method's arithmetic (no moments, no update, no codecs).

The five workloads stand in for the pages' trained-model gradients (the
reference GPT run on FineWeb, the TurboAdam GPT-2 runs) and for the KBench
blockwise task's absent inputs; none of those data exist here.

    1 "single-262k"      one tensor of 262,144 parameters, packed E4 mode
    2 "gpt-11m"          124-tensor GPT list, d=256, 10 blocks, vocab 12,096
    3 "gpt2-small-124m"  148-tensor GPT-2 small list (124,439,808 parameters)
    4 "llama-7b"         291-tensor Llama-7B list (6,738,415,616 parameters)
    5 "blockwise-268m"   one flat tensor of 2^28 parameters, blockwise 8-bit
    6 "gpt2-layer-7m"    the TurboAdam page's GPT-2-layer benchmark list as read
                         from its memory table: four 768x768 projections,
                         768x3072 and 3072x768 MLP matrices, three 768-value
                         vectors (7,080,192 parameters; the page prints no
                         shapes, these reproduce its four state-byte figures)

Seeds: parameters use 1000*c, gradients at step s use 1000*c + s, the
per-tensor gradient scales use 1000*c + 999, the blockwise code maps use 5500
(signed, first moment) and 5501 (unsigned, second moment).  Host draws are
NumPy PCG64 in float64 rounded once to float32; the 7B list and the 2^28
blockwise tensor are drawn on the device with a seeded torch generator.
"""
from __future__ import annotations

import numpy as np

NAMES = {1: "single-262k", 2: "gpt-11m", 3: "gpt2-small-124m", 4: "llama-7b",
         5: "blockwise-268m", 6: "gpt2-layer-7m"}
STEPS = {1: 10, 2: 100, 3: 50, 4: 20, 5: 20, 6: 100}
WARMUP = {4: 3}
HYPER = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def shapes(cfg: int):
    """[(name, shape), ...] of the tensor list of workload ``cfg``."""
    if cfg == 1:
        return [("w", (262144,))]
    if cfg == 2:
        d, v, ctx, blocks = 256, 12096, 1024, 10
        out = [("wte", (v, d)), ("wpe", (ctx, d))]
        for i in range(blocks):
            out += [(f"h{i}.qkv.w", (d, 3 * d)), (f"h{i}.qkv.b", (3 * d,)),
                    (f"h{i}.proj.w", (d, d)), (f"h{i}.proj.b", (d,)),
                    (f"h{i}.fc.w", (d, 4 * d)), (f"h{i}.fc.b", (4 * d,)),
                    (f"h{i}.fc2.w", (4 * d, d)), (f"h{i}.fc2.b", (d,)),
                    (f"h{i}.ln1.g", (d,)), (f"h{i}.ln1.b", (d,)),
                    (f"h{i}.ln2.g", (d,)), (f"h{i}.ln2.b", (d,))]
        out += [("lnf.g", (d,)), ("lnf.b", (d,))]
        return out
    if cfg == 3:
        d, v, ctx, blocks, ff = 768, 50257, 1024, 12, 3072
        out = [("wte", (v, d)), ("wpe", (ctx, d))]
        for i in range(blocks):
            out += [(f"h{i}.ln_1.g", (d,)), (f"h{i}.ln_1.b", (d,)),
                    (f"h{i}.attn.c_attn.w", (d, 3 * d)), (f"h{i}.attn.c_attn.b", (3 * d,)),
                    (f"h{i}.attn.c_proj.w", (d, d)), (f"h{i}.attn.c_proj.b", (d,)),
                    (f"h{i}.ln_2.g", (d,)), (f"h{i}.ln_2.b", (d,)),
                    (f"h{i}.mlp.c_fc.w", (d, ff)), (f"h{i}.mlp.c_fc.b", (ff,)),
                    (f"h{i}.mlp.c_proj.w", (ff, d)), (f"h{i}.mlp.c_proj.b", (d,))]
        out += [("ln_f.g", (d,)), ("ln_f.b", (d,))]
        return out
    if cfg == 4:
        d, v, layers, ff = 4096, 32000, 32, 11008
        out = [("embed_tokens", (v, d))]
        for i in range(layers):
            out += [(f"l{i}.q_proj", (d, d)), (f"l{i}.k_proj", (d, d)),
                    (f"l{i}.v_proj", (d, d)), (f"l{i}.o_proj", (d, d)),
                    (f"l{i}.gate_proj", (ff, d)), (f"l{i}.up_proj", (ff, d)),
                    (f"l{i}.down_proj", (d, ff)),
                    (f"l{i}.input_norm", (d,)), (f"l{i}.post_attn_norm", (d,))]
        out += [("norm", (d,)), ("lm_head", (v, d))]
        return out
    if cfg == 5:
        return [("flat", (1 << 28,))]
    if cfg == 6:
        d, ff = 768, 3072
        return [("q", (d, d)), ("k", (d, d)), ("v", (d, d)), ("o", (d, d)), ("fc", (d, ff)), ("proj", (ff, d)),
                ("vec0", (d,)), ("vec1", (d,)), ("vec2", (d,))]
    raise ValueError(f"unknown workload {cfg}")


def sizes(cfg: int):
    return [int(np.prod(s)) for _, s in shapes(cfg)]


def total(cfg: int) -> int:
    return sum(sizes(cfg))


def _kind(name: str) -> str:
    """'gain' for norm gains, 'bias' for biases, 'weight' otherwise."""
    if name.endswith(".g") or name.endswith("_norm") or name == "norm":
        return "gain"
    if name.endswith(".b"):
        return "bias"
    return "weight"


# ---------------------------------------------------------------- host draws

def _rng(seed: int):
    return np.random.Generator(np.random.PCG64(seed))


def grad_scales(cfg: int):
    """Fixed per-tensor gradient scale of workloads 2 and 4 (log-uniform)."""
    n = len(shapes(cfg))
    r = _rng(1000 * cfg + 999)
    if cfg == 2:
        return 10.0 ** r.uniform(-6.0, -1.0, n)
    if cfg == 4:
        return 1e-4 * 10.0 ** r.uniform(-1.0, 1.0, n)
    return np.ones(n)


def host_params(cfg: int, limit: int | None = None):
    """List of float32 parameter arrays (flat).  ``limit`` caps each tensor's
    length (for sampled runs of big workloads)."""
    r = _rng(1000 * cfg)
    out = []
    for name, shp in shapes(cfg):
        n = int(np.prod(shp)) if limit is None else min(int(np.prod(shp)), limit)
        if cfg in (3, 6):
            a = r.normal(0.0, 1e-3, n)
        elif cfg == 2 and _kind(name) == "gain":
            a = np.ones(n)
        elif cfg == 2 and _kind(name) == "bias":
            a = np.zeros(n)
        else:
            a = r.normal(0.0, 0.02, n)
        out.append(a.astype(np.float32))
    return out


def host_grads(cfg: int, step: int, limit: int | None = None):
    """List of float32 gradient arrays for step ``step`` (fresh per step)."""
    r = _rng(1000 * cfg + step)
    scales = grad_scales(cfg)
    out = []
    for k, (name, shp) in enumerate(shapes(cfg)):
        n = int(np.prod(shp)) if limit is None else min(int(np.prod(shp)), limit)
        if cfg == 1:
            u = r.uniform(0.0, 1.0, n)
            a = r.normal(0.0, 1e-3, n)
            sign = np.where(r.uniform(0.0, 1.0, n) < 0.5, -1.0, 1.0)
            a = np.where(u < 0.01, 0.0, np.where(u < 0.011, 0.1 * sign, a))
        elif cfg in (2, 4):
            a = scales[k] * r.normal(0.0, 1.0, n)
        else:
            a = r.normal(0.0, 1e-3, n)
        out.append(a.astype(np.float32))
    return out


def code_maps():
    """(qmap_m, qmap_v): ascending 256-entry float32 maps for the blockwise mode.

    A seeded stand-in for the KBench task's maps, which the pages do not
    print: the signed map holds 0, -1, +1, 126 further positive and 127
    further negative magnitudes 10^U(-7,0); the unsigned map holds 0, 1 and
    254 magnitudes 10^U(-14,0).  Duplicates (after rounding to float32) are
    redrawn so both maps are strictly ascending.
    """
    def draw(seed, npos, nneg, lo):
        r = _rng(seed)
        vals = {np.float32(0.0), np.float32(1.0)}
        if nneg:
            vals.add(np.float32(-1.0))
        pos, neg = set(), set()
        while len(pos) < npos:
            x = np.float32(10.0 ** r.uniform(lo, 0.0))
            if x not in vals and 0.0 < x < 1.0:
                pos.add(x)
        while len(neg) < nneg:
            x = np.float32(-(10.0 ** r.uniform(lo, 0.0)))
            if x not in vals and -1.0 < x < 0.0:
                neg.add(x)
        allv = sorted(vals | pos | neg)
        assert len(allv) == 256
        return np.array(allv, np.float32)

    return draw(5500, 126, 127, -7.0), draw(5501, 254, 0, -14.0)


# -------------------------------------------------------------- device draws

def device_fill_params(cfg: int, tensors, seed_offset: int = 0):
    """Fill a list of flat float32 CUDA tensors with workload ``cfg``'s
    parameters using a seeded device generator (used for workloads 4 and 5,
    too large to draw on the host)."""
    import torch

    gen = torch.Generator(device=tensors[0].device)
    gen.manual_seed(1000 * cfg + seed_offset)
    for (name, _), t in zip(shapes(cfg), tensors):
        if cfg == 2 and _kind(name) == "gain":
            t.fill_(1.0)
        elif cfg == 2 and _kind(name) == "bias":
            t.zero_()
        else:
            t.normal_(0.0, 1e-3 if cfg in (3, 6) else 0.02, generator=gen)


def device_fill_grads(cfg: int, step: int, tensors):
    """Fill flat float32 CUDA gradient tensors for step ``step`` on the device."""
    import torch

    gen = torch.Generator(device=tensors[0].device)
    gen.manual_seed(1000 * cfg + step)
    scales = grad_scales(cfg)
    for k, t in enumerate(tensors):
        if cfg in (2, 4):
            t.normal_(0.0, float(scales[k]), generator=gen)
        else:
            t.normal_(0.0, 1e-3, generator=gen)
