"""Helpers shared by the GPU parity tests: device transfers, the parity bar,
and case banners printed (and flushed) before each GPU step."""
import sys

import numpy as np

import workloads

H = workloads.HYPER


def banner(msg):
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def dev():
    import torch
    return torch.device("cuda:0")


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    elif a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a.copy()).to(dev())


def to_host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def gather(t, idx):
    """t[idx] on the device, for a 1-D tensor t and an index tensor idx.
    Refuses tensors of 2^31 elements or more: torch's advanced-indexing
    kernel has faulted the GPU on such a gather, so large tensors are read
    through contiguous slices instead."""
    assert t.dim() == 1 and t.numel() < (1 << 31), (
        f"advanced indexing on a tensor of {t.numel()} elements (2^31 or more): use contiguous slices")
    return t[idx]


def hyper(step_unused=None, nonfinite=None, **kw):
    h = dict(H)
    h.update(kw)
    if nonfinite is not None:
        h["nonfinite"] = nonfinite
    return h


def scalars(step, **kw):
    import oracle
    h = dict(H)
    h.update(kw)
    return oracle.scalars(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"], step)


def ulp_diff(a, b):
    """Distance in units in the last place between float32 arrays (same sign
    ordering), NaN-aware: NaN vs NaN counts as 0."""
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    a = np.where(a < 0, -(a & 0x7FFFFFFF), a)
    b = np.where(b < 0, -(b & 0x7FFFFFFF), b)
    return np.abs(a - b)


def assert_params(got, want, what="params"):
    """The parity bar for parameters: within 2 FP32 ulp, or 1e-6 relative.
    Returns (bit-identical count, max ulp)."""
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    nan_g, nan_w = np.isnan(got), np.isnan(want)
    assert np.array_equal(nan_g, nan_w), f"{what}: NaN positions differ"
    ok = ~nan_w
    d = ulp_diff(got[ok], want[ok])
    rel = np.abs(got[ok].astype(np.float64) - want[ok]) / np.maximum(np.abs(want[ok].astype(np.float64)), 1e-300)
    bad = (d > 2) & (rel > 1e-6)
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond 2 ulp / 1e-6 rel (max ulp {d.max()})"
    same = int((got[ok].view(np.uint32) == want[ok].view(np.uint32)).sum()) + int(nan_w.sum())
    return same, int(d.max()) if d.size else 0


def assert_words(got, want, fp16=False, what="state words"):
    """State words: bit-exact; binary16 NaN lanes compare by class."""
    got = np.asarray(got).view(np.uint32)
    want = np.asarray(want).view(np.uint32)
    if not fp16:
        diff = np.nonzero(got != want)[0]
        assert diff.size == 0, (f"{what}: {diff.size} words differ, first at {diff[:5]}: "
                                f"{[hex(x) for x in got[diff[:5]]]} vs {[hex(x) for x in want[diff[:5]]]}")
        return
    for shift in (0, 16):
        g = (got >> shift) & 0xFFFF
        w = (want >> shift) & 0xFFFF
        gnan = ((g & 0x7C00) == 0x7C00) & ((g & 0x3FF) != 0)
        wnan = ((w & 0x7C00) == 0x7C00) & ((w & 0x3FF) != 0)
        assert np.array_equal(gnan, wnan), f"{what}: NaN lanes differ"
        assert np.array_equal(g[~wnan], w[~wnan]), f"{what}: {(g[~wnan] != w[~wnan]).sum()} lanes differ"
