"""Python binding of libpa.so, the gfx950 packed-AdamW step library.

Argument marshalling only: every step of the update runs in the library's
HIP kernels.  PyTorch supplies device memory and the current stream.  If the
library is not built, importing works but every call raises; there is no
other path.

Functions keep the C names (see include/pa.h):

    pa_step(mode, params, grads, state, hyper, step, stream=None)
    pa_step_list(mode, params, grads, states, hyper, step, stream=None)
    pa_grad_stats_list(grads, sumsq, nonfinite=None, clip_scale=None, max_norm=0.0, stream=None)
    pa_state_bytes(mode, n), pa_format_info(mode), pa_status_string(rc)
    pa_debug_codec(lane, dir, inp, out, stream=None), pa_release_plans()

``state`` is, per mode: PA_PACKED_E4 / PA_PACKED_FP16 -> an int32 (or
uint32) tensor of words; PA_FP32 -> (m, v); PA_BLOCKWISE8 ->
(m_code, m_absmax, v_code, v_absmax, qmap_m, qmap_v, p_out_bf16).
``hyper`` is a mapping with lr, beta1, beta2, eps, weight_decay and the
optional device tensors ``nonfinite`` (int64, one element, incremented),
``grad_scale`` (float32, one element: every gradient is multiplied by it)
and ``skip_if_nonzero`` (int64, one element: a nonzero value skips the
update).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_FP32, PA_PACKED_E4, PA_PACKED_FP16, PA_BLOCKWISE8 = 0, 1, 2, 3
MODES = {"fp32": PA_FP32, "e4": PA_PACKED_E4, "fp16": PA_PACKED_FP16, "blockwise8": PA_BLOCKWISE8}
BLOCK = 2048

PA_OK, PA_ERR_ARG, PA_ERR_ALIGN, PA_ERR_SHAPE, PA_ERR_ALIAS, PA_ERR_DEVICE, PA_ERR_NOMEM = 0, -1, -2, -3, -4, -5, -6
PA_ERR_CAPACITY = -7
PA_NOALLOC_MAX_TENSORS = 4095   # include/pa.h


class PAError(RuntimeError):
    def __init__(self, rc, msg):
        super().__init__(f"{msg} (status {rc})")
        self.rc = rc


class Hyper(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double), ("beta2", ctypes.c_double),
                ("eps", ctypes.c_double), ("weight_decay", ctypes.c_double),
                ("nonfinite", ctypes.c_void_p), ("grad_scale", ctypes.c_void_p),
                ("skip_if_nonzero", ctypes.c_void_p)]


class Fp32State(ctypes.Structure):
    _fields_ = [("m", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class BlockwiseState(ctypes.Structure):
    _fields_ = [("m_code", ctypes.c_void_p), ("m_absmax", ctypes.c_void_p),
                ("v_code", ctypes.c_void_p), ("v_absmax", ctypes.c_void_p),
                ("qmap_m", ctypes.c_void_p), ("qmap_v", ctypes.c_void_p),
                ("p_out_bf16", ctypes.c_void_p)]


class TurboStateDesc(ctypes.Structure):
    _fields_ = [("compress_m", ctypes.c_int), ("compress_v", ctypes.c_int), ("tensor_id", ctypes.c_uint32),
                ("m_codes", ctypes.c_void_p), ("m_means", ctypes.c_void_p), ("m_fp32", ctypes.c_void_p),
                ("v_index", ctypes.c_void_p), ("v_ends", ctypes.c_void_p), ("v_fp32", ctypes.c_void_p),
                ("scalars", ctypes.c_void_p)]


class TurboConfig(ctypes.Structure):
    _fields_ = [("v_bits", ctypes.c_int), ("m_step_factor", ctypes.c_double), ("seed", ctypes.c_ulonglong),
                ("block_size", ctypes.c_int), ("m_block_size", ctypes.c_int), ("path", ctypes.c_int)]


class Format(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int), ("lanes", ctypes.c_int),
                ("m_sign_bits", ctypes.c_int), ("m_exp_bits", ctypes.c_int),
                ("m_mant_bits", ctypes.c_int), ("m_exp_bias", ctypes.c_int),
                ("r_sign_bits", ctypes.c_int), ("r_exp_bits", ctypes.c_int),
                ("r_mant_bits", ctypes.c_int), ("r_exp_bias", ctypes.c_int),
                ("m_max", ctypes.c_double), ("m_min_normal", ctypes.c_double),
                ("m_min_subnormal", ctypes.c_double), ("r_max", ctypes.c_double),
                ("r_min_normal", ctypes.c_double), ("r_min_subnormal", ctypes.c_double),
                ("block", ctypes.c_int)]


EXPORTS = ("pa_step", "pa_step_list", "pa_step_typed", "pa_step_list_typed", "pa_state_bytes",
           "pa_format_info", "pa_status_string", "pa_last_hip_error", "pa_release_plans", "pa_debug_codec",
           "pa_debug_sqrt", "pa_debug_scalars", "pa_debug_q1_ends", "pa_debug_q1_levels", "pa_debug_pow2_rn32", "pa_grad_stats_list", "pa_turbo_state_bytes", "pa_turbo_layout_bytes", "pa_turbo_workspace_bytes",
           "pa_turbo_step_list", "pa_turbo_step_list_typed", "pa_step_list_noalloc", "pa_debug_plan_count",
           "pa_debug_blockwise_path")

PA_DT_F32, PA_DT_BF16, PA_DT_F16 = 0, 1, 2

_lib = None


def lib():
    """Load libpa.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m adamw_step_amd.build` "
                           "(there is no fallback path)")
    import torch  # noqa: F401  -- loads the HIP runtime that the library binds to
    L = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.pa_step.argtypes = [ctypes.c_int, vp, vp, vp, sz, ctypes.POINTER(Hyper), ctypes.c_longlong, vp]
    L.pa_step.restype = ctypes.c_int
    L.pa_step_list.argtypes = [ctypes.c_int, sz, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                               ctypes.POINTER(sz), ctypes.POINTER(Hyper), ctypes.c_longlong, vp]
    L.pa_step_list.restype = ctypes.c_int
    L.pa_step_typed.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, sz, ctypes.POINTER(Hyper),
                                ctypes.c_longlong, vp]
    L.pa_step_typed.restype = ctypes.c_int
    L.pa_step_list_typed.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, sz, ctypes.POINTER(vp),
                                     ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(sz),
                                     ctypes.POINTER(Hyper), ctypes.c_longlong, vp]
    L.pa_step_list_typed.restype = ctypes.c_int
    L.pa_step_list_noalloc.argtypes = L.pa_step_list_typed.argtypes
    L.pa_step_list_noalloc.restype = ctypes.c_int
    L.pa_state_bytes.argtypes = [ctypes.c_int, sz]
    L.pa_state_bytes.restype = sz
    L.pa_format_info.argtypes = [ctypes.c_int, ctypes.POINTER(Format)]
    L.pa_format_info.restype = ctypes.c_int
    L.pa_status_string.argtypes = [ctypes.c_int]
    L.pa_status_string.restype = ctypes.c_char_p
    L.pa_last_hip_error.restype = ctypes.c_int
    L.pa_release_plans.restype = None
    L.pa_debug_codec.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, sz, vp]
    L.pa_debug_codec.restype = ctypes.c_int
    L.pa_debug_scalars.argtypes = [ctypes.POINTER(Hyper), ctypes.c_longlong, vp, vp]
    L.pa_debug_scalars.restype = ctypes.c_int
    L.pa_debug_sqrt.argtypes = [vp, vp, sz, vp]
    L.pa_debug_sqrt.restype = ctypes.c_int
    L.pa_debug_q1_ends.argtypes = [vp, vp, sz, vp]
    L.pa_debug_q1_ends.restype = ctypes.c_int
    L.pa_debug_q1_levels.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, sz, vp]
    L.pa_debug_q1_levels.restype = ctypes.c_int
    L.pa_debug_pow2_rn32.argtypes = [vp, ctypes.c_int, vp, sz, vp]
    L.pa_debug_pow2_rn32.restype = ctypes.c_int
    L.pa_grad_stats_list.argtypes = [ctypes.c_int, sz, ctypes.POINTER(vp), ctypes.POINTER(sz), ctypes.c_double,
                                     vp, vp, vp, vp]
    L.pa_grad_stats_list.restype = ctypes.c_int
    L.pa_turbo_state_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, sz]
    L.pa_turbo_state_bytes.restype = sz
    L.pa_turbo_layout_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, sz]
    L.pa_turbo_layout_bytes.restype = sz
    L.pa_turbo_workspace_bytes.argtypes = [sz, ctypes.POINTER(TurboStateDesc), ctypes.POINTER(sz)]
    L.pa_turbo_workspace_bytes.restype = sz
    L.pa_turbo_step_list.argtypes = [sz, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(TurboStateDesc),
                                     ctypes.POINTER(sz), ctypes.POINTER(Hyper), ctypes.POINTER(TurboConfig),
                                     ctypes.c_longlong, vp, sz, vp]
    L.pa_turbo_step_list.restype = ctypes.c_int
    L.pa_turbo_step_list_typed.argtypes = [ctypes.c_int, ctypes.c_int] + L.pa_turbo_step_list.argtypes
    L.pa_turbo_step_list_typed.restype = ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int)
    L.pa_debug_plan_count.argtypes = [ip, ip, ip]
    L.pa_debug_plan_count.restype = ctypes.c_int
    L.pa_debug_blockwise_path.argtypes = [ctypes.c_longlong]
    L.pa_debug_blockwise_path.restype = ctypes.c_int
    _lib = L
    return L


def _check(rc):
    if rc != PA_OK:
        L = lib()
        msg = L.pa_status_string(rc).decode()
        if rc == PA_ERR_DEVICE:
            msg += f"; hipError {L.pa_last_hip_error()}"
        raise PAError(rc, msg)


def _mode(mode):
    return MODES[mode] if isinstance(mode, str) else int(mode)


def _ptr(t):
    return None if t is None else int(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


def _device_word(t, dtype, what):
    import torch
    if t is None:
        return None
    _tensor_ok(t, what)
    if t.dtype != dtype or t.numel() != 1:
        raise TypeError(f"{what} must be a one-element {dtype} device tensor")
    return _ptr(t)


def _hyper(h):
    import torch
    return Hyper(float(h["lr"]), float(h["beta1"]), float(h["beta2"]), float(h["eps"]),
                 float(h["weight_decay"]), _device_word(h.get("nonfinite"), torch.int64, "nonfinite"),
                 _device_word(h.get("grad_scale"), torch.float32, "grad_scale"),
                 _device_word(h.get("skip_if_nonzero"), torch.int64, "skip_if_nonzero"))


def _tensor_ok(t, what):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{what} must be a contiguous device tensor")
    if t.is_sparse:
        raise TypeError(f"{what} must be dense")


def _dtype_code(t):
    import torch
    code = {torch.float32: PA_DT_F32, torch.bfloat16: PA_DT_BF16, torch.float16: PA_DT_F16}.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported tensor dtype {t.dtype} (float32, bfloat16, float16)")
    return code


def _check_pg(p, g):
    """Validate one parameter/gradient pair; returns their dtype codes."""
    _tensor_ok(p, "params")
    _tensor_ok(g, "grads")
    pdt, gdt = _dtype_code(p), _dtype_code(g)
    if not (pdt == gdt or gdt == PA_DT_F32):
        raise TypeError("grads must have the params' dtype, or be float32")
    if g.numel() != p.numel() or g.device != p.device:
        raise ValueError("grads must match params in size and device")
    return pdt, gdt


def _state_arg(mode, p, state, keep):
    """Host-side argument for one tensor's state; `keep` holds ctypes objects alive."""
    import torch
    n = p.numel()
    if mode in (PA_PACKED_E4, PA_PACKED_FP16):
        _tensor_ok(state, "state")
        if state.dtype not in (torch.int32, torch.uint32) or state.numel() != n or state.device != p.device:
            raise TypeError("packed state must be a 32-bit tensor with one word per parameter")
        return _ptr(state)
    if mode == PA_FP32:
        m, v = state
        for t, nm in ((m, "m"), (v, "v")):
            _tensor_ok(t, nm)
            if t.dtype != torch.float32 or t.numel() != n or t.device != p.device:
                raise TypeError(f"FP32 state {nm} must be float32 with one value per parameter")
        st = Fp32State(_ptr(m), _ptr(v))
        keep.append(st)
        return ctypes.addressof(st)
    if mode == PA_BLOCKWISE8:
        mc, ma, vc, va, qm, qv, pout = state
        for t, nm in ((mc, "m_code"), (ma, "m_absmax"), (vc, "v_code"), (va, "v_absmax"),
                      (qm, "qmap_m"), (qv, "qmap_v"), (pout, "p_out")):
            _tensor_ok(t, nm)
            if t.device != p.device:
                raise ValueError(f"{nm} is on another device")
        st = BlockwiseState(_ptr(mc), _ptr(ma), _ptr(vc), _ptr(va), _ptr(qm), _ptr(qv), _ptr(pout))
        keep.append(st)
        return ctypes.addressof(st)
    raise ValueError(f"unknown mode {mode}")


def pa_step(mode, params, grads, state, hyper, step, stream=None):
    """One tensor, updated in place (see include/pa.h).  float32, bfloat16
    or float16 params; grads of the same dtype or float32."""
    mode = _mode(mode)
    pdt, gdt = _check_pg(params, grads)
    keep = []
    st = _state_arg(mode, params, state, keep)
    h = _hyper(hyper)
    _check(lib().pa_step_typed(mode, pdt, gdt, _ptr(params), _ptr(grads), st, params.numel(), ctypes.byref(h),
                               int(step), _stream(stream)))


def pa_step_list(mode, params, grads, states, hyper, step, stream=None, noalloc=False):
    """A list of tensors sharing one hyperparameter set and step, one launch.
    noalloc=True calls pa_step_list_noalloc (no device allocation; the table
    in the library's static device array, see include/pa.h)."""
    mode = _mode(mode)
    k = len(params)
    if len(grads) != k or len(states) != k:
        raise ValueError("params, grads and states must have the same length")
    keep = []
    P = (ctypes.c_void_p * k)()
    G = (ctypes.c_void_p * k)()
    S = (ctypes.c_void_p * k)()
    N = (ctypes.c_size_t * k)()
    types = set()
    for i in range(k):
        types.add(_check_pg(params[i], grads[i]))
        if params[i].device != params[0].device:
            raise ValueError("all tensors of one call must be on one device")
        P[i], G[i] = _ptr(params[i]), _ptr(grads[i])
        S[i] = _state_arg(mode, params[i], states[i], keep)
        N[i] = params[i].numel()
    if len(types) > 1:
        raise TypeError("all tensors of one call must share the params' and the grads' dtypes")
    pdt, gdt = types.pop() if types else (PA_DT_F32, PA_DT_F32)
    h = _hyper(hyper)
    fn = lib().pa_step_list_noalloc if noalloc else lib().pa_step_list_typed
    _check(fn(mode, pdt, gdt, k, P, G, S, N, ctypes.byref(h), int(step), _stream(stream)))


class StepList:
    """A fixed tensor list, validated and marshalled once.

    ``step(hyper, t)`` is then a single call of pa_step_list with the cached
    pointer arrays.  The tensors must stay alive and in place (same storage)
    for as long as the object is used; build a new StepList if any of them
    is reallocated.
    """

    def __init__(self, mode, params, grads, states):
        self.mode = _mode(mode)
        k = len(params)
        if len(grads) != k or len(states) != k:
            raise ValueError("params, grads and states must have the same length")
        self._keep = [list(params), list(grads), list(states)]
        self._structs = []
        self._P = (ctypes.c_void_p * k)()
        self._G = (ctypes.c_void_p * k)()
        self._S = (ctypes.c_void_p * k)()
        self._N = (ctypes.c_size_t * k)()
        types = set()
        for i in range(k):
            types.add(_check_pg(params[i], grads[i]))
            if params[i].device != params[0].device:
                raise ValueError("all tensors of one call must be on one device")
            self._P[i], self._G[i] = _ptr(params[i]), _ptr(grads[i])
            self._S[i] = _state_arg(self.mode, params[i], states[i], self._structs)
            self._N[i] = params[i].numel()
        if len(types) > 1:
            raise TypeError("all tensors of one call must share the params' and the grads' dtypes")
        self.pdt, self.gdt = types.pop() if types else (PA_DT_F32, PA_DT_F32)
        self.count = k
        self._fn = lib().pa_step_list_typed

    def set_grads(self, grads):
        """Point the list at other gradient tensors of the same dtypes and
        sizes (torch allocates new ones after zero_grad(set_to_none=True));
        the library writes the new pointers into its cached table."""
        params = self._keep[0]
        if len(grads) != len(params):
            raise ValueError("one gradient per parameter")
        for i, (p, g) in enumerate(zip(params, grads)):
            if _check_pg(p, g) != (self.pdt, self.gdt):
                raise TypeError("the gradients must keep the list's dtype")
            self._G[i] = _ptr(g)
        self._keep[1] = list(grads)

    def step(self, hyper, step, stream=None):
        h = _hyper(hyper)
        _check(self._fn(self.mode, self.pdt, self.gdt, self.count, self._P, self._G, self._S, self._N,
                        ctypes.byref(h), int(step), _stream(stream)))


def _stats_outputs(sumsq, nonfinite, clip_scale):
    import torch
    return (_device_word(sumsq, torch.float64, "sumsq"), _device_word(nonfinite, torch.int64, "nonfinite"),
            _device_word(clip_scale, torch.float32, "clip_scale"))


class GradStats:
    """Gradient pre-pass over a fixed gradient list (validated and
    marshalled once): ``run(sumsq, nonfinite=None, clip_scale=None,
    max_norm=0.0)`` writes the sum of squares (float64), the non-finite count
    (int64) and the clip coefficient (float32) into one-element device
    tensors.  Feed ``clip_scale`` and ``nonfinite`` to the step as
    ``grad_scale`` and ``skip_if_nonzero``."""

    def __init__(self, grads):
        import torch
        k = len(grads)
        self._keep = list(grads)
        self._G = (ctypes.c_void_p * k)()
        self._N = (ctypes.c_size_t * k)()
        dts = set()
        for i, g in enumerate(grads):
            _tensor_ok(g, "grads")
            dts.add(_dtype_code(g))
            if g.device != grads[0].device:
                raise ValueError("all gradients of one call must be on one device")
            self._G[i] = _ptr(g)
            self._N[i] = g.numel()
        if len(dts) > 1:
            raise TypeError("all gradients of one call must share one dtype")
        self.gdt = dts.pop() if dts else PA_DT_F32
        self.count = k
        self._fn = lib().pa_grad_stats_list

    def set_grads(self, grads):
        """Other gradient tensors of the same dtype and sizes (see
        StepList.set_grads)."""
        if len(grads) != self.count:
            raise ValueError("as many gradients as before")
        for i, g in enumerate(grads):
            _tensor_ok(g, "grads")
            if _dtype_code(g) != self.gdt or g.numel() != self._N[i] or g.device != self._keep[0].device:
                raise TypeError("the gradients must keep the list's dtype, sizes and device")
            self._G[i] = _ptr(g)
        self._keep = list(grads)

    def run(self, sumsq, nonfinite=None, clip_scale=None, max_norm=0.0, stream=None):
        s, nf, cl = _stats_outputs(sumsq, nonfinite, clip_scale)
        _check(self._fn(self.gdt, self.count, self._G, self._N, float(max_norm), s, nf, cl, _stream(stream)))


def pa_grad_stats_list(grads, sumsq, nonfinite=None, clip_scale=None, max_norm=0.0, stream=None):
    """One-shot gradient pre-pass (see GradStats and include/pa.h)."""
    GradStats(grads).run(sumsq, nonfinite, clip_scale, max_norm, stream)


def plan_counts():
    """(list-step plans, gradient pre-pass plans, TurboAdam plans) cached in
    the library (pa_debug_plan_count)."""
    a, b, c = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    _check(lib().pa_debug_plan_count(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def blockwise_path(blocks_per_workgroup):
    """Which launch the blockwise step takes from now on, for tests of both
    (pa_debug_blockwise_path): 0 by size (the default), -1 the persistent
    launch, k >= 1 the ordered launch with k blocks per workgroup."""
    _check(lib().pa_debug_blockwise_path(int(blocks_per_workgroup)))


def pa_state_bytes(mode, n):
    return int(lib().pa_state_bytes(_mode(mode), int(n)))


def pa_format_info(mode):
    f = Format()
    _check(lib().pa_format_info(_mode(mode), ctypes.byref(f)))
    return {name: getattr(f, name) for name, _ in Format._fields_}


def pa_status_string(rc):
    return lib().pa_status_string(int(rc)).decode()


def pa_last_hip_error():
    return int(lib().pa_last_hip_error())


def pa_release_plans():
    lib().pa_release_plans()


def pa_debug_codec(lane, direction, inp, out, stream=None):
    """lane 0 E4M11, 1 E4M12, 2 binary16; direction 0 encode (float32 -> uint16
    held in an int16 tensor), 1 decode."""
    _tensor_ok(inp, "input")
    _tensor_ok(out, "output")
    if inp.numel() != out.numel():
        raise ValueError("input and output sizes differ")
    _check(lib().pa_debug_codec(int(lane), int(direction), _ptr(inp), _ptr(out), inp.numel(),
                                _stream(stream)))


def pa_debug_scalars(hyper, step):
    """The per-call binary32 scalars the kernels receive (host only): a
    float32 array [beta1, 1-beta1, beta2, 1-beta2, bc2, lr/bc1, 1-lr*wd, eps,
    beta1*2^112] and the double 1/bc2 (see include/pa.h)."""
    import numpy as np
    out = np.zeros(9, np.float32)
    inv = ctypes.c_double(0.0)
    h = Hyper(float(hyper["lr"]), float(hyper["beta1"]), float(hyper["beta2"]), float(hyper["eps"]),
              float(hyper["weight_decay"]), None, None, None)
    _check(lib().pa_debug_scalars(ctypes.byref(h), int(step), out.ctypes.data, ctypes.byref(inv)))
    return out, inv.value


def pa_debug_sqrt(inp, out, stream=None):
    """out = the GPU path's correctly rounded square root of inp (float32)."""
    _tensor_ok(inp, "input")
    _tensor_ok(out, "output")
    if inp.numel() != out.numel():
        raise ValueError("input and output sizes differ")
    _check(lib().pa_debug_sqrt(_ptr(inp), _ptr(out), inp.numel(), _stream(stream)))


def pa_debug_q1_ends(inp, out, stream=None):
    """out (int32, bit pattern) = the two 1Q endpoints of each positive float32
    in inp: binary16 of log2 rounded down (low half) and up (high half)."""
    _tensor_ok(inp, "input")
    _tensor_ok(out, "output")
    if inp.numel() != out.numel() or out.element_size() != 4:
        raise ValueError("output must hold one 32-bit word per input")
    _check(lib().pa_debug_q1_ends(_ptr(inp), _ptr(out), inp.numel(), _stream(stream)))



def pa_debug_q1_levels(ends, bits, exact, out, stream=None):
    """out (float32, len(ends) * 2^bits) = the 1Q levels of each endpoint word
    in ends (int32 bit patterns: fp16 lower endpoint low, upper high);
    exact=True takes every level through the double-double evaluation."""
    import torch

    _tensor_ok(ends, "endpoints")
    _tensor_ok(out, "output")
    if ends.element_size() != 4 or out.dtype != torch.float32:
        raise ValueError("endpoints must be 32-bit words and the output float32")
    if out.numel() != ends.numel() << int(bits):
        raise ValueError("output must hold 2^bits levels per endpoint word")
    _check(lib().pa_debug_q1_levels(_ptr(ends), int(bits), 1 if exact else 0, _ptr(out), ends.numel(),
                                    _stream(stream)))



def pa_debug_pow2_rn32(x, exact, out, stream=None):
    """out (float32) = RN32(2^x) for each float64 x, through the 4-bit tables'
    route or (exact=True) the double-double evaluation alone."""
    import torch

    _tensor_ok(x, "input")
    _tensor_ok(out, "output")
    if x.dtype != torch.float64 or out.dtype != torch.float32 or x.numel() != out.numel():
        raise ValueError("input must be float64 and output float32, of one size")
    _check(lib().pa_debug_pow2_rn32(_ptr(x), 1 if exact else 0, _ptr(out), x.numel(), _stream(stream)))


# ---------------------------------------------------------------- TurboAdam

class TurboState:
    """Device buffers of one tensor's TurboAdam state, zero-filled (the empty
    state): UState (compress_m) or an FP32 first moment, 1Q (compress_v) or
    an FP32 second moment (sizes as in include/pa.h).  block_size: values
    per 1Q endpoint pair; m_block_size: values per UState mean."""

    def __init__(self, n, device, compress_m=True, compress_v=True, v_bits=4, tensor_id=0, block_size=128,
                 m_block_size=64):
        import torch
        if not turbo_layout_ok(v_bits, block_size, m_block_size):
            raise ValueError(f"TurboAdam layout not taken: v_bits={v_bits}, block_size={block_size}, "
                             f"m_block_size={m_block_size}")
        z = lambda k, dt: torch.zeros(k, dtype=dt, device=device)
        self.n, self.compress_m, self.compress_v, self.v_bits = int(n), bool(compress_m), bool(compress_v), v_bits
        self.block_size, self.m_block_size = int(block_size), int(m_block_size)
        self.tensor_id = int(tensor_id)
        B, G = self.block_size, self.m_block_size
        self.m_codes = z(4 * ((n + 15) // 16), torch.uint8) if compress_m else None
        self.m_means = z((n + G - 1) // G, torch.int16) if compress_m else None
        self.scalars = z(3, torch.float32) if compress_m else None
        self.m_fp32 = None if compress_m else z(n, torch.float32)
        self.v_index = z(4 * ((n * v_bits + 31) // 32), torch.uint8) if compress_v else None
        self.v_ends = z(2 * ((n + B - 1) // B), torch.int16) if compress_v else None
        self.v_fp32 = None if compress_v else z(n, torch.float32)

    def desc(self):
        return TurboStateDesc(int(self.compress_m), int(self.compress_v), self.tensor_id, _ptr(self.m_codes),
                              _ptr(self.m_means), _ptr(self.m_fp32), _ptr(self.v_index), _ptr(self.v_ends),
                              _ptr(self.v_fp32), _ptr(self.scalars))

    def tensors(self):
        return [t for t in (self.m_codes, self.m_means, self.scalars, self.m_fp32, self.v_index, self.v_ends,
                            self.v_fp32) if t is not None]

    def nbytes(self):
        return sum(t.numel() * t.element_size() for t in self.tensors())


def pa_turbo_state_bytes(compress_m, compress_v, v_bits, n):
    return int(lib().pa_turbo_state_bytes(int(compress_m), int(compress_v), int(v_bits), int(n)))


def pa_turbo_layout_bytes(compress_m, compress_v, v_bits, block_size, m_block_size, n):
    return int(lib().pa_turbo_layout_bytes(int(compress_m), int(compress_v), int(v_bits), int(block_size),
                                           int(m_block_size), int(n)))


def turbo_layout_ok(v_bits, block_size, m_block_size):
    """The layouts of the TurboAdam fused path: 2, 3, 4, 6 or 8 index bits, a
    power-of-two block from 32 to 1024 values, a power-of-two mean group
    dividing it (the library refuses any other with PA_ERR_ARG)."""
    b, B, G = int(v_bits), int(block_size), int(m_block_size)
    return (b in (2, 3, 4, 6, 8) and 32 <= B <= 1024 and B & (B - 1) == 0 and 1 <= G <= B and G & (G - 1) == 0)


class TurboList:
    """A fixed list of parameters, gradients and TurboState objects,
    validated and marshalled once; ``step(hyper, t)`` is one
    pa_turbo_step_list_typed call.  Parameters are float32, bfloat16 or
    float16, all of one type; gradients are of the parameters' type or
    float32 (the pairs of pa_step_typed).  Owns its device workspace."""

    def __init__(self, params, grads, states, v_bits=4, m_step_factor=1.1, seed=0x12345678, block_size=128,
                 m_block_size=64, general=False):
        import torch
        k = len(params)
        if len(grads) != k or len(states) != k:
            raise ValueError("params, grads and states must have the same length")
        self._keep = [list(params), list(grads), list(states)]
        self._P = (ctypes.c_void_p * k)()
        self._G = (ctypes.c_void_p * k)()
        self._S = (TurboStateDesc * k)()
        self._N = (ctypes.c_size_t * k)()
        self.pdt = _dtype_code(params[0]) if k else PA_DT_F32
        self.gdt = _dtype_code(grads[0]) if k else PA_DT_F32
        for i in range(k):
            p, g, st = params[i], grads[i], states[i]
            _tensor_ok(p, "params")
            _tensor_ok(g, "grads")
            if _dtype_code(p) != self.pdt or _dtype_code(g) != self.gdt:
                raise TypeError("every parameter must share one dtype, and every gradient one dtype")
            if g.numel() != p.numel() or st.n != p.numel() or st.v_bits != v_bits:
                raise ValueError("params, grads and states disagree in size or v_bits")
            if (st.block_size, st.m_block_size) != (block_size, m_block_size):
                raise ValueError("states disagree with the list's block_size or m_block_size")
            self._P[i], self._G[i] = _ptr(p), _ptr(g)
            self._S[i] = st.desc()
            self._N[i] = p.numel()
        self.count = k
        self.config = TurboConfig(int(v_bits), float(m_step_factor), int(seed), int(block_size), int(m_block_size),
                                  1 if general else 0)
        L = lib()
        wsb = int(L.pa_turbo_workspace_bytes(k, self._S, self._N)) if k else 0
        dev = params[0].device if k else "cuda:0"
        self.workspace = torch.empty(max(wsb // 8, 1), dtype=torch.float64, device=dev)
        self._wsb = wsb
        self._fn = L.pa_turbo_step_list_typed

    def set_grads(self, grads):
        """Other gradient tensors of the same dtype and sizes (see
        StepList.set_grads)."""
        params = self._keep[0]
        if len(grads) != len(params):
            raise ValueError("one gradient per parameter")
        for i, (p, g) in enumerate(zip(params, grads)):
            _tensor_ok(g, "grads")
            if _dtype_code(g) != self.gdt or g.numel() != p.numel() or g.device != p.device:
                raise TypeError("the gradients must keep the list's dtype, sizes and device")
            self._G[i] = _ptr(g)
        self._keep[1] = list(grads)

    def step(self, hyper, step, stream=None):
        h = _hyper(hyper)
        _check(self._fn(self.pdt, self.gdt, self.count, self._P, self._G, self._S, self._N, ctypes.byref(h),
                        ctypes.byref(self.config), int(step), _ptr(self.workspace), self._wsb, _stream(stream)))
