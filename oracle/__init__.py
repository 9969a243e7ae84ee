"""CPU oracle of the packed-AdamW step (ctypes wrapper around pa_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the benchmark's ``cpu_baseline`` leg may import this package.  The
product path (the ``adamw_step_amd`` package and its HIP library) never
imports, links or runs it, and it imports nothing from the product path.

Every function here is a thin marshalling layer; the arithmetic lives in
pa_oracle.c, whose header lists the passages each part follows and the
readings taken where the pages are silent.

Lanes (argument ``lane`` of encode/decode):
    0  E4M11 signed first moment (low half of the packed word)
    1  E4M12 unsigned uncorrected RMS (high half of the packed word)
    2  IEEE binary16 (both halves of the FP16-first/FP16-RMS word)
    3  bfloat16 (parameter output of the blockwise mode; 16-bit parameters)

Parity of the E4 exponent bias (15) is unpinned: the pages never print it.
"""
import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa_oracle.so")

LANE_M_E4, LANE_R_E4, LANE_F16, LANE_BF16 = 0, 1, 2, 3
PACKED_E4, PACKED_F16 = 1, 2
BLOCK = 2048

_lib = None


class SumsqAcc(ctypes.Structure):
    """Exact sum-of-squares accumulator (a 640-bit integer in units of 2^-298)."""
    _fields_ = [("limb", ctypes.c_uint64 * 10), ("nonfinite", ctypes.c_ulonglong),
                ("has_nan", ctypes.c_int), ("has_inf", ctypes.c_int)]


_f32p = ctypes.POINTER(ctypes.c_float)
_u32p = ctypes.POINTER(ctypes.c_uint32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u8p = ctypes.POINTER(ctypes.c_uint8)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.oracle_scalars.argtypes = [ctypes.c_double] * 5 + [ctypes.c_longlong, _f32p]
    lib.oracle_scalars.restype = None
    lib.oracle_encode_batch.argtypes = [ctypes.c_int, _f32p, _u16p, ctypes.c_size_t]
    lib.oracle_encode_batch.restype = None
    lib.oracle_decode_batch.argtypes = [ctypes.c_int, _u16p, _f32p, ctypes.c_size_t]
    lib.oracle_decode_batch.restype = None
    lib.oracle_step_fp32.argtypes = [_f32p, _f32p, _f32p, _f32p, ctypes.c_size_t, _f32p]
    lib.oracle_step_fp32.restype = ctypes.c_ulonglong
    lib.oracle_step_packed.argtypes = [ctypes.c_int, _f32p, _f32p, _u32p, ctypes.c_size_t, _f32p]
    lib.oracle_step_packed.restype = ctypes.c_ulonglong
    lib.oracle_step_blockwise.argtypes = [_f32p, _f32p, _u8p, _f32p, _u8p, _f32p, _f32p, _f32p,
                                          _u16p, ctypes.c_size_t, _f32p]
    lib.oracle_step_blockwise.restype = ctypes.c_ulonglong
    lib.oracle_step_typed.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, _f32p]
    lib.oracle_step_typed.restype = ctypes.c_ulonglong
    lib.oracle_search_codes.argtypes = [_f32p, _f32p, _u8p, ctypes.c_size_t]
    lib.oracle_search_codes.restype = None
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_block_len.restype = ctypes.c_int
    lib.oracle_e4_bias.restype = ctypes.c_int
    lib.oracle_sumsq_add.argtypes = [ctypes.POINTER(SumsqAcc), ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t]
    lib.oracle_sumsq_add.restype = None
    lib.oracle_sumsq_value.argtypes = [ctypes.POINTER(SumsqAcc)]
    lib.oracle_sumsq_value.restype = ctypes.c_double
    lib.oracle_clip_scale.argtypes = [ctypes.c_double, ctypes.c_double]
    lib.oracle_clip_scale.restype = ctypes.c_float
    lib.oracle_scale_grads.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_float, _f32p, ctypes.c_size_t]
    lib.oracle_scale_grads.restype = None
    _lib = lib
    return lib


def _ptr(a, typ):
    return a.ctypes.data_as(typ)


def _need(a, dtype, name):
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a C-contiguous numpy array of {np.dtype(dtype).name}")


def scalars(lr, beta1, beta2, eps, weight_decay, step):
    """The eight binary32 scalars of one call, formed in double and rounded once:
    [beta1, 1-beta1, beta2, 1-beta2, bc2, lr/bc1, 1-lr*wd, eps]."""
    out = np.zeros(8, np.float32)
    _load().oracle_scalars(float(lr), float(beta1), float(beta2), float(eps),
                           float(weight_decay), int(step), _ptr(out, _f32p))
    return out


def encode(lane, x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, np.uint16)
    _load().oracle_encode_batch(int(lane), _ptr(x, _f32p), _ptr(out, _u16p), x.size)
    return out


def decode(lane, codes):
    c = np.ascontiguousarray(codes, dtype=np.uint16)
    out = np.empty(c.shape, np.float32)
    _load().oracle_decode_batch(int(lane), _ptr(c, _u16p), _ptr(out, _f32p), c.size)
    return out


def step_fp32(p, g, m, v, sc):
    """In place on p, m, v.  Returns the non-finite element count."""
    for a, nm in ((p, "p"), (g, "g"), (m, "m"), (v, "v"), (sc, "scalars")):
        _need(a, np.float32, nm)
    n = p.size
    assert g.size == n and m.size == n and v.size == n and sc.size == 8
    return int(_load().oracle_step_fp32(_ptr(p, _f32p), _ptr(g, _f32p), _ptr(m, _f32p),
                                        _ptr(v, _f32p), n, _ptr(sc, _f32p)))


def step_packed(kind, p, g, w, sc):
    """kind PACKED_E4 or PACKED_F16; in place on p and w.  Returns the non-finite count."""
    _need(p, np.float32, "p")
    _need(g, np.float32, "g")
    _need(w, np.uint32, "w")
    _need(sc, np.float32, "scalars")
    n = p.size
    assert g.size == n and w.size == n and sc.size == 8
    if kind not in (PACKED_E4, PACKED_F16):
        raise ValueError("kind must be PACKED_E4 or PACKED_F16")
    return int(_load().oracle_step_packed(int(kind), _ptr(p, _f32p), _ptr(g, _f32p),
                                          _ptr(w, _u32p), n, _ptr(sc, _f32p)))


def step_blockwise(p, g, m_code, m_absmax, v_code, v_absmax, qmap_m, qmap_v, p_out, sc):
    """Codes, absmax arrays and p_out (uint16 holding bfloat16 bits) are written
    in place; p is read only.  Returns the non-finite count."""
    _need(p, np.float32, "p")
    _need(g, np.float32, "g")
    _need(m_code, np.uint8, "m_code")
    _need(v_code, np.uint8, "v_code")
    _need(m_absmax, np.float32, "m_absmax")
    _need(v_absmax, np.float32, "v_absmax")
    _need(qmap_m, np.float32, "qmap_m")
    _need(qmap_v, np.float32, "qmap_v")
    _need(p_out, np.uint16, "p_out")
    _need(sc, np.float32, "scalars")
    n = p.size
    if n % BLOCK:
        raise ValueError("blockwise length must be a multiple of 2048")
    nb = n // BLOCK
    assert g.size == n and m_code.size == n and v_code.size == n and p_out.size == n
    assert m_absmax.size == nb and v_absmax.size == nb
    assert qmap_m.size == 256 and qmap_v.size == 256
    r = _load().oracle_step_blockwise(
        _ptr(p, _f32p), _ptr(g, _f32p), _ptr(m_code, _u8p), _ptr(m_absmax, _f32p),
        _ptr(v_code, _u8p), _ptr(v_absmax, _f32p), _ptr(qmap_m, _f32p), _ptr(qmap_v, _f32p),
        _ptr(p_out, _u16p), n, _ptr(sc, _f32p))
    return int(r)


DT_F32, DT_BF16, DT_F16 = 0, 1, 2
_DT_NP = {DT_F32: np.float32, DT_BF16: np.uint16, DT_F16: np.uint16}


def step_typed(state_kind, pdt, gdt, p, g, state, sc):
    """Typed step: p, g are float32 arrays (dtype 0) or uint16 bit patterns of
    bfloat16 (1) / binary16 (2).  state_kind 0: state = (m, v) float32;
    1: packed E4 words (uint32); 2: packed binary16 words.  In place on p
    and the state.  Returns the non-finite count."""
    _need(p, _DT_NP[pdt], "p")
    _need(g, _DT_NP[gdt], "g")
    _need(sc, np.float32, "scalars")
    n = p.size
    assert g.size == n
    if state_kind == 0:
        m, v = state
        _need(m, np.float32, "m")
        _need(v, np.float32, "v")
        assert m.size == n and v.size == n
        s0, s1 = m.ctypes.data, v.ctypes.data
    else:
        _need(state, np.uint32, "words")
        assert state.size == n
        s0, s1 = state.ctypes.data, None
    return int(_load().oracle_step_typed(int(state_kind), int(pdt), int(gdt), p.ctypes.data, g.ctypes.data,
                                         s0, s1, n, _ptr(sc, _f32p)))


def search_codes(qmap, c):
    """Map entry chosen for each normalised value c (midpoint search alone)."""
    _need(qmap, np.float32, "qmap")
    c = np.ascontiguousarray(c, dtype=np.float32)
    out = np.empty(c.shape, np.uint8)
    _load().oracle_search_codes(_ptr(qmap, _f32p), _ptr(c, _f32p), _ptr(out, _u8p), c.size)
    return out


def num_threads():
    return int(_load().oracle_num_threads())


def e4_bias():
    return int(_load().oracle_e4_bias())


def sumsq_add(acc, gdt, g):
    """Add the squares of array g (element type gdt) to an exact SumsqAcc."""
    _need(g, _DT_NP[gdt], "g")
    _load().oracle_sumsq_add(ctypes.byref(acc), int(gdt), g.ctypes.data, g.size)


def sumsq_value(acc):
    """The accumulated sum of squares, rounded once to double."""
    return float(_load().oracle_sumsq_value(ctypes.byref(acc)))


def grad_stats(gdt, grads, max_norm=None):
    """Gradient pre-pass over a list of arrays of one element type gdt:
    (sum of squares, exact then rounded once to double; non-finite count;
    clip coefficient for max_norm, or None)."""
    acc = SumsqAcc()
    for g in grads:
        sumsq_add(acc, gdt, g)
    sumsq = sumsq_value(acc)
    clip = None if max_norm is None else float(clip_scale(sumsq, max_norm))
    return sumsq, int(acc.nonfinite), clip


def clip_scale(sumsq, max_norm):
    """min(1, max_norm / (sqrt(sumsq) + 1e-6)) in double, rounded to binary32."""
    return np.float32(_load().oracle_clip_scale(float(sumsq), float(max_norm)))


def scale_grads(gdt, g, scale):
    """float32 array widen(g) * scale, one binary32 multiplication per element."""
    _need(g, _DT_NP[gdt], "g")
    out = np.empty(g.size, np.float32)
    _load().oracle_scale_grads(int(gdt), g.ctypes.data, float(np.float32(scale)), _ptr(out, _f32p), g.size)
    return out
