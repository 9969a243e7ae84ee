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
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
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
    lib.oracle_philox4x32.argtypes = [_u32p, _u32p, _u32p]
    lib.oracle_philox4x32.restype = None
    lib.oracle_turbo_state_bytes.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_size_t]
    lib.oracle_turbo_layout_ok.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    lib.oracle_turbo_layout_ok.restype = ctypes.c_int
    lib.oracle_turbo_state_bytes.restype = ctypes.c_size_t
    vp = ctypes.c_void_p
    lib.oracle_turbo_step.argtypes = [_f32p, _f32p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, vp, vp, _f32p, _f32p,
                                      _f32p, ctypes.c_double,
                                      ctypes.c_ulonglong, ctypes.c_longlong]
    lib.oracle_turbo_step.restype = ctypes.c_ulonglong
    lib.oracle_turbo_step_typed.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, ctypes.c_size_t, ctypes.c_uint32,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp,
                                            vp, vp, vp, vp, _f32p, _f32p, _f32p, ctypes.c_double, ctypes.c_ulonglong,
                                            ctypes.c_longlong]
    lib.oracle_turbo_step_typed.restype = ctypes.c_ulonglong
    lib.oracle_q1_levels.argtypes = [ctypes.c_uint16, ctypes.c_uint16, ctypes.c_int, _f32p]
    lib.oracle_q1_levels.restype = None
    lib.oracle_q1_levels_batch.argtypes = [_u32p, ctypes.c_size_t, ctypes.c_int, _f32p]
    lib.oracle_q1_levels_batch.restype = None
    lib.oracle_exp2_rn32_batch.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.c_size_t, _f32p]
    lib.oracle_exp2_rn32_batch.restype = None
    lib.oracle_q1_ends_batch.argtypes = [_f32p, _u32p, ctypes.c_size_t]
    lib.oracle_q1_ends_batch.restype = None
    lib.oracle_q1_block.argtypes = [_f32p, ctypes.c_size_t, ctypes.c_int, _f32p, _u8p, _u16p, _f32p]
    lib.oracle_q1_block.restype = None
    lib.oracle_ustate_group.argtypes = [_f32p, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_size_t, ctypes.c_float, _f32p,
                                        _u8p, _u16p,
                                        ctypes.POINTER(ctypes.c_double)]
    lib.oracle_ustate_group.restype = None
    lib.oracle_ustate_decode.argtypes = [_u8p, ctypes.c_size_t, ctypes.c_uint16, ctypes.c_float, _f32p]
    lib.oracle_ustate_decode.restype = None
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


def set_num_threads(k):
    """Threads the batch routines use from now on."""
    _load().oracle_set_num_threads(int(k))


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


def philox4x32(counter, key):
    """Philox4x32-10 of a 4-word counter and a 2-word key (four uint32 words)."""
    c = np.array(counter, np.uint32)
    k = np.array(key, np.uint32)
    out = np.zeros(4, np.uint32)
    _load().oracle_philox4x32(_ptr(c, _u32p), _ptr(k, _u32p), _ptr(out, _u32p))
    return out


def turbo_layout_ok(bits, block, group):
    """Whether the oracle takes this index width, 1Q block and UState group."""
    return bool(_load().oracle_turbo_layout_ok(int(bits), int(block), int(group)))


def turbo_state_bytes(compress_m, compress_v, bits, n, block=128, group=64):
    return int(_load().oracle_turbo_state_bytes(int(compress_m), int(compress_v), int(bits), int(block), int(group),
                                                int(n)))


class TurboState:
    """Host copy of one tensor's TurboAdam state, zero-filled (the empty state).
    block: the 1Q block (values per endpoint pair); group: the UState group
    (values per mean)."""

    def __init__(self, n, compress_m=True, compress_v=True, bits=4, block=128, group=64):
        assert turbo_layout_ok(bits, block, group), (bits, block, group)
        self.n, self.compress_m, self.compress_v, self.bits = n, bool(compress_m), bool(compress_v), bits
        self.block, self.group = block, group
        self.m_codes = np.zeros((n + 15) // 16, np.uint32) if compress_m else None
        self.m_means = np.zeros((n + group - 1) // group, np.uint16) if compress_m else None
        self.m_fp32 = None if compress_m else np.zeros(n, np.float32)
        self.v_index = np.zeros((n * bits + 31) // 32, np.uint32) if compress_v else None
        self.v_ends = np.zeros(2 * ((n + block - 1) // block), np.uint16) if compress_v else None
        self.v_fp32 = None if compress_v else np.zeros(n, np.float32)
        self.scal = np.zeros(3, np.float32)

    def arrays(self):
        return dict(m_codes=self.m_codes, m_means=self.m_means, m_fp32=self.m_fp32, v_index=self.v_index,
                    v_ends=self.v_ends, v_fp32=self.v_fp32, scal=self.scal)


def turbo_scalars(beta1, beta2, step):
    """[bc1, bc1 of the previous step, bc2 of the previous step], each formed in
    double and rounded once to binary32."""
    return np.array([1.0 - beta1 ** step, 1.0 - beta1 ** (step - 1), 1.0 - beta2 ** (step - 1)], np.float32)


def turbo_step(p, g, st, sc, ts, step, tensor_id=0, factor=1.1, seed=0x12345678):
    """One TurboAdam step of one tensor, in place on p and the TurboState st.
    Returns the non-finite count."""
    _need(p, np.float32, "p")
    _need(g, np.float32, "g")
    _need(sc, np.float32, "scalars")
    _need(ts, np.float32, "turbo scalars")
    assert p.size == g.size == st.n
    addr = lambda a: None if a is None else a.ctypes.data
    return int(_load().oracle_turbo_step(
        _ptr(p, _f32p), _ptr(g, _f32p), p.size, int(tensor_id), int(st.compress_m), int(st.compress_v), int(st.bits),
        int(st.block), int(st.group), addr(st.m_codes), addr(st.m_means), addr(st.m_fp32), addr(st.v_index), addr(st.v_ends), addr(st.v_fp32),
        _ptr(st.scal, _f32p), _ptr(sc, _f32p), _ptr(ts, _f32p), float(factor), int(seed), int(step)))


def turbo_step_typed(pdt, gdt, p, g, st, sc, ts, step, tensor_id=0, factor=1.1, seed=0x12345678):
    """turbo_step with typed parameters and gradients: float32 arrays (dtype 0)
    or uint16 bit patterns of bfloat16 (1) / binary16 (2), as for step_typed.
    In place on p and st; returns the non-finite count."""
    _need(p, _DT_NP[pdt], "p")
    _need(g, _DT_NP[gdt], "g")
    _need(sc, np.float32, "scalars")
    _need(ts, np.float32, "turbo scalars")
    assert p.size == g.size == st.n
    addr = lambda a: None if a is None else a.ctypes.data
    return int(_load().oracle_turbo_step_typed(
        int(pdt), int(gdt), p.ctypes.data, g.ctypes.data, p.size, int(tensor_id), int(st.compress_m),
        int(st.compress_v), int(st.bits), int(st.block), int(st.group), addr(st.m_codes), addr(st.m_means),
        addr(st.m_fp32), addr(st.v_index), addr(st.v_ends), addr(st.v_fp32), _ptr(st.scal, _f32p), _ptr(sc, _f32p),
        _ptr(ts, _f32p), float(factor), int(seed), int(step)))


def q1_levels(lo16, hi16, bits):
    """Decoded value of every 1Q index of a block with fp16 endpoints (bits)."""
    out = np.zeros(1 << bits, np.float32)
    _load().oracle_q1_levels(int(lo16), int(hi16), int(bits), _ptr(out, _f32p))
    return out


def exp2_rn32(x):
    """RN32 of the exact power 2^x for each double x: the rounding of the 1Q
    grid levels on its own."""
    a = np.ascontiguousarray(x, np.float64)
    out = np.zeros(a.size, np.float32)
    _load().oracle_exp2_rn32_batch(a.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), a.size, _ptr(out, _f32p))
    return out


def q1_levels_batch(ends, bits):
    """The levels of every block whose endpoint word (fp16 lower endpoint in
    the low half) is in ends: shape (len(ends), 2^bits)."""
    e = np.ascontiguousarray(ends, np.uint32)
    out = np.zeros((e.size, 1 << bits), np.float32)
    _load().oracle_q1_levels_batch(_ptr(e, _u32p), e.size, int(bits), _ptr(out, _f32p))
    return out


def q1_ends(v):
    """(RD16(log2 v), RU16(log2 v)) as binary16 bit patterns, for each
    positive finite float32 v: the endpoints of a one-value 1Q block."""
    v = np.ascontiguousarray(v, np.float32)
    out = np.empty(v.size, np.uint32)
    _load().oracle_q1_ends_batch(_ptr(v, _f32p), _ptr(out, _u32p), v.size)
    return (out & 0xFFFF).astype(np.uint16), (out >> 16).astype(np.uint16)


def q1_block(v, bits, u):
    """1Q encode of one block (<= 1024 values) with draws u: (indices, (lo, hi) fp16 bits, decoded)."""
    v = np.ascontiguousarray(v, np.float32)
    u = np.ascontiguousarray(u, np.float32)
    assert v.size == u.size <= 1024
    idx = np.zeros(v.size, np.uint8)
    ends = np.zeros(2, np.uint16)
    dec = np.zeros(v.size, np.float32)
    _load().oracle_q1_block(_ptr(v, _f32p), v.size, int(bits), _ptr(u, _f32p), _ptr(idx, _u8p), _ptr(ends, _u16p),
                            _ptr(dec, _f32p))
    return idx, ends, dec


def ustate_group(q, s_enc, u_pair, group=64, first=0):
    """UState encode of one group (<= group values, group a power of two up
    to 1024) whose first value has index `first` in its tensor: (codes, bf16
    mean bits, squared residuals)."""
    q = np.ascontiguousarray(q, np.float32)
    u_pair = np.ascontiguousarray(u_pair, np.float32)
    assert q.size <= group <= 1024 and group & (group - 1) == 0 and u_pair.size >= (q.size + 1) // 2
    codes = np.zeros(q.size, np.uint8)
    mean = np.zeros(1, np.uint16)
    r2 = np.zeros(q.size, np.float64)
    _load().oracle_ustate_group(_ptr(q, _f32p), q.size, int(group), int(first), float(np.float32(s_enc)),
                                _ptr(u_pair, _f32p),
                                _ptr(codes, _u8p), _ptr(mean, _u16p), r2.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return codes, int(mean[0]), r2


def ustate_decode(codes, mean16, s_dec):
    """UState decode of one group."""
    codes = np.ascontiguousarray(codes, np.uint8)
    out = np.zeros(codes.size, np.float32)
    _load().oracle_ustate_decode(_ptr(codes, _u8p), codes.size, int(mean16), float(np.float32(s_dec)), _ptr(out, _f32p))
    return out
