/*
 * pa_oracle.c -- plain, slow, CPU oracle for the packed-AdamW step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file; only the test suite, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no code, header, table or constant
 * generator with the HIP kernels.
 *
 * What it computes, and where each piece comes from:
 *
 *  - The state word (one uint32 per FP32 parameter; low half a signed finite
 *    E4M11 first moment, high half an unsigned finite E4M12 uncorrected RMS;
 *    no shadow moments, block scales or stochastic rounding):
 *    "Packed AdamW Reference" README, introduction (canonical format);
 *    "Packed AdamW / Reference / v1.0.0" project page, Release scope.
 *  - The update order (decode, square the RMS, new moments, FP32 AdamW step
 *    with the new unquantised moments, pack afterwards): same two passages.
 *  - The AdamW recurrence and the decoupled-decay update: TurboAdam package
 *    page, "The AdamW update remains AdamW" equation block.
 *  - The left-to-right FP32 operation sequence, the host-side scalars held
 *    in double precision, and the whole blockwise 8-bit mode (2048-element
 *    blocks, absmax per block, nearest entry of an ascending 256-point map
 *    through midpoints, BF16 parameter output): KBench task
 *    "quantized-optimizer-state", environment reference, routines
 *    `quantized_adamw_step` and `_requantise`.
 *
 *  - The gradient pre-pass (exact sum of squares, non-finite count, clip
 *    coefficient) and the TurboAdam compressed state (UState first moment,
 *    1Q second moment, Philox4x32-10 draws): see their sections below,
 *    each with its own readings.
 *
 * Readings where the pages are silent (kept here as named constants):
 *  - ORACLE_E4_BIAS = 15 for both E4 lanes, IEEE-style gradual underflow at
 *    exponent field 0, every exponent field finite (no Inf/NaN codes),
 *    sign|exponent|mantissa from the most significant bit down.
 *    The bias itself is a reading: parity unpinned.
 *  - Rounding is to nearest, ties to the even code; |x| at or above the
 *    largest finite value saturates to it (+-Inf too).
 *  - NaN encodes as code 0 in an E4 lane.  The RMS lane maps every negative
 *    input, -0 included, to code 0.  The first-moment lane keeps the sign of
 *    zero.
 *  - Binary16 lanes and the BF16 parameter output follow IEEE
 *    round-to-nearest-even with overflow to Inf.
 *  - A block whose new moment holds a NaN has a NaN absmax; every code in it
 *    is then 255, because the midpoint search orders NaN above every number,
 *    as the page's bucketize does.
 *
 * Arithmetic: every float operation is one IEEE binary32 operation rounded to
 * nearest even (the build uses SSE arithmetic, -ffp-contract=off, no fast
 * math), sqrtf and division are correctly rounded, denormals are kept.
 * Codec tables are built in double precision, in which every value of every
 * lane is exact.
 */
#include <math.h>
#include <quadmath.h>
#include <stdio.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_E4_BIAS 15
#define ORACLE_BLOCK 2048

/* ---------------------------------------------------------------------- */
/* Codec tables.                                                           */
/* ---------------------------------------------------------------------- */

/* Non-negative magnitudes in ascending code order.  Each table ends with the
 * largest finite value; the binary16 and bfloat16 tables carry one more entry
 * standing for Inf, placed at the next power of two so that the usual
 * IEEE overflow threshold (largest finite plus half an ulp, ties to even)
 * falls out of the same nearest-entry rule. */
static double tab_m_e4[0x8000];     /* E4M11 magnitudes, codes 0x0000..0x7FFF */
static double tab_r_e4[0x10000];    /* E4M12 values,     codes 0x0000..0xFFFF */
static double tab_h[0x7C01];        /* binary16 magnitudes 0x0000..0x7BFF, 0x7C00 = Inf */
static double tab_bf[0x7F81];       /* bfloat16 magnitudes 0x0000..0x7F7F, 0x7F80 = Inf */
static int tables_ready = 0;

/* Value of a sign-less mini float with `ebits` exponent bits, `mbits`
 * mantissa bits and exponent bias `bias`: exponent field 0 is the subnormal
 * binade f * 2^(1-bias-mbits); otherwise (2^mbits + f) * 2^(e-bias-mbits). */
static double minifloat_value(unsigned code, int mbits, int bias) {
    unsigned e = code >> mbits;
    unsigned f = code & ((1u << mbits) - 1u);
    if (e == 0) return ldexp((double)f, 1 - bias - mbits);
    return ldexp((double)((1u << mbits) + f), (int)e - bias - mbits);
}

static void build_tables(void) {
    if (tables_ready) return;
    for (unsigned c = 0; c < 0x8000; ++c) tab_m_e4[c] = minifloat_value(c, 11, ORACLE_E4_BIAS);
    for (unsigned c = 0; c < 0x10000; ++c) tab_r_e4[c] = minifloat_value(c, 12, ORACLE_E4_BIAS);
    for (unsigned c = 0; c < 0x7C00; ++c) tab_h[c] = minifloat_value(c, 10, 15);
    tab_h[0x7C00] = 65536.0;                       /* 2^16: Inf as a rounding target */
    for (unsigned c = 0; c < 0x7F80; ++c) tab_bf[c] = minifloat_value(c, 7, 127);
    tab_bf[0x7F80] = ldexp(1.0, 128);              /* 2^128: Inf as a rounding target */
    tables_ready = 1;
}

/* Nearest entry of an ascending table to a >= 0: the bracketing pair
 * tab[k] <= a < tab[k+1] is found by bisection, then a is compared with the
 * pair's exact midpoint (exact in double: both ends have at most 24
 * significant bits).  Below the midpoint gives k, above gives k+1, on it
 * gives whichever of the two codes is even.  a at or past the last entry
 * gives the last code. */
static unsigned nearest_code(const double* tab, unsigned ncodes, double a) {
    if (a >= tab[ncodes - 1]) return ncodes - 1;
    unsigned lo = 0, hi = ncodes - 1;             /* tab[lo] <= a < tab[hi] */
    while (hi - lo > 1) {
        unsigned mid = lo + (hi - lo) / 2;
        if (tab[mid] <= a) lo = mid; else hi = mid;
    }
    double midpoint = 0.5 * (tab[lo] + tab[lo + 1]);
    if (a < midpoint) return lo;
    if (a > midpoint) return lo + 1;
    return (lo % 2 == 0) ? lo : lo + 1;
}

/* ---------------------------------------------------------------------- */
/* Lane codecs.                                                            */
/* ---------------------------------------------------------------------- */

/* E4M11 first-moment lane: bit 15 sign, bits 14..11 exponent, 10..0 mantissa. */
float oracle_decode_m_e4(uint16_t code) {
    build_tables();
    double mag = tab_m_e4[code & 0x7FFF];
    return (float)((code & 0x8000) ? -mag : mag);
}

uint16_t oracle_encode_m_e4(float x) {
    build_tables();
    if (isnan(x)) return 0;
    unsigned sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs((double)x);                   /* +-Inf lands on the last entry */
    return (uint16_t)(sign | nearest_code(tab_m_e4, 0x8000, a));
}

/* E4M12 RMS lane: no sign, bits 15..12 exponent, 11..0 mantissa. */
float oracle_decode_r_e4(uint16_t code) {
    build_tables();
    return (float)tab_r_e4[code];
}

uint16_t oracle_encode_r_e4(float x) {
    build_tables();
    if (isnan(x) || signbit(x)) return 0;         /* negative, -0 and NaN -> 0 */
    return (uint16_t)nearest_code(tab_r_e4, 0x10000, (double)x);
}

/* IEEE binary16: bit 15 sign, 5 exponent bits (bias 15), 10 mantissa bits. */
float oracle_decode_f16(uint16_t code) {
    build_tables();
    unsigned mag = code & 0x7FFF;
    double v;
    if (mag < 0x7C00) v = tab_h[mag];
    else if (mag == 0x7C00) v = INFINITY;
    else v = NAN;
    return (float)((code & 0x8000) ? -v : v);
}

uint16_t oracle_encode_f16(float x) {
    build_tables();
    unsigned sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7E00u);
    return (uint16_t)(sign | nearest_code(tab_h, 0x7C01, fabs((double)x)));
}

/* bfloat16 (the parameter output of the blockwise mode, and 16-bit
 * parameters/gradients of the typed step). */
float oracle_decode_bf16(uint16_t code) {
    build_tables();
    unsigned mag = code & 0x7FFF;
    double v;
    if (mag < 0x7F80) v = tab_bf[mag];
    else if (mag == 0x7F80) v = INFINITY;
    else v = NAN;
    return (float)((code & 0x8000) ? -v : v);
}

uint16_t oracle_encode_bf16(float x) {
    build_tables();
    unsigned sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    return (uint16_t)(sign | nearest_code(tab_bf, 0x7F81, fabs((double)x)));
}

/* Batch forms, for tests. */
void oracle_encode_batch(int lane, const float* x, uint16_t* out, size_t n) {
    build_tables();
    ptrdiff_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (ptrdiff_t)n; ++i) {
        switch (lane) {
            case 0: out[i] = oracle_encode_m_e4(x[i]); break;
            case 1: out[i] = oracle_encode_r_e4(x[i]); break;
            case 2: out[i] = oracle_encode_f16(x[i]); break;
            default: out[i] = oracle_encode_bf16(x[i]); break;
        }
    }
}

void oracle_decode_batch(int lane, const uint16_t* c, float* out, size_t n) {
    build_tables();
    for (size_t i = 0; i < n; ++i) {
        switch (lane) {
            case 0: out[i] = oracle_decode_m_e4(c[i]); break;
            case 1: out[i] = oracle_decode_r_e4(c[i]); break;
            case 2: out[i] = oracle_decode_f16(c[i]); break;
            default: out[i] = oracle_decode_bf16(c[i]); break;
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Scalars.                                                                */
/* ---------------------------------------------------------------------- */

/* The per-call scalars.  The KBench reference holds lr, the betas, eps, wd,
 * the bias corrections and their quotients as double-precision host numbers
 * and meets FP32 tensors with them, so each is formed in double and rounded
 * to binary32 once, at the point where it meets a tensor.
 * Layout: [0] beta1, [1] 1-beta1, [2] beta2, [3] 1-beta2,
 *         [4] bc2 = 1-beta2^t, [5] lr/bc1 with bc1 = 1-beta1^t,
 *         [6] 1-lr*wd, [7] eps. */
void oracle_scalars(double lr, double beta1, double beta2, double eps, double wd,
                    long long step, float out[8]) {
    double bc1 = 1.0 - pow(beta1, (double)step);
    double bc2 = 1.0 - pow(beta2, (double)step);
    out[0] = (float)beta1;
    out[1] = (float)(1.0 - beta1);
    out[2] = (float)beta2;
    out[3] = (float)(1.0 - beta2);
    out[4] = (float)bc2;
    out[5] = (float)(lr / bc1);
    out[6] = (float)(1.0 - lr * wd);
    out[7] = (float)eps;
}

/* ---------------------------------------------------------------------- */
/* The FP32 AdamW element update (shared by every mode of the oracle).     */
/* ---------------------------------------------------------------------- */

typedef struct {
    float m1, v1, p1;
} oracle_elem;

/* New moments from the prior ones, then the bias-corrected step with
 * decoupled decay, in the order the KBench reference writes it:
 *   m' = beta1*m + (1-beta1)*g
 *   v' = beta2*v + ((1-beta2)*g)*g
 *   denom = sqrt(v'/bc2) + eps
 *   upd = ((lr/bc1)*m') / denom
 *   p' = p*(1-lr*wd) - upd
 * which equals the TurboAdam equation block in exact arithmetic. */
static oracle_elem adamw_element(float p, float g, float m, float v, const float* s) {
    oracle_elem r;
    float beta1 = s[0], one_m_beta1 = s[1], beta2 = s[2], one_m_beta2 = s[3];
    float bc2 = s[4], lr_over_bc1 = s[5], decay = s[6], eps = s[7];
    float a = beta1 * m;
    float b = one_m_beta1 * g;
    r.m1 = a + b;
    float c = beta2 * v;
    float d = one_m_beta2 * g;
    float e = d * g;
    r.v1 = c + e;
    float q = r.v1 / bc2;
    float denom = sqrtf(q) + eps;
    float num = lr_over_bc1 * r.m1;
    float upd = num / denom;
    float kept = p * decay;
    r.p1 = kept - upd;
    return r;
}

static int elem_nonfinite(const oracle_elem* e) {
    return !isfinite(e->p1) || !isfinite(e->m1) || !isfinite(e->v1);
}

/* ---------------------------------------------------------------------- */
/* Elementwise modes.                                                      */
/* ---------------------------------------------------------------------- */

/* Plain FP32 AdamW (the comparison mode with two FP32 moment tensors). */
unsigned long long oracle_step_fp32(float* p, const float* g, float* m, float* v,
                                    size_t n, const float s[8]) {
    unsigned long long bad = 0;
    ptrdiff_t i;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (i = 0; i < (ptrdiff_t)n; ++i) {
        oracle_elem e = adamw_element(p[i], g[i], m[i], v[i], s);
        p[i] = e.p1;
        m[i] = e.m1;
        v[i] = e.v1;
        bad += (unsigned long long)elem_nonfinite(&e);
    }
    return bad;
}

/* Packed modes: one uint32 word per parameter, first moment in the low half,
 * RMS in the high half.  lane_kind 1 = E4M11/E4M12, 2 = binary16/binary16.
 * Decode the prior state, square the RMS, update in FP32 with the new
 * moments, and only then encode m' and sqrt(v') for the next step. */
unsigned long long oracle_step_packed(int lane_kind, float* p, const float* g, uint32_t* w,
                                      size_t n, const float s[8]) {
    build_tables();
    unsigned long long bad = 0;
    ptrdiff_t i;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (i = 0; i < (ptrdiff_t)n; ++i) {
        uint16_t lo = (uint16_t)(w[i] & 0xFFFFu);
        uint16_t hi = (uint16_t)(w[i] >> 16);
        float m, r;
        if (lane_kind == 1) {
            m = oracle_decode_m_e4(lo);
            r = oracle_decode_r_e4(hi);
        } else {
            m = oracle_decode_f16(lo);
            r = oracle_decode_f16(hi);
        }
        float v = r * r;
        oracle_elem e = adamw_element(p[i], g[i], m, v, s);
        float r1 = sqrtf(e.v1);
        uint16_t mc, rc;
        if (lane_kind == 1) {
            mc = oracle_encode_m_e4(e.m1);
            rc = oracle_encode_r_e4(r1);
        } else {
            mc = oracle_encode_f16(e.m1);
            rc = oracle_encode_f16(r1);
        }
        p[i] = e.p1;
        w[i] = ((uint32_t)rc << 16) | (uint32_t)mc;
        bad += (unsigned long long)elem_nonfinite(&e);
    }
    return bad;
}

/* ---------------------------------------------------------------------- */
/* Typed parameters and gradients.                                         */
/* ---------------------------------------------------------------------- */

/* Element types: 0 binary32, 1 bfloat16, 2 binary16 (16-bit ones as their
 * bit patterns).  The KBench reference widens parameters and gradients to
 * FP32 before the update and narrows the new parameters afterwards; here a
 * 16-bit value widens exactly and the new parameter is rounded to nearest
 * even in its own type. */
static float widen_at(int dt, const void* base, size_t i) {
    if (dt == 0) return ((const float*)base)[i];
    uint16_t c = ((const uint16_t*)base)[i];
    return dt == 1 ? oracle_decode_bf16(c) : oracle_decode_f16(c);
}

static void narrow_at(int dt, void* base, size_t i, float x) {
    if (dt == 0) ((float*)base)[i] = x;
    else ((uint16_t*)base)[i] = dt == 1 ? oracle_encode_bf16(x) : oracle_encode_f16(x);
}

/* One step over n elements with typed parameters (pdt) and gradients (gdt).
 * state_kind 0: FP32 moments in s0 (m) and s1 (v); 1: packed E4 words in s0;
 * 2: packed binary16 words in s0.  Returns the non-finite count. */
unsigned long long oracle_step_typed(int state_kind, int pdt, int gdt, void* p, const void* g,
                                     void* s0, void* s1, size_t n, const float s[8]) {
    build_tables();
    unsigned long long bad = 0;
    ptrdiff_t i;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (i = 0; i < (ptrdiff_t)n; ++i) {
        float pw = widen_at(pdt, p, (size_t)i);
        float gw = widen_at(gdt, g, (size_t)i);
        oracle_elem e;
        if (state_kind == 0) {
            float* m = (float*)s0;
            float* v = (float*)s1;
            e = adamw_element(pw, gw, m[i], v[i], s);
            m[i] = e.m1;
            v[i] = e.v1;
        } else {
            uint32_t* w = (uint32_t*)s0;
            uint16_t lo = (uint16_t)(w[i] & 0xFFFFu), hi = (uint16_t)(w[i] >> 16);
            float m = state_kind == 1 ? oracle_decode_m_e4(lo) : oracle_decode_f16(lo);
            float r = state_kind == 1 ? oracle_decode_r_e4(hi) : oracle_decode_f16(hi);
            float v = r * r;
            e = adamw_element(pw, gw, m, v, s);
            float r1 = sqrtf(e.v1);
            uint16_t mc = state_kind == 1 ? oracle_encode_m_e4(e.m1) : oracle_encode_f16(e.m1);
            uint16_t rc = state_kind == 1 ? oracle_encode_r_e4(r1) : oracle_encode_f16(r1);
            w[i] = ((uint32_t)rc << 16) | (uint32_t)mc;
        }
        narrow_at(pdt, p, (size_t)i, e.p1);
        bad += (unsigned long long)elem_nonfinite(&e);
    }
    return bad;
}

/* ---------------------------------------------------------------------- */
/* Blockwise 8-bit mode (KBench quantized-optimizer-state reference).      */
/* ---------------------------------------------------------------------- */

/* Index of the first midpoint that is not below c, i.e. the number of
 * midpoints strictly below c (an exact tie goes to the lower map entry).
 * NaN is ordered above every number, as a sorted search orders it. */
static unsigned search_code(const float* mid, unsigned nmid, float c) {
    if (isnan(c)) return nmid;
    unsigned k = 0;
    while (k < nmid && mid[k] < c) ++k;
    return k;
}

/* Requantise one block of new moments: absmax of the block (NaN if any
 * element is NaN), normalise by the absmax clamped below at the binary32
 * value of 1e-30, and pick each element's map entry through the 255 FP32
 * midpoints.  The stored absmax is the unclamped one. */
static float requantise_block(const float* x, const float* qmap, uint8_t* code, size_t len) {
    float mid[255];
    for (unsigned j = 0; j < 255; ++j) mid[j] = (qmap[j] + qmap[j + 1]) * 0.5f;
    float amax = 0.0f;
    int saw_nan = 0;
    for (size_t i = 0; i < len; ++i) {
        if (isnan(x[i])) saw_nan = 1;
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    if (saw_nan) amax = NAN;
    float floor_val = (float)1e-30;
    float d = isnan(amax) ? amax : (amax < floor_val ? floor_val : amax);
    for (size_t i = 0; i < len; ++i) {
        float c = x[i] / d;
        code[i] = (uint8_t)search_code(mid, 255, c);
    }
    return amax;
}

/* One blockwise step over n parameters (n a multiple of 2048).  Parameters
 * are read as FP32 and left untouched; the updated parameters go to p_out as
 * BF16.  m_code/v_code and the per-block absmax arrays are replaced by the
 * requantised new moments.  qmap_m and qmap_v are ascending 256-entry maps.
 * Returns the number of elements whose p', m' or v' is non-finite, or
 * (unsigned long long)-1 if n is not a multiple of the block length. */
unsigned long long oracle_step_blockwise(const float* p, const float* g,
                                         uint8_t* m_code, float* m_absmax,
                                         uint8_t* v_code, float* v_absmax,
                                         const float* qmap_m, const float* qmap_v,
                                         uint16_t* p_out, size_t n, const float s[8]) {
    build_tables();
    if (n % ORACLE_BLOCK != 0) return (unsigned long long)-1;
    size_t nb = n / ORACLE_BLOCK;
    unsigned long long bad = 0;
    ptrdiff_t b;
#pragma omp parallel for schedule(static) reduction(+ : bad)
    for (b = 0; b < (ptrdiff_t)nb; ++b) {
        float m1[ORACLE_BLOCK], v1[ORACLE_BLOCK];
        size_t base = (size_t)b * ORACLE_BLOCK;
        float am = m_absmax[b], av = v_absmax[b];
        for (size_t i = 0; i < ORACLE_BLOCK; ++i) {
            float m = qmap_m[m_code[base + i]] * am;
            float v = qmap_v[v_code[base + i]] * av;
            oracle_elem e = adamw_element(p[base + i], g[base + i], m, v, s);
            m1[i] = e.m1;
            v1[i] = e.v1;
            p_out[base + i] = oracle_encode_bf16(e.p1);
            bad += (unsigned long long)elem_nonfinite(&e);
        }
        m_absmax[b] = requantise_block(m1, qmap_m, m_code + base, ORACLE_BLOCK);
        v_absmax[b] = requantise_block(v1, qmap_v, v_code + base, ORACLE_BLOCK);
    }
    return bad;
}

/* Midpoint search alone, for tests against a library search. */
void oracle_search_codes(const float* qmap, const float* c, uint8_t* code, size_t n) {
    float mid[255];
    for (unsigned j = 0; j < 255; ++j) mid[j] = (qmap[j] + qmap[j + 1]) * 0.5f;
    for (size_t i = 0; i < n; ++i) code[i] = (uint8_t)search_code(mid, 255, c[i]);
}

/* Threads the parallel loops use. */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads the batch routines use from now on (tests and timing). */
void oracle_set_num_threads(int k) {
#ifdef _OPENMP
    if (k > 0) omp_set_num_threads(k);
#else
    (void)k;
#endif
}

int oracle_block_len(void) { return ORACLE_BLOCK; }
int oracle_e4_bias(void) { return ORACLE_E4_BIAS; }

/* ---------------------------------------------------------------------- */
/* Gradient pre-pass: sum of squares, non-finite count, clip coefficient.  */
/* ---------------------------------------------------------------------- */

/* The pages run AdamW on ordinary dense gradients of FP32, FP16 or BF16
 * parameters (TurboAdam package page, Verification; KBench reference,
 * `grads.float()`), and the smoke check of the Packed AdamW Reference README
 * counts non-finite optimizer values.  The pre-pass gathers, in one read of
 * the gradients, what a training loop needs before the update: the squared
 * L2 norm of all gradients, the number of non-finite gradient values, and
 * the usual clipping coefficient min(1, max_norm / (norm + 1e-6)).
 *
 * The sum is exact: every binary32 value is m * 2^e with an integer m below
 * 2^24 and e >= -149, so its square m^2 * 2^(2e) is an integer multiple of
 * 2^-298 below 2^554.  The accumulator holds the sum as a 640-bit integer
 * in units of 2^-298 (room for 2^86 maximal terms), and the value is that
 * integer rounded once to double, to nearest even.  Any NaN makes the sum
 * NaN; otherwise any infinity makes it +Inf, as IEEE addition of
 * non-negative terms does. */
#define ORACLE_ACC_LIMBS 10

typedef struct {
    uint64_t limb[ORACLE_ACC_LIMBS];   /* least significant first */
    unsigned long long nonfinite;
    int has_nan;
    int has_inf;
} oracle_sumsq_acc;

static void acc_add_square(oracle_sumsq_acc* a, float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    uint32_t ex = (u >> 23) & 0xFFu, mant = u & 0x7FFFFFu;
    if (ex == 0xFFu) {
        a->nonfinite++;
        if (mant) a->has_nan = 1;
        else a->has_inf = 1;
        return;
    }
    uint64_t m = ex ? (mant | 0x800000u) : mant;   /* x = m * 2^e */
    int e = ex ? (int)ex - 150 : -149;
    if (m == 0) return;
    uint64_t m2 = m * m;                            /* < 2^48 */
    int shift = 2 * e + 298;                        /* 0 .. 506 */
    int k = shift >> 6, off = shift & 63;
    unsigned __int128 t = (unsigned __int128)m2 << off;
    uint64_t parts[2] = {(uint64_t)t, (uint64_t)(t >> 64)};
    unsigned carry = 0;
    for (int i = k; i < ORACLE_ACC_LIMBS; ++i) {
        uint64_t add = (i - k < 2) ? parts[i - k] : 0;
        uint64_t s1 = a->limb[i] + add;
        unsigned c1 = s1 < add;
        uint64_t s2 = s1 + carry;
        unsigned c2 = s2 < carry;
        a->limb[i] = s2;
        carry = c1 | c2;
        if (i - k >= 1 && carry == 0) break;
    }
}

static void acc_merge(oracle_sumsq_acc* dst, const oracle_sumsq_acc* src) {
    unsigned carry = 0;
    for (int i = 0; i < ORACLE_ACC_LIMBS; ++i) {
        uint64_t s1 = dst->limb[i] + src->limb[i];
        unsigned c1 = s1 < src->limb[i];
        uint64_t s2 = s1 + carry;
        unsigned c2 = s2 < carry;
        dst->limb[i] = s2;
        carry = c1 | c2;
    }
    dst->nonfinite += src->nonfinite;
    dst->has_nan |= src->has_nan;
    dst->has_inf |= src->has_inf;
}

/* Add the squares of n gradients of element type gdt (0 binary32,
 * 1 bfloat16, 2 binary16; 16-bit ones as bit patterns) to the accumulator
 * (zero-filled by the caller before the first call). */
void oracle_sumsq_add(oracle_sumsq_acc* acc, int gdt, const void* g, size_t n) {
    build_tables();
#pragma omp parallel
    {
        oracle_sumsq_acc local;
        memset(&local, 0, sizeof(local));
        ptrdiff_t i;
#pragma omp for schedule(static)
        for (i = 0; i < (ptrdiff_t)n; ++i) acc_add_square(&local, widen_at(gdt, g, (size_t)i));
#pragma omp critical
        acc_merge(acc, &local);
    }
}

static int acc_bit(const oracle_sumsq_acc* a, int i) {
    return (int)((a->limb[i >> 6] >> (i & 63)) & 1u);
}

/* The accumulated sum of squares, rounded once to double (nearest even). */
double oracle_sumsq_value(const oracle_sumsq_acc* a) {
    if (a->has_nan) return NAN;
    if (a->has_inf) return INFINITY;
    int top = -1;
    for (int i = ORACLE_ACC_LIMBS * 64 - 1; i >= 0; --i)
        if (acc_bit(a, i)) { top = i; break; }
    if (top < 0) return 0.0;
    int lo = top - 52 > 0 ? top - 52 : 0;
    uint64_t mant = 0;
    for (int i = top; i >= lo; --i) mant = (mant << 1) | (uint64_t)acc_bit(a, i);
    if (lo > 0) {
        int round = acc_bit(a, lo - 1), sticky = 0;
        for (int i = lo - 2; i >= 0 && !sticky; --i) sticky = acc_bit(a, i);
        if (round && (sticky || (mant & 1u))) {
            mant += 1;
            if (mant >> 53) { mant >>= 1; lo += 1; }
        }
    }
    return ldexp((double)mant, lo - 298);
}

/* Clipping coefficient of the global norm sqrt(sumsq) for max_norm, in
 * double: max_norm / (norm + 1e-6), capped at 1 (a NaN stays NaN), then
 * rounded to binary32 once. */
float oracle_clip_scale(double sumsq, double max_norm) {
    double coef = max_norm / (sqrt(sumsq) + 1e-6);
    if (isnan(coef)) return NAN;
    return (float)(coef < 1.0 ? coef : 1.0);
}

/* Gradients scaled before the update: out[i] = widen(g[i]) * scale, one
 * binary32 multiplication per element. */
void oracle_scale_grads(int gdt, const void* g, float scale, float* out, size_t n) {
    build_tables();
    for (size_t i = 0; i < n; ++i) out[i] = widen_at(gdt, g, i) * scale;
}

/* ---------------------------------------------------------------------- */
/* TurboAdam compressed state: UState first moment, 1Q second moment.     */
/* ---------------------------------------------------------------------- */

/* TurboAdam package page, "How it works", "UState", "1Q" and "Fused CUDA
 * path": AdamW from FP32 transient moments, with the first moment persisted
 * as UState (normalised update units q = (m/bc1) / (sqrt(v_persisted/bc2) +
 * eps), a four-level code per value, one bf16 mean per 64 values recentred
 * on decode, antithetic stochastic rounding, a one-step-lagged tensor scale
 * of 1.1 x the residual RMS) and the second moment persisted as 1Q (a
 * logarithmic grid per 128-value block between two fp16 log endpoints,
 * packed indices, stochastic rounding between decoded positive values from
 * a counter hash).  The page prints no code for any of these; the readings
 * taken here (parity unpinned where the page is silent) are:
 *
 *  1Q, L = 2^bits indices: index 0 is exactly 0; index k in 1..L-1 decodes to
 *    level_k = RN32(2^x), x = lo + (hi - lo) * (k - 1) / (L - 2) in double
 *    and 2^x the exact power (not a double exp2 rounded again), where lo
 *    and hi are the block's fp16 endpoints: log2 (in double) of the
 *    smallest positive finite v rounded down to fp16, and of the largest
 *    rounded up.  Encode: 0 -> 0, NaN -> 0, +Inf -> L-1; else the largest k
 *    with level_k <= v (at least 1), then k+1 with probability
 *    (v - level_k) / (level_{k+1} - level_k): chosen when u < that fraction.
 *  UState: codes 0..3 stand for -1.5, -0.5, 0.5, 1.5 times the scale.
 *    Encode: mean = bf16(RN32(pairwise double sum of q over the group /
 *    count)); r = q - mean; x = r / s_enc (s_enc = 0: x = 0), clamped to
 *    [-1.5, 1.5]; the lower bracketing level k, then k+1 when u < x - L_k.
 *    The two values 2j, 2j+1 of a pair use u and 1 - u (antithetic).
 *    Decode: q = mean + s_dec * (L_code - Lbar), Lbar the group's mean level,
 *    which keeps the decoded group mean at the stored mean.
 *  The first moment of step t-1 is rebuilt as
 *    m = (q * bc1_{t-1}) * (sqrt(v_persisted / bc2_{t-1}) + eps);
 *    at t = 1 the state is empty and both prior moments are 0.
 *  The residual sum of squares is a perfect pairwise tree, in double, over
 *    r^2 in index order padded with zeros to a power of two; after the
 *    step s_dec <- s_enc, s_enc <- RN32(factor * sqrt(sum / n)), acc <- 0.
 *  Layout (the page's "Fused CUDA path": power-of-two storage blocks from
 *    32 to 1024 values, UState mean blocks that divide the storage block,
 *    and 2, 3, 4, 6 or 8 index bits; defaults 128, 64 and 4): a 1Q block
 *    of B values shares one pair of endpoints; a UState group of G values
 *    (G a power of two dividing B) shares one mean; the storage block
 *    does not otherwise enter the arithmetic.  Indices are packed densely,
 *    value i in bits [b*i, b*i + b) of the little-endian bit stream of the
 *    index words (so 3- and 6-bit indices straddle words); UState codes
 *    likewise at 2 bits.
 *  Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11), the
 *    counter-based generator Triton builds in, so the counter hash that a
 *    PyTorch path and a Triton path can share.  Key (low and high 32 bits of
 *    the seed); counter (j, step, tensor id, stream) for the values
 *    4j..4j+3, with j and step taken modulo 2^32.  Stream 0: the high 24
 *    bits of word k give the 1Q draw of value 4j+k.  Stream 1: the high 24
 *    bits of words 0 and 1 give the UState draws of the pairs (4j, 4j+1)
 *    and (4j+2, 4j+3).  A draw is those 24 bits times 2^-24. */

#define T_MAX_BLOCK 1024

/* Ten rounds of the Philox-4x32 bijection.  A round multiplies words 0 and 2
 * by the two round multipliers, xors each product's high half with the other
 * odd word and a key word, and permutes; the key is bumped by the two Weyl
 * constants before every round but the first. */
static void philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int r = 0; r < 10; ++r) {
        if (r) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        uint64_t p0 = (uint64_t)0xD2511F53u * x0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ x1 ^ k0, n2 = hi0 ^ x3 ^ k1;
        x0 = n0; x1 = lo1; x2 = n2; x3 = lo0;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

void oracle_philox4x32(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    philox4x32_10(ctr, key, out);
}

/* The draws of values 4j..4j+3: q1[k] for 1Q, us[0..1] for the UState pairs. */
static void turbo_draws(unsigned long long seed, uint32_t tensor_id, long long step, size_t j,
                        float q1[4], float us[2]) {
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t ctr[4] = {(uint32_t)j, (uint32_t)step, tensor_id, 0u}, w[4];
    philox4x32_10(ctr, key, w);
    for (int k = 0; k < 4; ++k) q1[k] = (float)(w[k] >> 8) * 0x1p-24f;
    ctr[3] = 1u;
    philox4x32_10(ctr, key, w);
    for (int k = 0; k < 2; ++k) us[k] = (float)(w[k] >> 8) * 0x1p-24f;
}

/* fp16 value of x rounded toward -Inf (dir < 0) or +Inf (dir > 0), as bits:
 * the nearest binary16 value on that side, found in the ordered table. */
static uint16_t f16_directed(double x, int dir) {
    build_tables();
    /* tab_h holds the 0x7C01 non-negative binary16 values, ascending. */
    double a = fabs(x);
    int neg = x < 0;
    /* largest non-negative code with value <= a, and smallest with value >= a */
    unsigned lo = 0, hi = 0x7C00;
    if (a >= tab_h[0x7C00]) { lo = hi = 0x7C00; }
    else {
        while (hi - lo > 1) {
            unsigned mid = (lo + hi) / 2;
            if (tab_h[mid] <= a) lo = mid; else hi = mid;
        }
        if (tab_h[lo] == a) hi = lo;
    }
    /* toward +Inf: for x >= 0 the upper code, for x < 0 the lower magnitude */
    unsigned mag = (dir > 0) ? (neg ? lo : hi) : (neg ? hi : lo);
    if (mag == 0) return neg && dir < 0 ? 0x8000u : 0;
    return (uint16_t)((neg ? 0x8000u : 0u) | mag);
}

static double f16_value(uint16_t h) {
    return (double)oracle_decode_f16(h);
}

/* RN32(2^x), the exact power of two rounded once to binary32, for a double
 * x.  For an integer x the power is a power of two (a binary32 value, or the
 * midpoint 2^-150 that rounds to even 0, or beyond the range); for any other
 * x it is irrational, so it never lies on a binary32 midpoint and the
 * rounding is well defined.  The 64-bit-significand exp2l is within a few
 * of its ulps (2^-62 relative): when every value within 2^-56 of its result
 * rounds to the same binary32 value, that is the answer.  Otherwise (about
 * one x in 2^31) the binary128 exp2q (error below 2^-110) decides with a
 * 2^-100 margin; a power closer than that to a midpoint stops the oracle
 * rather than let it guess. */
static float exp2_rn32(double x) {
    if (isnan(x)) return NAN;
    if (x >= 128.0) return INFINITY;
    if (x <= -150.0) return 0.0f;
    if (x == nearbyint(x)) return ldexpf(1.0f, (int)x);
    const long double y = exp2l((long double)x);
    const float a = (float)(y * (1.0L - 0x1p-56L)), b = (float)(y * (1.0L + 0x1p-56L));
    if (a == b) return a;
    const __float128 q = exp2q((__float128)x), m = (__float128)0x1p-100;
    const float c = (float)(q * (1 - m)), d = (float)(q * (1 + m));
    if (c == d) return c;
    fprintf(stderr, "oracle: 2^%a lies within 2^-100 of a binary32 midpoint\n", x);
    abort();
}

static void level_table(uint16_t lo16, uint16_t hi16, int L, float* lev) {
    double lo = f16_value(lo16), hi = f16_value(hi16);
    lev[0] = 0.0f;
    for (int k = 1; k < L; ++k) {
        double x = lo + ((hi - lo) * (double)(k - 1)) / (double)(L - 2);
        lev[k] = exp2_rn32(x);
    }
}

static double pairwise_sum(const double* a, size_t n) {   /* n a power of two */
    if (n == 1) return a[0];
    return pairwise_sum(a, n / 2) + pairwise_sum(a + n / 2, n / 2);
}

/* The two 1Q endpoints a one-value block holding v would get, for n values
 * (tests): low half RD16(log2 v), high half RU16(log2 v). */
void oracle_q1_ends_batch(const float* v, uint32_t* out, size_t n) {
    build_tables();
    ptrdiff_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < (ptrdiff_t)n; ++i) {
        const double y = log2((double)v[i]);
        out[i] = (uint32_t)f16_directed(y, -1) | ((uint32_t)f16_directed(y, +1) << 16);
    }
}

/* The decoded values of a block's 2^bits indices. */
void oracle_q1_levels(uint16_t lo16, uint16_t hi16, int bits, float* lev) {
    build_tables();
    level_table(lo16, hi16, 1 << bits, lev);
}

/* RN32(2^x) for n doubles x (the level rounding of exp2_rn32 alone, so
 * that the tests can reach its binary128 branch with x near midpoints). */
void oracle_exp2_rn32_batch(const double* x, size_t n, float* out) {
    for (size_t i = 0; i < n; ++i) out[i] = exp2_rn32(x[i]);
}

/* The levels of n blocks at once: ends[i] holds block i's fp16 endpoints
 * (lower in the low 16 bits), lev[i * 2^bits + k] its level k. */
void oracle_q1_levels_batch(const uint32_t* ends, size_t n, int bits, float* lev) {
    build_tables();
    const int L = 1 << bits;
    for (size_t i = 0; i < n; ++i)
        level_table((uint16_t)(ends[i] & 0xFFFFu), (uint16_t)(ends[i] >> 16), L, lev + i * (size_t)L);
}

/* 1Q encode of one block of len (<= 1024) second-moment values with draws u:
 * the fp16 endpoints, each value's index, and the decoded (persisted) value. */
void oracle_q1_block(const float* v, size_t len, int bits, const float* u, uint8_t* idx, uint16_t ends[2],
                     float* vdec) {
    build_tables();
    const int L = 1 << bits;
    float vmin = INFINITY, vmax = 0.0f;
    for (size_t i = 0; i < len; ++i) {
        if (v[i] > 0.0f && isfinite(v[i])) {
            if (v[i] < vmin) vmin = v[i];
            if (v[i] > vmax) vmax = v[i];
        }
    }
    uint16_t lo16 = 0, hi16 = 0;
    if (vmax > 0.0f) {
        lo16 = f16_directed(log2((double)vmin), -1);
        hi16 = f16_directed(log2((double)vmax), +1);
    }
    ends[0] = lo16;
    ends[1] = hi16;
    float lev[256];
    level_table(lo16, hi16, L, lev);
    for (size_t i = 0; i < len; ++i) {
        float x = v[i];
        unsigned k;
        if (!(x > 0.0f)) k = 0;                      /* zero, negative, NaN */
        else if (isinf(x)) k = (unsigned)(L - 1);
        else {
            k = 1;
            while (k + 1 < (unsigned)L && lev[k + 1] <= x) ++k;
            if (k < (unsigned)(L - 1) && x > lev[k]) {
                float f = (x - lev[k]) / (lev[k + 1] - lev[k]);
                if (u[i] < f) ++k;
            }
        }
        idx[i] = (uint8_t)k;
        vdec[i] = lev[k];
    }
}

static const float T_LEVEL[4] = {-1.5f, -0.5f, 0.5f, 1.5f};

/* UState encode of one group of len (<= group) values q, group a power of
 * two up to 1024, whose first value has index `first` in its tensor, with
 * encode scale s_enc and one draw per pair of the tensor's values 2j and
 * 2j+1 (the second using 1 - u; u_pair[0] is the draw of the pair holding
 * the group's first value, so a one-value group at an odd index takes
 * 1 - u): the bf16 mean (the pairwise tree over the group's values padded
 * with zeros to `group`, divided by len), each code, and each residual's
 * square (double). */
void oracle_ustate_group(const float* q, size_t len, size_t group, size_t first, float s_enc, const float* u_pair,
                         uint8_t* codes, uint16_t* mean16, double* r2) {
    build_tables();
    double qd[T_MAX_BLOCK];
    for (size_t k = 0; k < group; ++k) qd[k] = k < len ? (double)q[k] : 0.0;
    float meanf = (float)(pairwise_sum(qd, group) / (double)len);
    *mean16 = oracle_encode_bf16(meanf);
    float mean = oracle_decode_bf16(*mean16);
    for (size_t i = 0; i < len; ++i) {
        float r = q[i] - mean;
        r2[i] = (double)r * (double)r;
        float x = s_enc > 0.0f ? r / s_enc : 0.0f;
        if (x > 1.5f) x = 1.5f;
        if (x < -1.5f) x = -1.5f;
        float u = u_pair[(first + i) / 2 - first / 2];
        if ((first + i) % 2) u = 1.0f - u;
        unsigned k = (x >= -0.5f) + (x >= 0.5f);
        unsigned code = k;
        if (x >= 1.5f) code = 3;
        else if (u < x - T_LEVEL[k]) code = k + 1;
        codes[i] = (uint8_t)code;
    }
}

/* UState decode of one group: mean + s_dec * (level - mean level). */
void oracle_ustate_decode(const uint8_t* codes, size_t len, uint16_t mean16, float s_dec, float* q) {
    build_tables();
    double lsum = 0.0;
    for (size_t k = 0; k < len; ++k) lsum += T_LEVEL[codes[k]];
    float lbar = (float)(lsum / (double)len);
    float mean = oracle_decode_bf16(mean16);
    for (size_t k = 0; k < len; ++k) q[k] = mean + s_dec * (T_LEVEL[codes[k]] - lbar);
}

/* Value i of a dense little-endian bit stream of `bits`-bit fields: bit j
 * of the field is stream bit bits*i + j, stream bit k is bit k % 32 of word
 * k / 32.  Taken one bit at a time, so that straddling a word needs no
 * case of its own. */
static unsigned get_bits(const uint32_t* w, size_t i, int bits) {
    unsigned v = 0;
    for (int j = 0; j < bits; ++j) {
        size_t k = (size_t)bits * i + (size_t)j;
        v |= ((w[k / 32] >> (k % 32)) & 1u) << j;
    }
    return v;
}

static void put_bits(uint32_t* w, size_t i, int bits, unsigned v) {
    for (int j = 0; j < bits; ++j) {
        size_t k = (size_t)bits * i + (size_t)j;
        uint32_t m = 1u << (k % 32);
        w[k / 32] = ((v >> j) & 1u) ? (w[k / 32] | m) : (w[k / 32] & ~m);
    }
}

/* The layouts the page's fused path takes: index widths 2, 3, 4, 6, 8;
 * storage blocks a power of two from 32 to 1024; mean groups a power of two
 * dividing the block. */
int oracle_turbo_layout_ok(int bits, int block, int group) {
    if (bits != 2 && bits != 3 && bits != 4 && bits != 6 && bits != 8) return 0;
    if (block < 32 || block > T_MAX_BLOCK || (block & (block - 1))) return 0;
    if (group < 1 || group > block || (group & (group - 1))) return 0;
    return 1;
}

/* Persistent bytes of one tensor of n values (TurboAdam package page,
 * Persistent memory: UState 2 bits + one bf16 per group + 12 bytes per
 * tensor; 1Q bits per value + two fp16 per block; an uncompressed moment is
 * FP32), in 32-bit words for the packed streams.  0 for a layout outside
 * oracle_turbo_layout_ok. */
size_t oracle_turbo_state_bytes(int compress_m, int compress_v, int bits, int block, int group, size_t n) {
    if (!oracle_turbo_layout_ok(bits, block, group)) return 0;
    size_t b = 0;
    b += compress_m ? 4 * ((n + 15) / 16) + 2 * ((n + (size_t)group - 1) / (size_t)group) + 12 : 4 * n;
    b += compress_v ? 4 * ((n * (size_t)bits + 31) / 32) + 4 * ((n + (size_t)block - 1) / (size_t)block) : 4 * n;
    return b;
}

/* One TurboAdam step of one tensor of n FP32 parameters, in place.
 * s: the eight scalars of oracle_scalars for this step.  ts: bc1 = 1-beta1^t,
 * bc1_prev = 1-beta1^(t-1), bc2_prev = 1-beta2^(t-1), each rounded once to
 * binary32.  scal: the tensor's s_dec, s_enc, acc (used when compress_m).
 * bits, block, group: the index width, the 1Q block and the UState group
 * (a layout oracle_turbo_layout_ok accepts; the oracle stops otherwise).
 * Returns the number of values whose p', m' or v' is not finite. */
unsigned long long oracle_turbo_step(float* p, const float* g, size_t n, uint32_t tensor_id,
                                     int compress_m, int compress_v, int bits, int block, int group,
                                     uint32_t* m_codes, uint16_t* m_means, float* m_fp32,
                                     uint32_t* v_index, uint16_t* v_ends, float* v_fp32,
                                     float* scal, const float s[8], const float ts[3],
                                     double factor, unsigned long long seed, long long step) {
    build_tables();
    const float bc1 = ts[0], bc1p = ts[1], bc2p = ts[2], bc2 = s[4], eps = s[7];
    if (!oracle_turbo_layout_ok(bits, block, group)) abort();
    const size_t B = (size_t)block, G = (size_t)group;
    const size_t nb = (n + B - 1) / B;
    const size_t ng = (n + G - 1) / G;
    size_t padded = 1;
    while (padded < n) padded *= 2;
    size_t nn = n ? n : 1;
    double* r2 = (double*)calloc(padded, sizeof(double));
    float* m1 = (float*)malloc(sizeof(float) * nn);
    float* v1 = (float*)malloc(sizeof(float) * nn);
    float* vp = (float*)malloc(sizeof(float) * nn);             /* persisted new v */
    float* u1 = (float*)malloc(sizeof(float) * nn);             /* 1Q draws */
    float* up = (float*)malloc(sizeof(float) * (nn / 2 + 2));   /* UState pair draws */
    float* mprev = (float*)calloc(nn, sizeof(float));
    float* vprev = (float*)calloc(nn, sizeof(float));
    unsigned long long bad = 0;
    const float s_dec = compress_m ? scal[0] : 0.0f, s_enc = compress_m ? scal[1] : 0.0f;

    for (size_t j = 0; j * 4 < n; ++j) {
        float q1[4], us[2];
        turbo_draws(seed, tensor_id, step, j, q1, us);
        for (size_t k = 0; k < 4 && 4 * j + k < n; ++k) u1[4 * j + k] = q1[k];
        up[2 * j] = us[0];
        up[2 * j + 1] = us[1];
    }

    /* 1. prior moments (the state is empty at step 1), the update, new FP32 moments */
    if (step > 1) {
        for (size_t b = 0; b < nb; ++b) {
            size_t i0 = b * B, len = i0 + B < n ? B : n - i0;
            float lev[256];
            if (compress_v) oracle_q1_levels(v_ends[2 * b], v_ends[2 * b + 1], bits, lev);
            for (size_t i = i0; i < i0 + len; ++i)
                vprev[i] = compress_v ? lev[get_bits(v_index, i, bits)] : v_fp32[i];
        }
        for (size_t gi = 0; gi < ng; ++gi) {
            size_t i0 = gi * G, len = i0 + G < n ? G : n - i0;
            if (!compress_m) {
                for (size_t i = i0; i < i0 + len; ++i) mprev[i] = m_fp32[i];
                continue;
            }
            uint8_t codes[T_MAX_BLOCK];
            float q[T_MAX_BLOCK];
            for (size_t k = 0; k < len; ++k) codes[k] = (uint8_t)get_bits(m_codes, i0 + k, 2);
            oracle_ustate_decode(codes, len, m_means[gi], s_dec, q);
            for (size_t k = 0; k < len; ++k) {
                float den = sqrtf(vprev[i0 + k] / bc2p) + eps;
                mprev[i0 + k] = (q[k] * bc1p) * den;
            }
        }
    }
    for (size_t i = 0; i < n; ++i) {
        oracle_elem e = adamw_element(p[i], g[i], mprev[i], vprev[i], s);
        p[i] = e.p1;
        m1[i] = e.m1;
        v1[i] = e.v1;
        bad += (unsigned long long)elem_nonfinite(&e);
    }

    /* 2. second moment: 1Q per block, or FP32 */
    for (size_t b = 0; b < nb; ++b) {
        size_t i0 = b * B, len = i0 + B < n ? B : n - i0;
        if (!compress_v) {
            for (size_t i = i0; i < i0 + len; ++i) { v_fp32[i] = v1[i]; vp[i] = v1[i]; }
            continue;
        }
        uint8_t idx[T_MAX_BLOCK];
        oracle_q1_block(v1 + i0, len, bits, u1 + i0, idx, v_ends + 2 * b, vp + i0);
        for (size_t k = 0; k < len; ++k) put_bits(v_index, i0 + k, bits, idx[k]);
    }

    /* 3. first moment: UState per group of G values, or FP32 */
    for (size_t gi = 0; gi < ng; ++gi) {
        size_t i0 = gi * G, len = i0 + G < n ? G : n - i0;
        if (!compress_m) {
            for (size_t i = i0; i < i0 + len; ++i) m_fp32[i] = m1[i];
            continue;
        }
        float q[T_MAX_BLOCK];
        for (size_t k = 0; k < len; ++k) {
            float den = sqrtf(vp[i0 + k] / bc2) + eps;
            q[k] = (m1[i0 + k] / bc1) / den;
        }
        uint8_t codes[T_MAX_BLOCK];
        oracle_ustate_group(q, len, G, i0, s_enc, up + i0 / 2, codes, m_means + gi, r2 + i0);
        for (size_t k = 0; k < len; ++k) put_bits(m_codes, i0 + k, 2, codes[k]);
    }

    /* 4. scale rotation: s_dec <- s_enc, s_enc <- factor * residual RMS */
    if (compress_m) {
        double total = n ? pairwise_sum(r2, padded) : 0.0;
        double rms = n ? sqrt(total / (double)n) : 0.0;
        scal[0] = s_enc;
        scal[1] = (float)(factor * rms);
        scal[2] = 0.0f;
    }
    free(r2); free(m1); free(v1); free(vp); free(u1); free(up); free(mprev); free(vprev);
    return bad;
}

/* oracle_turbo_step with typed parameters (pdt) and gradients (gdt), as for
 * oracle_step_typed (TurboAdam package page, Verification: its tests run
 * fp16, bf16 and fp32 parameters).  The page's update reads the parameter
 * only in its own line ("The AdamW update remains AdamW"): the moments,
 * their compression and the scales never see it.  So the step widens both
 * inputs exactly, takes the FP32 step, and rounds only the new parameter
 * back to its type. */
unsigned long long oracle_turbo_step_typed(int pdt, int gdt, void* p, const void* g, size_t n, uint32_t tensor_id,
                                           int compress_m, int compress_v, int bits, int block, int group,
                                           uint32_t* m_codes, uint16_t* m_means, float* m_fp32,
                                           uint32_t* v_index, uint16_t* v_ends, float* v_fp32,
                                           float* scal, const float s[8], const float ts[3],
                                           double factor, unsigned long long seed, long long step) {
    size_t nn = n ? n : 1;
    float* pw = (float*)calloc(nn, sizeof(float));
    float* gw = (float*)calloc(nn, sizeof(float));
    for (size_t i = 0; i < n; ++i) {
        pw[i] = widen_at(pdt, p, i);
        gw[i] = widen_at(gdt, g, i);
    }
    unsigned long long bad = oracle_turbo_step(pw, gw, n, tensor_id, compress_m, compress_v, bits, block, group,
                                               m_codes, m_means, m_fp32, v_index, v_ends, v_fp32, scal, s, ts,
                                               factor, seed, step);
    for (size_t i = 0; i < n; ++i) narrow_at(pdt, p, i, pw[i]);
    free(pw);
    free(gw);
    return bad;
}
