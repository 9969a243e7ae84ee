// turbo.hpp -- gfx950 kernels of the TurboAdam compressed-state step.
//
// TurboAdam package page, "How it works" (UState, 1Q, "The AdamW update
// remains AdamW", "Fused CUDA path"): the update runs in FP32 on transient
// moments; the first moment persists as UState (normalised update units,
// 2-bit codes, one bf16 mean per 64 values, a lagged tensor scale) and the
// second as 1Q (a log grid per 128-value block between two fp16 endpoints).
// The page prints neither code nor constants for the grid, the code levels,
// the scale rule or the rounding hash; the readings implemented here:
//
//  * 1Q: index 0 is zero; index k >= 1 decodes to the exact power 2^x of
//    the k-th of L-1 evenly spaced points x from lo to hi (computed in
//    double), rounded once to binary32.  lo and hi are log2 of the block's smallest positive and
//    largest finite value, rounded to binary16 down and up.  A value goes to
//    the largest level at or below it, or the next one with probability
//    equal to its position between the two.
//  * UState: codes 0..3 are -1.5, -0.5, 0.5, 1.5 times the scale around the
//    group's bf16 mean; decoding subtracts the group's mean level, so the
//    decoded mean is the stored one.  Pairs of values use draws u and 1 - u.
//    The scale for the next encode is 1.1 x the RMS of this step's
//    residuals; decoding uses the scale the codes were written with.
//  * Draws: Philox4x32-10, the counter-based generator Triton builds in, so
//    one counter hash for a PyTorch and a Triton path.  Key: the seed's low
//    and high 32 bits; counter (value index / 4, step, tensor id, stream),
//    the entry point keeping index / 4 and step below 2^32.  Stream 0: the
//    top 24 bits of word k serve the 1Q rounding of value 4j + k.  Stream 1:
//    the top 24 bits of words 0 and 1 serve the two UState pairs.
//  * Sums (group means, the residual sum of squares) are perfect pairwise
//    trees in double over the values in index order, padded with zeros, so
//    their results do not depend on the launch.
//
// Work split: one wavefront per 256-value tile; lane l holds values 4l..4l+3,
// lanes 0-31 one 1Q block and lanes 32-63 the next, 16 lanes one UState
// group.  Every reduction is a butterfly of shuffles inside the wavefront;
// the per-block level tables sit in a wavefront-private slice of LDS, so no
// workgroup barrier is ever needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.hpp"
#include "pow2.hpp"

#pragma clang fp contract(off)

namespace pa {

constexpr int kTurboTile = 256;     // values per wavefront tile
constexpr int kTurboBlock = 128;    // 1Q block
constexpr int kTurboGroup = 64;     // UState mean group

struct TurboEntry {
  float* p;            // parameters: FP32, or 16-bit patterns (flags bits 2-3)
  const float* g;      // gradients: FP32, or 16-bit patterns (flags bits 4-5)
  uint8_t* m_codes;    // 2-bit codes, 4 per byte (compress_m)
  uint16_t* m_means;   // bf16 per 64 (compress_m)
  float* m_fp32;       // (!compress_m)
  uint8_t* v_index;    // bits per value, little-endian (compress_v)
  uint16_t* v_ends;    // fp16 lo, hi per 128 (compress_v)
  float* v_fp32;       // (!compress_v)
  float* scal;         // s_dec, s_enc, acc (compress_m)
  long long n;
  long long tile0;     // first global tile of this tensor
  long long ws0;       // first workspace slot (one double per tile)
  unsigned long long seed;   // the call's rounding seed (kept here so the
                             // Philox key schedule is formed per tile, not
                             // hoisted into scalar registers for the launch)
  uint32_t tensor_id;
  int flags;           // bit 0: compress_m, bit 1: compress_v, bits 2-3 and
                       // 4-5: parameter and gradient type (kF32, kBF16, kF16)
};

// Four consecutive parameters or gradients from i0 (a multiple of four),
// widened to FP32: one vector load for a whole quad, else one load per
// valid value (0 for the others).  The type is uniform across the
// wavefront, so the branch is a scalar one.
template <int T>
__device__ __forceinline__ void load4_as(const void* base, long long i0, bool full, const bool valid[4],
                                         float out[4]) {
  using E = Elem<T>;
  const typename E::scalar* b = static_cast<const typename E::scalar*>(base);
  if (full) {
    const typename E::vec4 v = stream_load(reinterpret_cast<const typename E::vec4*>(b + i0));
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = E::widen(v[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = valid[k] ? E::widen(b[i0 + k]) : 0.0f;
  }
}

__device__ __forceinline__ void load4_typed(int t, const void* base, long long i0, bool full, const bool valid[4],
                                            float out[4]) {
  if (t == kBF16) load4_as<kBF16>(base, i0, full, valid, out);
  else if (t == kF16) load4_as<kF16>(base, i0, full, valid, out);
  else load4_as<kF32>(base, i0, full, valid, out);
}

// The new parameters, rounded to their type (to nearest even).
template <int T>
__device__ __forceinline__ void store4_as(void* base, long long i0, bool full, const bool valid[4], const float x[4]) {
  using E = Elem<T>;
  typename E::scalar* b = static_cast<typename E::scalar*>(base);
  if (full) {
    typename E::vec4 v;
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = E::narrow(x[k]);
    stream_store(reinterpret_cast<typename E::vec4*>(b + i0), v);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (valid[k]) b[i0 + k] = E::narrow(x[k]);
  }
}

__device__ __forceinline__ void store4_typed(int t, void* base, long long i0, bool full, const bool valid[4],
                                             const float x[4]) {
  if (t == kBF16) store4_as<kBF16>(base, i0, full, valid, x);
  else if (t == kF16) store4_as<kF16>(base, i0, full, valid, x);
  else store4_as<kF32>(base, i0, full, valid, x);
}


struct TurboScalars {
  float bc1, bc1p, bc2p, pad_;
  double inv_bc1, inv_bc2p;       // 1/bc1 and 1/bc2_{t-1} rounded to double
  unsigned long long seed;
  long long step;
};

// Ten rounds of the Philox-4x32 bijection: words 0 and 2 times the two round
// multipliers; each product's high half xors the other odd word and a key
// word; the key steps by the two Weyl constants between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1, uint32_t w[4]) {
  uint32_t x0 = c0, x1 = c1, x2 = c2, x3 = c3;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0, p1 = (uint64_t)0xCD9E8D57u * x2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0, n2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
    x0 = n0;
    x1 = (uint32_t)p1;
    x2 = n2;
    x3 = (uint32_t)p0;
  }
  w[0] = x0;
  w[1] = x1;
  w[2] = x2;
  w[3] = x3;
}

// x / d for a uniform binary32 d with rd = RN64(1/d): the correctly rounded
// quotient (see div_bc2 in kernels.hpp for the argument).
__device__ __forceinline__ float div_uniform(float x, double rd) { return (float)((double)x * rd); }

// binary16 bit pattern of x rounded toward -Inf (up = false) or +Inf (up =
// true); |x| is far inside the binary16 range here (a log2 of a float).
__device__ __forceinline__ uint32_t f16_directed_dev(double x, bool up) {
  const bool neg = x < 0.0;
  const double a = neg ? -x : x;
  // round the magnitude toward zero when the direction points to zero
  const bool mag_up = neg ? !up : up;
  uint32_t bits;
  if (a < 0x1p-14) {                                    // subnormal range: multiples of 2^-24
    const double q = a * 0x1p24;
    const double r = mag_up ? __builtin_ceil(q) : __builtin_floor(q);
    bits = (uint32_t)r;                                 // r <= 1024: 1024 is the smallest normal
  } else {
    int e;
    const double f = __builtin_frexp(a, &e);           // a = f * 2^e, f in [0.5, 1)
    double q = __builtin_ldexp(f, 11);                  // in [1024, 2048)
    q = mag_up ? __builtin_ceil(q) : __builtin_floor(q);
    int be = e - 1 + 15;                                // biased exponent of 2^(e-1)
    if (q >= 2048.0) {
      q = 1024.0;
      be += 1;
    }
    bits = ((uint32_t)be << 10) | ((uint32_t)q - 1024u);
  }
  if (bits == 0) return 0u;
  return (neg ? 0x8000u : 0u) | bits;
}

__device__ __forceinline__ double f16_to_double(uint32_t h) { return (double)f16_decode(h); }

// One binary16 step up or down in value from pattern h (not +-Inf, not -0);
// a zero result is +0.  The magnitude grows when the direction and the sign
// agree; a step down from +0 lands on the smallest negative subnormal.
// Written as selects: `up` differs between lanes.
__device__ __forceinline__ uint32_t f16_step(uint32_t h, bool up) {
  const uint32_t grow = (up ? 1u : 0u) ^ (h >> 15);
  uint32_t r = h + (grow ? 1u : 0xFFFFFFFFu);
  r = ((h & 0x7FFFu) == 0u && !up) ? 0x8001u : r;
  return r == 0x8000u ? 0u : r;
}

// x rounded to binary16 toward -Inf (up = false) or +Inf (up = true), for
// |x| far inside the binary16 range: the nearest-even conversion, moved one
// step when it landed on the wrong side of x; a zero result is +0 (as
// f16_directed_dev).
__device__ __forceinline__ uint32_t f16_directed_f32(float x, bool up) {
  uint32_t h = f16_encode(x);
  h = h == 0x8000u ? 0u : h;
  const float hv = f16_decode(h);
  const bool wrong = (hv < x && up) || (hv > x && !up);
  const uint32_t stepped = f16_step(h, up);
  return wrong ? stepped : h;
}

// The exact endpoint through the double log2 (out of line, as build_levels).
__device__ __attribute__((noinline)) uint32_t log2_directed16_exact(float v, bool up) {
  return f16_directed_dev(log2((double)v), up);
}

// A 1Q endpoint: log2(v) rounded to binary16 down (up = false) or up, for a
// positive finite v.  The hardware log2 (v below 2^-64 scaled by 2^64 first)
// is within one binary32 ulp of log2(v) for every positive binary32, which
// was measured on gfx950 against the double log2 over all of them.  So
// log2(v) lies in [y - d, y + d] with d = |y| 2^-21 + 2^-60 (four times that
// bound, which also covers the rounding of y - 64 and of the interval ends),
// and when both ends round to the same binary16 value, so does log2(v), and
// so does any double within 2^-52 of it.  Otherwise (a binary16 point inside
// the interval: about one value in a thousand, and every power of two) the
// double log2 decides, on the lanes that are `active`.
__device__ __forceinline__ uint32_t log2_directed16(float v, bool up, bool active) {
  const bool small = v < 0x1p-64f;
  float y = __builtin_amdgcn_logf(small ? v * 0x1p64f : v);
  y = small ? y - 64.0f : y;
  const float d = __builtin_fabsf(y) * 0x1p-21f + 0x1p-60f;
  const uint32_t a = f16_directed_f32(y - d, up), b = f16_directed_f32(y + d, up);
  if (active && a != b) return log2_directed16_exact(v, up);
  return a;
}

// The exponent of level k >= 1 of a 1Q block, in double.
__device__ __forceinline__ double q1_level_x(double lo, double hi, int k, int L) {
  return lo + ((hi - lo) * (double)(k - 1)) / (double)(L - 2);
}

// The double-double decision, out of line for the self-test export.
__device__ __attribute__((noinline)) float pow2_rn32_slow(double x) { return pow2_rn32_dd(x); }

// Level k >= 1 of a 1Q block is the exact 2^x rounded once to binary32.  The
// device exp2 is within one double ulp (2^-52 relative) of 2^x; when every
// value within 2^-48 of its result rounds to the same binary32 value, so
// does 2^x (the products below are monotone and off by at most 2^-53), and
// this returns true with the level in *out.  Otherwise (2^x near a binary32
// midpoint: about one level in 2^23) the double-double evaluation decides.
__device__ __forceinline__ bool q1_level_fast(double x, float* out) {
  const double y = exp2(x);
  const float a = (float)(y * (1.0 - 0x1p-48)), b = (float)(y * (1.0 + 0x1p-48));
  *out = a;
  return a == b;
}

// A pointer into LDS.  The out-of-line table builders take their tables as
// such, so that they write them with 32-bit LDS addresses (a plain pointer
// would arrive as a 64-bit flat address).
typedef __attribute__((address_space(3))) float lds_float;

// The table builders and the exact log2 below are called out of line on
// purpose: inlined, the double-precision polynomial coefficients were
// hoisted out of the tile loop into about 40 vector registers held for the
// whole kernel, which cut occupancy from 7 to 4 wavefronts per SIMD; a call
// per table costs a few instructions against thousands per tile.  Levels
// left undecided are redone afterwards in one rolled loop, so that the
// double-double code appears once and its registers stay few.
//
// 6- and 8-bit tables (L = 64, 256): lane j of a half builds levels j,
// j + 32, ..., below L (lane 0 starts at 32; level 0 is 0).  The levels form a geometric
// grid, so after its first level y = exp2(x_k0) the lane multiplies by
// C = exp2(32 d), d = RN64((hi - lo) / (L - 2)), instead of calling exp2
// for each level.  Level k is the exact power 2^x_k of its own double x_k
// (q1_level_x).  With |lo|, |hi| <= 256 the product is within 2^-42
// (relative) of it: the exponents differ by the roundings in x_k, x_k0 and
// 32 m d (below 2^-42 absolute together, scaled by ln 2 in the value), and
// the two exp2 and up to seven products add below 2^-48.  So when every
// value within 2^-40 of the product rounds to the same binary32 value, so
// does 2^x_k; otherwise (about one level in 2^15) the double-double
// evaluation decides, as it does for every level of endpoints outside that
// range (no block has them: its endpoints lie in [-149, 128]).
template <int BITS>
__device__ __attribute__((noinline)) void build_levels(lds_float* lev, uint32_t ends, int lane_in_half) {
  constexpr int L = 1 << BITS;
  static_assert(L == 64 || L == 256, "32 lanes, L / 32 levels each");
  const double lo = f16_to_double(ends & 0xFFFFu), hi = f16_to_double(ends >> 16);
  const int k0 = lane_in_half == 0 ? 32 : lane_in_half;
  if (lane_in_half == 0) lev[0] = 0.0f;
  double y = exp2(q1_level_x(lo, hi, k0, L));
  const double c = exp2(32.0 * ((hi - lo) / (double)(L - 2)));
  const bool in_range = __builtin_fabs(lo) <= 256.0 && __builtin_fabs(hi) <= 256.0;
  uint32_t undecided = 0;   // bit j: level k0 + 32 j
#pragma unroll
  for (int j = 0; j < L / 32; ++j) {
    const int k = k0 + 32 * j;
    if (k >= L) break;
    const float a = (float)(y * (1.0 - 0x1p-40)), b = (float)(y * (1.0 + 0x1p-40));
    if (!in_range || a != b) undecided |= 1u << j;
    lev[k] = a;
    y *= c;
  }
  while (undecided) {
    const int j = __builtin_ctz(undecided);
    undecided &= undecided - 1;
    const int k = k0 + 32 * j;
    lev[k] = pow2_rn32_dd(q1_level_x(lo, hi, k, L));
  }
}

// Offset, within a half-wavefront's LDS slice, of the decode table when
// indices have at most 4 bits (the encode table sits at 0).
constexpr int kDecodeTable = 128;

// Tables for indices of at most 4 bits (L <= 16 levels): entry k is the pair
// (level k, sqrt(level k / bc) + eps), the second being the denominator the
// UState codec takes from the persisted second moment (bc the bias
// correction of the step that persisted it, r = RN64(1/bc)).  A block's
// persisted values are its levels, so each denominator is computed once per
// level instead of once per value; it is the same correctly rounded
// function of the same input either way.  Lanes 0..L-1 of each half build
// the table of `ends` at lev.
template <int BITS>
__device__ __attribute__((noinline)) void build_tables(lds_float* lev, uint32_t ends, double r, float eps,
                                                       int lane_in_half) {
  constexpr int L = 1 << BITS;
  static_assert(L <= 16, "one level per lane");
  const int k = lane_in_half;
  if (k >= L) return;
  float a = 0.0f;
  if (k > 0) {
    const double x = q1_level_x(f16_to_double(ends & 0xFFFFu), f16_to_double(ends >> 16), k, L);
    if (!q1_level_fast(x, &a)) a = pow2_rn32_dd(x);
  }
  lds_float* dst = lev + 2 * k;
  dst[0] = a;
  dst[1] = sqrt_rn(div_uniform(a, r)) + eps;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int W>
__device__ __forceinline__ double butterfly_sum(double x) {
#pragma unroll
  for (int off = 1; off < W; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int W>
__device__ __forceinline__ int butterfly_isum(int x) {
#pragma unroll
  for (int off = 1; off < W; off <<= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int W>
__device__ __forceinline__ float butterfly_min(float x) {
#pragma unroll
  for (int off = 1; off < W; off <<= 1) x = fminf(x, __shfl_xor(x, off, 64));
  return x;
}

template <int W>
__device__ __forceinline__ float butterfly_max(float x) {
#pragma unroll
  for (int off = 1; off < W; off <<= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ float ustate_level(uint32_t c) { return (float)(int)(2 * c) * 0.5f - 1.5f; }

template <int BITS>
__device__ __forceinline__ uint32_t load_index4(const uint8_t* base, long long lane_word) {
  if constexpr (BITS == 2) return base[lane_word];
  else if constexpr (BITS == 4) return reinterpret_cast<const uint16_t*>(base)[lane_word];
  else return reinterpret_cast<const uint32_t*>(base)[lane_word];
}

// The 4 * BITS-bit field of values i0..i0+3 of a dense little-endian index
// stream of n values.  Widths that straddle 32-bit words (3, 6) read the
// word holding the field's first bit and, when the field's valid bits reach
// it, the next one.
template <int BITS>
__device__ __forceinline__ uint32_t load_field(const uint8_t* base, long long i0, long long n) {
  if constexpr (BITS == 2 || BITS == 4 || BITS == 8) {
    return load_index4<BITS>(base, i0 >> 2);
  } else {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(base);
    const long long b0 = i0 * BITS, b_end = (i0 + 4 < n ? i0 + 4 : n) * BITS;
    const long long w0 = b0 >> 5;
    unsigned long long both = w[w0];
    if (b_end > (w0 + 1) * 32) both |= (unsigned long long)w[w0 + 1] << 32;
    return (uint32_t)(both >> (b0 & 31)) & ((1u << (4 * BITS)) - 1u);
  }
}

// For widths that straddle words (3, 6): the 128 indices of the
// half-wavefront's block as its 4 * BITS dense words, each gathered by
// shuffles from the (at most 32 / (4 * BITS) + 2) lane fields it overlaps,
// and stored by the half's first 4 * BITS lanes (words past the stream's
// end are not written).  Called by every lane of the wavefront.
template <int BITS>
__device__ __forceinline__ void store_fields_dense(uint8_t* base, long long blk, long long n, uint32_t field, int half,
                                                   int lane_in_half) {
  constexpr int F = 4 * BITS;                       // field bits per lane, and words per block
  constexpr int Q = 32 / F + 2;
  const int w = lane_in_half;
  const int first = (32 * w) / F;
  uint32_t word = 0;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int src = first + q;
    const uint32_t f = (uint32_t)__shfl((int)field, (half << 5) + (src < 32 ? src : 31), 64);
    const int off = src * F - 32 * w;               // the field's first bit, relative to the word
    if (src < 32 && off < 32 && off + F > 0) word |= off >= 0 ? f << off : f >> -off;
  }
  const long long gw = blk * F + w, nwords = (n * BITS + 31) >> 5;
  if (w < F && gw < nwords) reinterpret_cast<uint32_t*>(base)[gw] = word;
}

template <int BITS>
__device__ __forceinline__ void store_index4(uint8_t* base, long long lane_word, uint32_t v) {
  if constexpr (BITS == 2) base[lane_word] = (uint8_t)v;
  else if constexpr (BITS == 4) reinterpret_cast<uint16_t*>(base)[lane_word] = (uint16_t)v;
  else reinterpret_cast<uint32_t*>(base)[lane_word] = v;
}

// One 256-value tile of one tensor, by one wavefront.
// The entry is read through a pointer at each use: held whole, its fields
// crowd the scalar registers and spill.
// FULL: the tile lies wholly inside its tensor, so every validity test below
// folds away (one instantiation per case; the partial one runs only on a
// tensor's last tile).  TYPED: parameters and gradients of the entry's
// element types (else FP32).
template <int BITS, bool FULL, bool TYPED>
__device__ __forceinline__ void turbo_tile(const TurboEntry* __restrict__ ep, long long tile, const Scalars& s,
                                           const TurboScalars& ts, float* lev_half, double* ws, uint32_t& bad) {
  const TurboEntry& e = *ep;
  constexpr int L = 1 << BITS;
  const int lane = threadIdx.x & 63;
  const int half = lane >> 5, lane_in_half = lane & 31;
  const bool cm = e.flags & 1, cv = e.flags & 2;
  const long long base = tile * kTurboTile;
  const long long i0 = base + 4 * lane;                 // this lane's first value
  const long long n = e.n;
  const bool full = FULL;
  bool valid[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) valid[k] = FULL || i0 + k < n;
  const long long blk = (base >> 7) + half;              // 1Q block of this lane
  const bool blk_exists = FULL || blk * kTurboBlock < n;
  const long long grp = i0 >> 6;                         // UState group of this lane
  const long long glen_ll = n - (grp << 6);
  const int glen = (FULL || glen_ll >= kTurboGroup) ? kTurboGroup : (int)glen_ll;

  // ---- loads
  float p[4], g[4], mprev[4] = {0.f, 0.f, 0.f, 0.f}, vprev[4] = {0.f, 0.f, 0.f, 0.f};
  // The UState decode denominators sqrt(vprev / bc2_{t-1}) + eps, from the
  // decode table (indices of at most 4 bits, 1Q second moment).
  constexpr bool kDenTables = BITS <= 4;
  float dprev[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (TYPED) {
    load4_typed((e.flags >> 2) & 3, e.p, i0, full, valid, p);
    load4_typed((e.flags >> 4) & 3, e.g, i0, full, valid, g);
  } else if (full) {
    const f32x4 pv = stream_load(reinterpret_cast<const f32x4*>(e.p + i0));
    const f32x4 gv = stream_load(reinterpret_cast<const f32x4*>(e.g + i0));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      p[k] = pv[k];
      g[k] = gv[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      p[k] = valid[k] ? e.p[i0 + k] : 0.0f;
      g[k] = valid[k] ? e.g[i0 + k] : 0.0f;
    }
  }
  // The state words of the prior moments, loaded together with p and g so
  // that one memory latency covers them all.
  uint32_t idx4 = 0, mcodes = 0, mean16 = 0;
  if (ts.step > 1 && valid[0]) {
    if (cv) idx4 = load_field<BITS>(e.v_index, i0, n);
    if (cm) {
      mcodes = e.m_codes[i0 >> 2];
      mean16 = e.m_means[grp];
    }
  }
  const float s_dec = cm ? e.scal[0] : 0.0f, s_enc = cm ? e.scal[1] : 0.0f;

  // ---- decode the prior moments (the state is empty at step 1)
  if (ts.step > 1) {
    if (cv) {
      float* dec = BITS <= 4 ? lev_half + kDecodeTable : lev_half;
      {
        const uint32_t ends = blk_exists ? *reinterpret_cast<const uint32_t*>(e.v_ends + 2 * blk) : 0u;
        if constexpr (BITS <= 4)
          build_tables<BITS>((lds_float*)dec, ends, ts.inv_bc2p, s.eps, lane_in_half);
        else
          build_levels<BITS>((lds_float*)dec, ends, lane_in_half);
        wave_lds_sync();
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t ix = (idx4 >> (BITS * k)) & (L - 1);
        if constexpr (BITS <= 4) {
          const float2 entry = reinterpret_cast<const float2*>(dec)[ix];
          vprev[k] = valid[k] ? entry.x : 0.0f;
          dprev[k] = entry.y;
        } else {
          vprev[k] = valid[k] ? dec[ix] : 0.0f;
        }
      }
      wave_lds_sync();
    } else if (full) {
      const f32x4 vv = *reinterpret_cast<const f32x4*>(e.v_fp32 + i0);
#pragma unroll
      for (int k = 0; k < 4; ++k) vprev[k] = vv[k];
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) vprev[k] = valid[k] ? e.v_fp32[i0 + k] : 0.0f;
    }
    if (cm) {
      int s2 = 0;                                        // sum of 2 * level over this lane's values
#pragma unroll
      for (int k = 0; k < 4; ++k) s2 += valid[k] ? (int)(2 * ((mcodes >> (2 * k)) & 3u)) - 3 : 0;
      s2 = butterfly_isum<16>(s2);
      const float lbar = (float)((double)s2 * 0.5 / (double)glen);
      const float mean = __uint_as_float(mean16 << 16);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float q = mean + s_dec * (ustate_level((mcodes >> (2 * k)) & 3u) - lbar);
        const float den = (kDenTables && cv) ? dprev[k] : sqrt_rn(div_uniform(vprev[k], ts.inv_bc2p)) + s.eps;
        mprev[k] = valid[k] ? (q * ts.bc1p) * den : 0.0f;
      }
    } else if (full) {
      const f32x4 mv = *reinterpret_cast<const f32x4*>(e.m_fp32 + i0);
#pragma unroll
      for (int k = 0; k < 4; ++k) mprev[k] = mv[k];
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) mprev[k] = valid[k] ? e.m_fp32[i0 + k] : 0.0f;
    }
  }

  // ---- the update with the FP32 moments
  float m1[4], v1[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float p1;
    adamw(p[k], g[k] * s.gmul, s.beta1 * mprev[k], vprev[k], s, p1, m1[k], v1[k]);
    if (valid[k]) bad += nonfinite3(p1, m1[k], v1[k]);
    p[k] = p1;
  }
  if constexpr (TYPED) {
    store4_typed((e.flags >> 2) & 3, e.p, i0, full, valid, p);
  } else if (full) {
    f32x4 pv;
#pragma unroll
    for (int k = 0; k < 4; ++k) pv[k] = p[k];
    stream_store(reinterpret_cast<f32x4*>(e.p + i0), pv);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (valid[k]) e.p[i0 + k] = p[k];
  }

  // ---- draws of this lane's four values
  const uint32_t ctr = (uint32_t)(i0 >> 2), stp = (uint32_t)ts.step, tid = e.tensor_id;
  const uint32_t sk0 = (uint32_t)e.seed, sk1 = (uint32_t)(e.seed >> 32);

  // ---- second moment: 1Q per block, or FP32
  // vq: with a 1Q table of at most 4-bit indices, the UState encode
  // denominator sqrt(v_persisted / bc2) + eps looked up with each value's
  // index; otherwise the persisted second moment it is computed from.
  float vq[4];
  if (cv) {
    uint32_t w[4];
    philox4x32_10(ctr, stp, tid, 0u, sk0, sk1, w);
    float lo_c = __builtin_inff(), hi_c = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v = v1[k];
      const bool pos = valid[k] && v > 0.0f && __builtin_isfinite(v);
      lo_c = pos ? fminf(lo_c, v) : lo_c;
      hi_c = pos ? fmaxf(hi_c, v) : hi_c;
    }
    const float vmin = butterfly_min<32>(lo_c), vmax = butterfly_max<32>(hi_c);
    // Endpoints: lanes 0 and 1 of each half round log2 of the minimum down
    // and of the maximum up (one pass for both), then broadcast.
    const bool ends_lane = lane_in_half < 2 && vmax > 0.0f;
    const uint32_t e16 = log2_directed16(lane_in_half == 0 ? vmin : vmax, lane_in_half != 0, ends_lane);
    const int src = half << 5;
    const uint32_t lo16 = (uint32_t)__shfl((int)e16, src, 64), hi16 = (uint32_t)__shfl((int)e16, src + 1, 64);
    const uint32_t ends = vmax > 0.0f ? (lo16 | (hi16 << 16)) : 0u;
    if constexpr (BITS <= 4)
      build_tables<BITS>((lds_float*)lev_half, ends, s.inv_bc2, s.eps, lane_in_half);
    else
      build_levels<BITS>((lds_float*)lev_half, ends, lane_in_half);
    // level k of the encode table
    constexpr int kStride = BITS <= 4 ? 2 : 1;
    // 8-bit tables: the grid is uniform in log2 between the endpoints, so
    // a value's bracket is first estimated from the hardware log2.
    float est_lo = 0.0f, est_scale = 0.0f;
    if constexpr (BITS == 8) {
      est_lo = f16_decode(ends & 0xFFFFu);
      est_scale = (float)(L - 2) / (f16_decode(ends >> 16) - est_lo);
    }
    wave_lds_sync();
    uint32_t idx4 = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v = v1[k];
      // The largest level k >= 1 at or below v (1 when none is): by binary
      // lifting over the sorted table (exact for any non-decreasing table,
      // no data-dependent branch).  8-bit tables try the log2 estimate
      // first and keep it when the table confirms it; values that are not
      // positive and finite get their index from the special cases below,
      // so their estimate is kept unchecked.
      int kk = 1;
      bool found = false;
      if constexpr (BITS == 8) {
        float t = (__builtin_amdgcn_logf(v) - est_lo) * est_scale + 1.0f;
        t = t >= 1.0f ? t : 1.0f;   // also NaN
        t = t <= (float)(L - 1) ? t : (float)(L - 1);
        kk = (int)t;
        const bool special = !(v > 0.0f) || __builtin_isinf(v);
        found = special || (lev_half[kk] <= v && (kk == L - 1 || lev_half[kk < L - 1 ? kk + 1 : kk] > v));
        if (!found) kk = 1;
      }
      if (!found) {
#pragma unroll
        for (int step = L >> 1; step >= 1; step >>= 1) {
          const int c = kk + step;
          kk = (c < L && lev_half[kStride * (c < L ? c : L - 1)] <= v) ? c : kk;
        }
      }
      const float lk = lev_half[kStride * kk], lk1 = lev_half[kStride * (kk < L - 1 ? kk + 1 : kk)];
      const float f = __fdiv_rn(v - lk, lk1 - lk);
      const float u = (float)(w[k] >> 8) * 0x1p-24f;
      const uint32_t up = (kk < L - 1 && v > lk && u < f) ? 1u : 0u;
      uint32_t idx = (uint32_t)kk + up;
      idx = __builtin_isinf(v) ? (uint32_t)(L - 1) : idx;
      idx = v > 0.0f ? idx : 0u;                            // zero, negative, NaN
      if constexpr (BITS <= 4) vq[k] = reinterpret_cast<const float2*>(lev_half)[idx].y;
      else vq[k] = lev_half[idx];
      idx4 |= valid[k] ? idx << (BITS * k) : 0u;           // padding past the end stays zero
    }
    wave_lds_sync();
    if constexpr (BITS == 3 || BITS == 6)
      store_fields_dense<BITS>(e.v_index, blk, n, idx4, half, lane_in_half);
    else if (valid[0])
      store_index4<BITS>(e.v_index, i0 >> 2, idx4);
    if (lane_in_half == 0 && blk_exists) *reinterpret_cast<uint32_t*>(e.v_ends + 2 * blk) = ends;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) vq[k] = v1[k];
    if (full) {
      f32x4 vv;
#pragma unroll
      for (int k = 0; k < 4; ++k) vv[k] = v1[k];
      *reinterpret_cast<f32x4*>(e.v_fp32 + i0) = vv;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (valid[k]) e.v_fp32[i0 + k] = v1[k];
    }
  }

  // ---- first moment: UState per group, or FP32
  if (cm) {
    uint32_t w[4];
    philox4x32_10(ctr, stp, tid, 1u, sk0, sk1, w);
    float q[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float den = (kDenTables && cv) ? vq[k] : sqrt_rn(div_bc2(vq[k], s)) + s.eps;
      q[k] = valid[k] ? __fdiv_rn(div_uniform(m1[k], ts.inv_bc1), den) : 0.0f;
    }
    const double gsum = butterfly_sum<16>(((double)q[0] + (double)q[1]) + ((double)q[2] + (double)q[3]));
    const uint32_t mean16 = bf16_encode((float)(gsum / (double)glen));
    const float mean = __uint_as_float(mean16 << 16);
    uint32_t codes = 0;
    double r2[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float r = q[k] - mean;
      r2[k] = valid[k] ? (double)r * (double)r : 0.0;
      float x = s_enc > 0.0f ? __fdiv_rn(r, s_enc) : 0.0f;
      x = x > 1.5f ? 1.5f : x;
      x = x < -1.5f ? -1.5f : x;
      float u = (float)(w[k >> 1] >> 8) * 0x1p-24f;
      if (k & 1) u = 1.0f - u;
      const uint32_t kk = (uint32_t)(x >= -0.5f) + (uint32_t)(x >= 0.5f);
      uint32_t code = kk;
      if (x >= 1.5f) code = 3;
      else if (u < x - ustate_level(kk)) code = kk + 1;
      codes |= valid[k] ? code << (2 * k) : 0u;
    }
    if (valid[0]) e.m_codes[i0 >> 2] = (uint8_t)codes;
    if ((lane & 15) == 0 && valid[0]) e.m_means[grp] = (uint16_t)mean16;
    const double tsum = butterfly_sum<64>((r2[0] + r2[1]) + (r2[2] + r2[3]));
    if (lane == 0) ws[e.ws0 + tile] = tsum;
  } else if (full) {
    f32x4 mv;
#pragma unroll
    for (int k = 0; k < 4; ++k) mv[k] = m1[k];
    *reinterpret_cast<f32x4*>(e.m_fp32 + i0) = mv;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (valid[k]) e.m_fp32[i0 + k] = m1[k];
  }
}

// One tile per wavefront, in dispatch order: wavefront w of the launch takes
// tile tile_base + w, so the tiles in flight form one compact window that
// advances through the list (faster than a persistent grid striding over
// the tiles: the hardware starts each new wavefront as one finishes, and
// its loads overlap the work of the wavefronts around it).  The tile's
// tensor is found by a bisection over the table's first tiles.
template <int BITS, bool COUNT, bool TYPED>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BITS <= 4 ? 7 : 6)))
turbo_list(const TurboEntry* __restrict__ table, int count, long long total_tiles, long long tile_base, Scalars s,
           TurboScalars ts, double* ws, unsigned long long* nonfinite) {
  __shared__ float lev[kThreads / 64][2][256];
  if (!resolve_inputs(s)) return;
  // The wavefront index is uniform across the wavefront; saying so lets the
  // compiler keep the tile, the table search and every field of the entry
  // in scalar registers (scalar loads, the Philox key schedule on the
  // scalar unit) instead of repeating them in every lane.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), half = (threadIdx.x >> 5) & 1;
  const long long tile = tile_base + (long long)blockIdx.x * (kThreads / 64) + wave;
  uint32_t bad = 0;
  if (tile < total_tiles) {
    int lo = 0, hi = count - 1;                      // the last entry with tile0 <= tile
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (table[mid].tile0 <= tile) lo = mid;
      else hi = mid - 1;
    }
    const long long local = tile - table[lo].tile0;
    if ((local + 1) * kTurboTile <= table[lo].n)
      turbo_tile<BITS, true, TYPED>(table + lo, local, s, ts, lev[wave][half], ws, bad);
    else
      turbo_tile<BITS, false, TYPED>(table + lo, local, s, ts, lev[wave][half], ws, bad);
  }
  if constexpr (COUNT) flush_count(bad, nonfinite);
}

// ---------------------------------------------------------------------------
// The general step: every layout of the page's fused path (1Q blocks of 32
// to 1024 values, UState groups of a power of two dividing the block, 2, 3,
// 4, 6 or 8 index bits), with the arithmetic and draws of turbo_tile.  One
// 256-thread workgroup per 1024-value tile of one tensor, so a tile holds
// whole blocks and whole groups; thread t holds values 4t..4t+3 of its
// tile.  When a block has at least as many values as levels (L <= B), the
// lanes of each block build its decode and encode tables in LDS, each entry
// the pair (level, UState denominator) as in build_tables; otherwise the
// levels are computed per value (the same exact power), since per-block
// tables would cost more levels than the block has values.  Reductions over a block or a
// group are xor butterflies over its lanes; segments wider than a
// wavefront finish through LDS as further levels of the same tree.  The
// residual partial sums go to turbo_list's workspace slots (one per 256
// values), so turbo_chunks and turbo_reduce complete them unchanged.
constexpr int kGenTile = 1024;

// x reduced over aligned segments of `seg` lanes of the workgroup (a power
// of two from 1 to 256), every lane receiving its segment's result.  Every
// thread must call it (segments above 64 lanes synchronise the workgroup);
// slot is four LDS entries.
template <class T, class Op>
__device__ __forceinline__ T seg_reduce(T x, int seg, Op op, T* slot) {
  const int inwave = seg < 64 ? seg : 64;
  for (int off = 1; off < inwave; off <<= 1) x = op(x, __shfl_xor(x, off, 64));
  if (seg > 64) {
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) slot[wave] = x;
    __syncthreads();
    const int first = wave & ~(seg / 64 - 1);
    x = seg == 128 ? op(slot[first], slot[first + 1])
                   : op(op(slot[first], slot[first + 1]), op(slot[first + 2], slot[first + 3]));
    __syncthreads();   // the slots are reused by the next call
  }
  return x;
}

// Level k >= 1 of a block whose endpoints decode to lo and hi.
__device__ __forceinline__ float q1_level(double lo, double hi, int k, int L) {
  const double x = q1_level_x(lo, hi, k, L);
  float a;
  if (!q1_level_fast(x, &a)) a = pow2_rn32_slow(x);
  return a;
}

// One 1024-value tile of the general step (the workgroup's), its LDS
// passed in.  FULL: the tile lies wholly inside its tensor, so every
// validity test folds away (the partial copy runs on a tensor's last tile).
// TYPED as for turbo_tile.
template <int BITS, bool FULL, bool TYPED>
__device__ __forceinline__ void general_tile(const TurboEntry* __restrict__ ep, long long local, const Scalars& s,
                                             const TurboScalars& ts, int blog, int glog, double* ws, uint32_t& bad,
                                             uint32_t* words, float2* tabs, uint32_t* eslot, float* fslot,
                                             double* dslot, int* islot) {
  constexpr int L = 1 << BITS;
  constexpr int kWords = kGenTile * BITS / 32;       // index words of a tile
  const TurboEntry& e = *ep;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long long i0 = local * kGenTile + 4 * tid;  // this thread's first value
  const long long n = e.n;
  const bool cm = e.flags & 1, cv = e.flags & 2;
  const int B = 1 << blog, G = 1 << glog;
  const bool use_tab = L <= B;                       // uniform
  const int lb = tid & (B / 4 - 1);                  // lane within the block
  float2* const dec_tab = tabs + ((4 * tid) >> blog) * L;
  float2* const enc_tab = tabs + kGenTile + ((4 * tid) >> blog) * L;
  bool valid[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) valid[k] = FULL || i0 + k < n;
  const bool full = FULL || valid[3];
  for (int j = tid; j < kWords; j += kThreads) words[j] = 0u;

  // ---- loads
  float p[4], g[4], mprev[4] = {0.f, 0.f, 0.f, 0.f}, vprev[4] = {0.f, 0.f, 0.f, 0.f};
  float dprev[4] = {0.f, 0.f, 0.f, 0.f};              // UState decode denominators (tables)
  if constexpr (TYPED) {
    load4_typed((e.flags >> 2) & 3, e.p, i0, full, valid, p);
    load4_typed((e.flags >> 4) & 3, e.g, i0, full, valid, g);
  } else if (full) {
    const f32x4 pv = stream_load(reinterpret_cast<const f32x4*>(e.p + i0));
    const f32x4 gv = stream_load(reinterpret_cast<const f32x4*>(e.g + i0));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      p[k] = pv[k];
      g[k] = gv[k];
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      p[k] = valid[k] ? e.p[i0 + k] : 0.0f;
      g[k] = valid[k] ? e.g[i0 + k] : 0.0f;
    }
  }
  const long long blk = i0 >> blog;                  // 1Q block of this thread's values
  const bool blk_exists = FULL || (blk << blog) < n;
  const float s_dec = cm ? e.scal[0] : 0.0f, s_enc = cm ? e.scal[1] : 0.0f;

  // ---- decode the prior moments (the state is empty at step 1)
  if (ts.step > 1) {
    if (cv) {
      uint32_t field = 0, ends = 0;
      if (valid[0]) {
        // this thread's 4*BITS-bit field of the dense stream, read from the
        // words it touches (the second only when its own values reach it)
        const uint32_t* w32 = reinterpret_cast<const uint32_t*>(e.v_index);
        const long long bit0 = i0 * BITS, bit_end = (valid[3] ? i0 + 4 : n) * BITS;
        const long long w0 = bit0 >> 5;
        const int sh = (int)(bit0 & 31);
        unsigned long long both = w32[w0];
        if (bit_end > (w0 + 1) * 32) both |= (unsigned long long)w32[w0 + 1] << 32;
        field = (uint32_t)(both >> sh);
      }
      // every lane of an existing block needs its endpoints (table builders
      // past the tensor's end included)
      if (blk_exists) ends = reinterpret_cast<const uint32_t*>(e.v_ends)[blk];
      const double lo = f16_to_double(ends & 0xFFFFu), hi = f16_to_double(ends >> 16);
      if (use_tab) {
        for (int k = lb; k < L; k += B / 4) {
          const float a = k ? q1_level(lo, hi, k, L) : 0.0f;
          dec_tab[k] = make_float2(a, sqrt_rn(div_uniform(a, ts.inv_bc2p)) + s.eps);
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float2 t = dec_tab[(field >> (BITS * k)) & (uint32_t)(L - 1)];
          vprev[k] = valid[k] ? t.x : 0.0f;
          dprev[k] = t.y;
        }
      } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int ix = (int)((field >> (BITS * k)) & (uint32_t)(L - 1));
          vprev[k] = (valid[k] && ix > 0) ? q1_level(lo, hi, ix, L) : 0.0f;
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) vprev[k] = valid[k] ? e.v_fp32[i0 + k] : 0.0f;
    }
  }
  // The group mean level, summed as integers (2 x level), is exact in any
  // order; every thread takes part in the reduction (it may synchronise).
  uint32_t mcodes = 0;
  if (cm && ts.step > 1 && valid[0]) mcodes = e.m_codes[i0 >> 2];
  int s2[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) s2[k] = valid[k] ? (int)(2 * ((mcodes >> (2 * k)) & 3u)) - 3 : 0;
  if (G >= 4) {
    const int t = seg_reduce(s2[0] + s2[1] + s2[2] + s2[3], G / 4, [](int a, int b) { return a + b; }, islot);
    s2[0] = s2[1] = s2[2] = s2[3] = t;
  } else if (G == 2) {
    s2[0] = s2[1] = s2[0] + s2[1];
    s2[2] = s2[3] = s2[2] + s2[3];
  }
  if (ts.step > 1) {
    if (cm) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        if (!valid[k]) continue;
        const long long g0 = ((i0 + k) >> glog) << glog;
        const long long glen = n - g0 < G ? n - g0 : G;
        const float lbar = (float)((double)s2[k] * 0.5 / (double)glen);
        const float mean = __uint_as_float((uint32_t)e.m_means[(i0 + k) >> glog] << 16);
        const float q = mean + s_dec * (ustate_level((mcodes >> (2 * k)) & 3u) - lbar);
        const float den = (use_tab && cv) ? dprev[k] : sqrt_rn(div_uniform(vprev[k], ts.inv_bc2p)) + s.eps;
        mprev[k] = (q * ts.bc1p) * den;
      }
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) mprev[k] = valid[k] ? e.m_fp32[i0 + k] : 0.0f;
    }
  }

  // ---- the update with the FP32 moments
  float m1[4], v1[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float p1;
    adamw(p[k], g[k] * s.gmul, s.beta1 * mprev[k], vprev[k], s, p1, m1[k], v1[k]);
    if (valid[k]) bad += nonfinite3(p1, m1[k], v1[k]);
    p[k] = p1;
  }
  if constexpr (TYPED) {
    store4_typed((e.flags >> 2) & 3, e.p, i0, full, valid, p);
  } else if (full) {
    f32x4 pv;
#pragma unroll
    for (int k = 0; k < 4; ++k) pv[k] = p[k];
    stream_store(reinterpret_cast<f32x4*>(e.p + i0), pv);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (valid[k]) e.p[i0 + k] = p[k];
  }

  const uint32_t ctr = (uint32_t)(i0 >> 2), stp = (uint32_t)ts.step, tsr = e.tensor_id;
  const uint32_t sk0 = (uint32_t)e.seed, sk1 = (uint32_t)(e.seed >> 32);

  // ---- second moment: 1Q per block, or FP32
  float vq[4];       // the persisted second moment, or (tables) its UState denominator
  {
    float lo_c = __builtin_inff(), hi_c = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float v = v1[k];
      const bool pos = valid[k] && v > 0.0f && __builtin_isfinite(v);
      lo_c = pos ? fminf(lo_c, v) : lo_c;
      hi_c = pos ? fmaxf(hi_c, v) : hi_c;
    }
    // every thread takes part (the reductions may synchronise)
    const float vmin = seg_reduce(lo_c, B / 4, [](float a, float b) { return fminf(a, b); }, fslot);
    const float vmax = seg_reduce(hi_c, B / 4, [](float a, float b) { return fmaxf(a, b); }, fslot);
    if (cv) {
      uint32_t w[4];
      philox4x32_10(ctr, stp, tsr, 0u, sk0, sk1, w);
      // the block's first lane rounds log2 of the minimum down, its second
      // that of the maximum up; the block reads both back
      const bool any = vmax > 0.0f;
      const int bl = (4 * tid) >> blog;
      if (lb < 2) eslot[2 * bl + lb] = log2_directed16(lb ? vmax : vmin, lb != 0, any);
      __syncthreads();
      const uint32_t lo16 = eslot[2 * bl], hi16 = eslot[2 * bl + 1];
      const uint32_t ends = any ? (lo16 | (hi16 << 16)) : 0u;
      const double lo = f16_to_double(ends & 0xFFFFu), hi = f16_to_double(ends >> 16);
      const float est_lo = f16_decode(ends & 0xFFFFu);
      const float est_scale = (float)(L - 2) / (f16_decode(ends >> 16) - est_lo);
      if (use_tab) {
        for (int k = lb; k < L; k += B / 4) {
          const float a = k ? q1_level(lo, hi, k, L) : 0.0f;
          enc_tab[k] = make_float2(a, sqrt_rn(div_bc2(a, s)) + s.eps);
        }
      }
      __syncthreads();   // the encode tables built; the index words cleared
      uint32_t field = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float v = v1[k];
        uint32_t idx = 0;
        float keep = 0.0f;
        if (use_tab) {
          // the largest level k >= 1 at or below v (1 when none is), by
          // binary lifting over the sorted table
          int kk = 1;
#pragma unroll
          for (int step = L >> 1; step >= 1; step >>= 1) {
            const int c = kk + step;
            kk = (c < L && enc_tab[c < L ? c : L - 1].x <= v) ? c : kk;
          }
          const float lk = enc_tab[kk].x, lk1 = enc_tab[kk < L - 1 ? kk + 1 : kk].x;
          const float f = __fdiv_rn(v - lk, lk1 - lk);
          const float u = (float)(w[k] >> 8) * 0x1p-24f;
          const uint32_t up = (kk < L - 1 && v > lk && u < f) ? 1u : 0u;
          idx = (uint32_t)kk + up;
          idx = __builtin_isinf(v) ? (uint32_t)(L - 1) : idx;
          idx = (valid[k] && v > 0.0f) ? idx : 0u;           // zero, negative, NaN
          keep = enc_tab[idx].y;
        } else if (valid[k] && v > 0.0f) {
          // the largest level k >= 1 at or below v (1 when none is): from
          // the log2 estimate, moved down while the level is above v and up
          // while the next level is not (levels do not decrease with k)
          float t = (__builtin_amdgcn_logf(v) - est_lo) * est_scale + 1.0f;
          t = t >= 1.0f ? t : 1.0f;   // also NaN
          t = t <= (float)(L - 1) ? t : (float)(L - 1);
          int kk = (int)t;
          float lk = q1_level(lo, hi, kk, L);
          while (kk > 1 && lk > v) lk = q1_level(lo, hi, --kk, L);
          float lk1 = kk < L - 1 ? q1_level(lo, hi, kk + 1, L) : lk;
          while (kk < L - 1 && lk1 <= v) {
            ++kk;
            lk = lk1;
            lk1 = kk < L - 1 ? q1_level(lo, hi, kk + 1, L) : lk;
          }
          const float f = __fdiv_rn(v - lk, lk1 - lk);
          const float u = (float)(w[k] >> 8) * 0x1p-24f;
          const bool up = kk < L - 1 && v > lk && u < f;
          idx = (uint32_t)kk + (up ? 1u : 0u);
          keep = up ? lk1 : lk;
          if (__builtin_isinf(v)) {
            idx = (uint32_t)(L - 1);
            keep = lk;   // kk reached L - 1
          }
        }
        vq[k] = keep;
        field |= idx << (BITS * k);
      }
      // the tile's index words, assembled in LDS (fields straddle words)
      const int b0 = 4 * tid * BITS, sh = b0 & 31;
      if (field) {
        atomicOr(&words[b0 >> 5], field << sh);
        if (sh + 4 * BITS > 32) atomicOr(&words[(b0 >> 5) + 1], field >> (32 - sh));
      }
      __syncthreads();
      const long long nwords = (n * BITS + 31) >> 5, base_w = local * kWords;
      uint32_t* out = reinterpret_cast<uint32_t*>(e.v_index);
      for (int j = tid; j < kWords; j += kThreads)
        if (base_w + j < nwords) out[base_w + j] = words[j];
      if ((tid & (B / 4 - 1)) == 0 && valid[0]) reinterpret_cast<uint32_t*>(e.v_ends)[blk] = ends;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        vq[k] = v1[k];
        if (valid[k]) e.v_fp32[i0 + k] = v1[k];
      }
    }
  }

  // ---- first moment: UState per group, or FP32
  {
    float q[4] = {0.f, 0.f, 0.f, 0.f};
    if (cm) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float den = (use_tab && cv) ? vq[k] : sqrt_rn(div_bc2(vq[k], s)) + s.eps;
        q[k] = valid[k] ? __fdiv_rn(div_uniform(m1[k], ts.inv_bc1), den) : 0.0f;
      }
    }
    // group sums: a perfect pairwise tree in double (zero padding past the end)
    double gs[4];
    if (G >= 4) {
      const double t = seg_reduce(((double)q[0] + (double)q[1]) + ((double)q[2] + (double)q[3]), G / 4,
                                  [](double a, double b) { return a + b; }, dslot);
      gs[0] = gs[1] = gs[2] = gs[3] = t;
    } else if (G == 2) {
      gs[0] = gs[1] = (double)q[0] + (double)q[1];
      gs[2] = gs[3] = (double)q[2] + (double)q[3];
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) gs[k] = (double)q[k];
    }
    if (cm) {
      uint32_t w[4];
      philox4x32_10(ctr, stp, tsr, 1u, sk0, sk1, w);
      uint32_t codes = 0;
      double r2[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const long long g0 = ((i0 + k) >> glog) << glog;
        const long long glen = n - g0 < G ? n - g0 : G;
        const uint32_t mean16 = bf16_encode((float)(gs[k] / (double)glen));
        const float mean = __uint_as_float(mean16 << 16);
        const float r = q[k] - mean;
        r2[k] = valid[k] ? (double)r * (double)r : 0.0;
        float x = s_enc > 0.0f ? __fdiv_rn(r, s_enc) : 0.0f;
        x = x > 1.5f ? 1.5f : x;
        x = x < -1.5f ? -1.5f : x;
        float u = (float)(w[k >> 1] >> 8) * 0x1p-24f;
        if (k & 1) u = 1.0f - u;
        const uint32_t kk = (uint32_t)(x >= -0.5f) + (uint32_t)(x >= 0.5f);
        uint32_t code = kk;
        if (x >= 1.5f) code = 3;
        else if (u < x - ustate_level(kk)) code = kk + 1;
        codes |= valid[k] ? code << (2 * k) : 0u;
        // the first value of each group stores its mean
        if (valid[k] && i0 + k == g0) e.m_means[(i0 + k) >> glog] = (uint16_t)mean16;
      }
      if (valid[0]) e.m_codes[i0 >> 2] = (uint8_t)codes;
      const double tsum = butterfly_sum<64>((r2[0] + r2[1]) + (r2[2] + r2[3]));
      const long long sub = local * (kGenTile / kTurboTile) + wave;   // this wavefront's 256 values
      if (lane == 0 && sub * kTurboTile < n) ws[e.ws0 + sub] = tsum;
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (valid[k]) e.m_fp32[i0 + k] = m1[k];
    }
  }
}

// Six wavefronts per SIMD: measured faster than the five the registers
// allow unasked (4-6% at table layouts) and than seven or eight, where the
// spills grow.
template <int BITS, bool COUNT, bool TYPED>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6)))
turbo_general(const TurboEntry* __restrict__ table, int count, long long tile_base, Scalars s, TurboScalars ts,
              int blog, int glog, double* ws, unsigned long long* nonfinite) {
  __shared__ uint32_t words[kGenTile * BITS / 32];   // the tile's index words
  __shared__ float2 tabs[2 * kGenTile];              // decode, encode tables (L <= B)
  __shared__ uint32_t eslot[2 * kGenTile / 32];      // each block's two endpoints
  __shared__ float fslot[4];
  __shared__ double dslot[4];
  __shared__ int islot[4];
  if (!resolve_inputs(s)) return;   // uniform: before any barrier
  const long long tile = tile_base + blockIdx.x;
  int lo_t = 0, hi_t = count - 1;                    // the last entry with tile0 <= tile
  while (lo_t < hi_t) {
    const int mid = (lo_t + hi_t + 1) >> 1;
    if (table[mid].tile0 <= tile) lo_t = mid;
    else hi_t = mid - 1;
  }
  const TurboEntry* ep = table + lo_t;
  const long long local = tile - ep->tile0;
  uint32_t bad = 0;
  if ((local + 1) * kGenTile <= ep->n)
    general_tile<BITS, true, TYPED>(ep, local, s, ts, blog, glog, ws, bad, words, tabs, eslot, fslot, dslot, islot);
  else
    general_tile<BITS, false, TYPED>(ep, local, s, ts, blog, glog, ws, bad, words, tabs, eslot, fslot, dslot, islot);
  if constexpr (COUNT) flush_count(bad, nonfinite);
}

// The residual sums of the tensors with a UState first moment.  Each tile
// wrote one double; a tensor's sum is the perfect pairwise tree over its
// tile sums in index order, zero-padded to a power of two.  turbo_chunks
// reduces every 2048-sum chunk of every tensor in parallel; the chunks are
// aligned subtrees of each tensor's tree (a padded length above 2048 is a
// multiple of 2048, and zero subtrees add exactly), so turbo_reduce, run
// over the chunk sums, completes exactly the same tree.
struct TurboReduceEntry {
  float* scal;
  long long ws0;       // first tile sum in the workspace
  long long tiles;
  long long n;
  long long cs0;       // first chunk sum in the workspace
  long long chunk0;    // global index of the tensor's first chunk
  long long chunks;    // ceil(tiles / 2048)
};

constexpr int kTurboChunk = 2048;

// Perfect pairwise tree over a[0..m) zero-padded to kTurboChunk values, in
// LDS, by the whole workgroup; returns the sum in every thread.
__device__ __forceinline__ double chunk_tree(const double* a, long long m, double* buf) {
  const int tid = threadIdx.x;
  for (int j = tid; j < kTurboChunk; j += kThreads) buf[j] = j < m ? a[j] : 0.0;
  __syncthreads();
  for (int width = kTurboChunk / 2; width >= 1; width >>= 1) {
    double t[kTurboChunk / 2 / kThreads];           // this level's sums, then written back
#pragma unroll
    for (int q = 0; q < kTurboChunk / 2 / kThreads; ++q) {
      const int j = tid + q * kThreads;
      t[q] = j < width ? buf[2 * j] + buf[2 * j + 1] : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kTurboChunk / 2 / kThreads; ++q) {
      const int j = tid + q * kThreads;
      if (j < width) buf[j] = t[q];
    }
    __syncthreads();
  }
  const double r = buf[0];
  __syncthreads();                                   // buf is refilled by the next call
  return r;
}

// One workgroup per chunk of tile sums over all tensors.
__global__ void __launch_bounds__(kThreads)
turbo_chunks(const TurboReduceEntry* __restrict__ list, int nreduce, double* ws) {
  __shared__ double buf[kTurboChunk];
  const long long c = blockIdx.x;
  int lo = 0, hi = nreduce - 1;                      // the last entry with chunk0 <= c
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (list[mid].chunk0 <= c) lo = mid;
    else hi = mid - 1;
  }
  const TurboReduceEntry r = list[lo];
  const long long k = c - r.chunk0;
  const double sum = chunk_tree(ws + r.ws0 + k * kTurboChunk, r.tiles - k * kTurboChunk, buf);
  if (threadIdx.x == 0) ws[r.cs0 + k] = sum;
}

// One workgroup per tensor: the rest of the tree over its chunk sums (in
// chunks of 2048, level by level, written back in place), then the scale
// rotation.
__global__ void __launch_bounds__(kThreads)
turbo_reduce(const TurboReduceEntry* __restrict__ list, double* ws, double factor, const unsigned long long* skip) {
  __shared__ double buf[kTurboChunk];
  if (skip != nullptr && *skip != 0ull) return;   // the step was skipped: no new sums, no rotation
  const TurboReduceEntry r = list[blockIdx.x];
  double* a = ws + r.cs0;
  long long m = r.chunks;
  while (m > 1) {
    const long long groups = (m + kTurboChunk - 1) / kTurboChunk;
    for (long long c = 0; c < groups; ++c) {
      const double sum = chunk_tree(a + c * kTurboChunk, m - c * kTurboChunk, buf);
      if (threadIdx.x == 0) a[c] = sum;
      __syncthreads();
    }
    m = groups;
  }
  if (threadIdx.x == 0) {
    const double total = a[0];
    const float s_enc = r.scal[1];
    r.scal[0] = s_enc;
    r.scal[1] = (float)(factor * __builtin_sqrt(total / (double)r.n));
    r.scal[2] = 0.0f;
  }
}

// Self-test of the endpoint rounding: for each positive finite in[i], the
// two endpoints of a one-value block, low half down, high half up.
__global__ void __launch_bounds__(kThreads) q1_ends_kernel(const float* in, uint32_t* out, long long n) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n; i += (long long)gridDim.x * kThreads) {
    const float v = in[i];
    out[i] = log2_directed16(v, false, true) | (log2_directed16(v, true, true) << 16);
  }
}

// Self-test export: out[i] = RN32(2^x[i]) as the 4-bit tables decide it
// (the device exp2 with its 2^-48 margin, then the double-double
// evaluation), or with exact != 0 through the double-double evaluation
// alone.
__global__ void __launch_bounds__(kThreads) pow2_rn32_kernel(const double* x, int exact, float* out, long long n) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n; i += (long long)gridDim.x * kThreads) {
    float a;
    out[i] = (!exact && q1_level_fast(x[i], &a)) ? a : pow2_rn32_slow(x[i]);
  }
}

// Self-test export: the levels of endpoint word ends[w] at out[w L + k],
// one half-wavefront per word.  exact = 0: through the step's own table
// builders (build_tables for indices of at most 4 bits, build_levels for
// 6 and 8); exact != 0: every level through the double-double evaluation.
template <int BITS>
__global__ void __launch_bounds__(kThreads) q1_levels_kernel(const uint32_t* ends, int exact, float* out, long long n) {
  constexpr int L = 1 << BITS;
  __shared__ float lev[kThreads / 64][2][256];
  const int lane = threadIdx.x & 63, half = lane >> 5, lane_in_half = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float* t = lev[wave][half];
  const long long nw = (long long)gridDim.x * (kThreads / 64);
  for (long long pw = (long long)blockIdx.x * (kThreads / 64) + wave; 2 * pw < n; pw += nw) {
    const long long w = 2 * pw + half;
    const uint32_t word = w < n ? ends[w] : 0u;
    if (exact) {
      const double lo = f16_to_double(word & 0xFFFFu), hi = f16_to_double(word >> 16);
      for (int k = lane_in_half; k < L; k += 32)
        if (w < n) out[w * L + k] = k == 0 ? 0.0f : pow2_rn32_slow(q1_level_x(lo, hi, k, L));
      continue;
    }
    if constexpr (BITS <= 4)
      build_tables<BITS>((lds_float*)t, word, 1.0, 0.0f, lane_in_half);
    else
      build_levels<BITS>((lds_float*)t, word, lane_in_half);
    wave_lds_sync();
    constexpr int kStride = BITS <= 4 ? 2 : 1;
    for (int k = lane_in_half; k < L; k += 32)
      if (w < n) out[w * L + k] = t[kStride * k];
    wave_lds_sync();
  }
}

}  // namespace pa
