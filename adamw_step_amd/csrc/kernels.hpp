// kernels.hpp -- gfx950 kernels of the packed-AdamW step.
//
// Elementwise modes (packed E4, packed FP16, FP32): one launch covers a
// table of tensors cut into 4096-element tiles, one tile per workgroup, in
// tile order.  Each thread moves 16-byte vectors of parameter, gradient and
// state (one read and one write per word), keeps the whole update in
// registers, and never touches LDS.  A workgroup finds its tensor by a
// bisection over the table on scalar loads.
//
// Blockwise 8-bit mode: a persistent grid over 2048-element blocks, one
// 256-thread workgroup per block at a time; the code maps and their
// midpoints sit in LDS, the block absmax is a wavefront shuffle reduction
// followed by a four-entry LDS reduction.
//
// The FP32 update follows the KBench quantized-optimizer-state reference
// (`quantized_adamw_step`) left to right, one IEEE binary32 operation at a
// time: no contraction into FMA (this file is compiled with contraction
// off), correctly rounded division and square root, denormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codec.hpp"

#pragma clang fp contract(off)

namespace pa {

// The eight binary32 scalars of one call (formed on the host in double,
// each rounded once), and the call's optional device inputs.
struct Scalars {
  float beta1, one_m_beta1, beta2, one_m_beta2;
  float bc2, lr_over_bc1, decay, eps;
  float beta1_x2p112;   // beta1 * 2^112, exact (pairs with e4_decode_m_unscaled)
  float gmul;           // gradient multiplier: 1, or *gscale once read on the device
  double inv_bc2;       // 1/bc2 rounded to double, for the exact quotient v'/bc2
  const float* gscale;                // nullable device gradient scale
  const unsigned long long* skip;     // nullable device flag: nonzero skips the call
};

// Reads the optional device inputs at the start of a launch (uniform across
// the grid).  Returns false when the update is to be skipped; otherwise
// sets the gradient multiplier.  A product with 1 is exact, so gradients
// without a scale would pass through unchanged; the elementwise kernels
// still leave the product out when no scale is given (template flag
// SCALE), since it costs registers in their unrolled tiles.
__device__ __forceinline__ bool resolve_inputs(Scalars& s) {
  if (s.skip != nullptr && *s.skip != 0ull) return false;
  if (s.gscale != nullptr) s.gmul = *s.gscale;
  return true;
}

template <bool SCALE>
__device__ __forceinline__ float scaled(float g, const Scalars& s) {
  if constexpr (SCALE) return g * s.gmul;
  else return g;
}

// One tensor of an elementwise launch.  Every buffer of a tensor shares one
// 16-byte phase; `phase` is that phase in elements, so element i sits at
// virtual index i + phase and virtual indices 4k..4k+3 form one aligned
// 16-byte vector.
struct Entry {
  void* p;           // parameters, element type PT of the launch
  const void* g;     // gradients, element type GT
  void* s0;          // packed words, or the FP32 first moment
  float* s1;         // FP32 second moment (FP32 mode only)
  long long n;       // elements
  long long tile0;   // first global tile of this tensor
  int phase;
  int pad_;
};

// Streaming access policy: every byte is read once and written once, so the
// 16-byte vector loads and stores carry the nontemporal hint (measured on
// MI355X: the 3-in/2-out stream runs about 4% faster with it).
#ifndef PA_STREAM_NT_LOADS
#define PA_STREAM_NT_LOADS 1
#endif
#ifndef PA_STREAM_NT_STORES
#define PA_STREAM_NT_STORES 1
#endif
#ifndef PA_TILE_UNROLL
#define PA_TILE_UNROLL 4
#endif

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T stream_load(const T* p) {
  if constexpr (PA_STREAM_NT_LOADS) return __builtin_nontemporal_load(p);
  else return *p;
}

template <typename T>
__device__ __forceinline__ void stream_store(T* p, T v) {
  if constexpr (PA_STREAM_NT_STORES) __builtin_nontemporal_store(v, p);
  else *p = v;
}

constexpr int kThreads = 256;
constexpr int kUnroll = PA_TILE_UNROLL;
constexpr int kTile = kThreads * 4 * kUnroll;   // elements per tile of a large list
// Lists of fewer elements than this take tiles a quarter as large (one
// 16-byte vector per thread per stream): more workgroups, so the last
// workgroups to finish hold less work.
#ifndef PA_SMALL_LIST_ELEMS
#define PA_SMALL_LIST_ELEMS (32LL << 20)
#endif
constexpr long long kSmallList = PA_SMALL_LIST_ELEMS;
constexpr int kSmallUnroll = 1;
constexpr int kBlock = 2048;                    // blockwise quantisation block

enum { kModeFp32 = 0, kModeE4 = 1, kModeF16 = 2 };

// Element types of parameters and gradients.  The update always runs in
// FP32: 16-bit inputs widen exactly, and the new parameter is rounded back
// to its own type, to nearest even (the KBench reference widens its inputs
// with .float() and narrows its output with .to(bfloat16)).
enum { kF32 = 0, kBF16 = 1, kF16 = 2 };

template <int T> struct Elem;
template <> struct Elem<kF32> {
  using scalar = float;
  using vec4 = f32x4;
  static __device__ __forceinline__ float widen(float x) { return x; }
  static __device__ __forceinline__ float narrow(float x) { return x; }
};
template <> struct Elem<kBF16> {
  using scalar = uint16_t;
  using vec4 = u16x4;
  static __device__ __forceinline__ float widen(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
  static __device__ __forceinline__ uint16_t narrow(float x) { return (uint16_t)bf16_encode(x); }
};
template <> struct Elem<kF16> {
  using scalar = uint16_t;
  using vec4 = u16x4;
  static __device__ __forceinline__ float widen(uint16_t x) { return f16_decode(x); }
  static __device__ __forceinline__ uint16_t narrow(float x) { return (uint16_t)f16_encode(x); }
};

// Correctly rounded FP32 square root.
//
// The hardware estimate s (v_sqrt_f32) is within one ulp of sqrt(x), so
// RN(sqrt(x)) is one of s-1ulp, s, s+1ulp (integer steps of the bit
// pattern).  With u the ulp of s, sqrt(x) lies below the midpoint between
// s-1ulp and s exactly when x <= (s-1ulp)*s: the two sides differ by u^2/4
// while x and (s-1ulp)*s are both multiples of u^2 (x of a much coarser
// power of two), so nothing lies strictly between them.  The FMA forms
// x - (s-1ulp)*s with a single rounding, which keeps the sign, and the test
// above the midpoint between s and s+1ulp is the mirror image.  Inputs below
// 2^-96 (denormals included) are first scaled by 2^64, and the root by 2^-32,
// so that the residuals stay far from underflow.  Zero, Inf and NaN fall
// through unchanged: the neighbour residuals are then NaN or zero and
// neither test fires.
__device__ __forceinline__ float sqrt_pick(float xs) {
  float s = __builtin_amdgcn_sqrtf(xs);
  const float s_dn = __uint_as_float(__float_as_uint(s) - 1u);
  const float s_up = __uint_as_float(__float_as_uint(s) + 1u);
  const float r_dn = __builtin_fmaf(-s_dn, s, xs);
  const float r_up = __builtin_fmaf(-s_up, s, xs);
  s = r_dn <= 0.0f ? s_dn : s;
  return r_up > 0.0f ? s_up : s;
}

__device__ __forceinline__ float sqrt_rn(float x) {
  float s = sqrt_pick(x);
  if (__builtin_expect(x < 0x1p-96f, 0)) s = sqrt_pick(x * 0x1p64f) * 0x1p-32f;
  return s;
}

// v'/bc2, correctly rounded: the product of v' and the double nearest 1/bc2
// is within 2^-52 (relative) of the exact quotient, while a quotient of two
// binary32 numbers that is not itself a binary32 number lies at least 2^-49
// (relative) away from every binary32 rounding midpoint, so rounding the
// double product to binary32 gives the correctly rounded quotient.
__device__ __forceinline__ float div_bc2(float v1, const Scalars& s) {
  return (float)((double)v1 * s.inv_bc2);
}

// New moments and the FP32 step with decoupled decay.  `beta1_m` is the
// product beta1 * m, formed by the caller (see e4_decode_m_unscaled).
// `g` is the gradient already multiplied by the call's gradient scale.
__device__ __forceinline__ void adamw(float p, float g, float beta1_m, float v, const Scalars& s,
                                      float& p1, float& m1, float& v1) {
  m1 = beta1_m + s.one_m_beta1 * g;
  v1 = s.beta2 * v + (s.one_m_beta2 * g) * g;
  const float denom = sqrt_rn(div_bc2(v1, s)) + s.eps;
  const float upd = __fdiv_rn(s.lr_over_bc1 * m1, denom);
  p1 = p * s.decay - upd;
}

__device__ __forceinline__ uint32_t nonfinite3(float a, float b, float c) {
  return (__builtin_isfinite(a) && __builtin_isfinite(b) && __builtin_isfinite(c)) ? 0u : 1u;
}

// Packed modes: decode the prior word, update, encode m' and sqrt(v').
template <int MODE>
__device__ __forceinline__ uint32_t packed_elem(float& p, float g, uint32_t w, const Scalars& s,
                                                uint32_t& bad) {
  float beta1_m, r;
  if constexpr (MODE == kModeE4) {
    beta1_m = s.beta1_x2p112 * e4_decode_m_unscaled(w);
    r = e4_decode_r(w);
  } else {
    beta1_m = s.beta1 * f16_decode(w);
    r = f16_decode(w >> 16);
  }
  float p1, m1, v1;
  adamw(p, g, beta1_m, r * r, s, p1, m1, v1);
  bad += nonfinite3(p1, m1, v1);
  p = p1;
  const float r1 = sqrt_rn(v1);
  if constexpr (MODE == kModeE4) {
    return (e4_encode_r(r1) << 16) | e4_encode_m(m1);
  } else {
    return (f16_encode(r1) << 16) | f16_encode(m1);
  }
}

__device__ __forceinline__ void fp32_elem(float& p, float g, float& m, float& v, const Scalars& s,
                                          uint32_t& bad) {
  float p1, m1, v1;
  adamw(p, g, s.beta1 * m, v, s, p1, m1, v1);
  bad += nonfinite3(p1, m1, v1);
  p = p1;
  m = m1;
  v = v1;
}


// One element at index i of tensor e (ragged edges only).
template <int MODE, int PT, int GT, bool SCALE>
__device__ __forceinline__ void scalar_elem(const Entry& e, long long i, const Scalars& s, uint32_t& bad) {
  using PE = Elem<PT>;
  using GE = Elem<GT>;
  typename PE::scalar* P = static_cast<typename PE::scalar*>(e.p);
  float p = PE::widen(P[i]);
  const float g = scaled<SCALE>(GE::widen(static_cast<const typename GE::scalar*>(e.g)[i]), s);
  if constexpr (MODE == kModeFp32) {
    float* m = static_cast<float*>(e.s0);
    float mm = m[i], vv = e.s1[i];
    fp32_elem(p, g, mm, vv, s, bad);
    m[i] = mm;
    e.s1[i] = vv;
  } else {
    uint32_t* w = static_cast<uint32_t*>(e.s0);
    w[i] = packed_elem<MODE>(p, g, w[i], s, bad);
  }
  P[i] = PE::narrow(p);
}

// Tile `tile` (local to tensor e).  Each thread moves four elements per
// vector access of each stream: 16 bytes for FP32 data, 8 for 16-bit data.
// SPLIT > 1 takes a whole tile in that many rounds of loads, arithmetic and
// stores, one after the other: fewer values live at once, so more
// wavefronts fit (the variants that also count or scale need it).
// UNROLL: 16-byte vectors per thread per stream in a tile (a tile holds
// 1024 * UNROLL elements).
template <int MODE, int PT, int GT, bool SCALE, int SPLIT = 1, int UNROLL = kUnroll>
__device__ __forceinline__ void run_tile(const Entry& e, long long tile, const Scalars& s, uint32_t& bad) {
  static_assert(UNROLL % SPLIT == 0, "whole rounds");
  constexpr int U = UNROLL / SPLIT;
  constexpr int kTile = kThreads * 4 * UNROLL;
  using PE = Elem<PT>;
  using GE = Elem<GT>;
  using PV = typename PE::vec4;
  using GV = typename GE::vec4;
  const long long v0 = tile * kTile;
  const long long vend = e.n + e.phase;
  const int tid = threadIdx.x;
  if (v0 >= e.phase && v0 + kTile <= vend) {
    // Whole tile inside the tensor: unguarded vector accesses.
    const long long q0 = v0 / 4 + tid;
    PV* P = reinterpret_cast<PV*>(static_cast<typename PE::scalar*>(e.p) - e.phase);
    const GV* G = reinterpret_cast<const GV*>(static_cast<const typename GE::scalar*>(e.g) - e.phase);
    if constexpr (MODE == kModeFp32) {
      f32x4* M = reinterpret_cast<f32x4*>(static_cast<float*>(e.s0) - e.phase);
      f32x4* V = reinterpret_cast<f32x4*>(e.s1 - e.phase);
#pragma unroll 1
      for (int r = 0; r < SPLIT; ++r) {
        PV p[U];
        GV g[U];
        f32x4 m[U], v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const long long q = q0 + (long long)(r * U + u) * kThreads;
          p[u] = stream_load(P + q);
          g[u] = stream_load(G + q);
          m[u] = stream_load(M + q);
          v[u] = stream_load(V + q);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            float pk = PE::widen(p[u][k]), mk = m[u][k], vk = v[u][k];
            fp32_elem(pk, scaled<SCALE>(GE::widen(g[u][k]), s), mk, vk, s, bad);
            p[u][k] = PE::narrow(pk);
            m[u][k] = mk;
            v[u][k] = vk;
          }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const long long q = q0 + (long long)(r * U + u) * kThreads;
          stream_store(P + q, p[u]);
          stream_store(M + q, m[u]);
          stream_store(V + q, v[u]);
        }
      }
    } else {
      u32x4* W = reinterpret_cast<u32x4*>(static_cast<uint32_t*>(e.s0) - e.phase);
#pragma unroll 1
      for (int r = 0; r < SPLIT; ++r) {
        PV p[U];
        GV g[U];
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const long long q = q0 + (long long)(r * U + u) * kThreads;
          p[u] = stream_load(P + q);
          g[u] = stream_load(G + q);
          w[u] = stream_load(W + q);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            float pk = PE::widen(p[u][k]);
            w[u][k] = packed_elem<MODE>(pk, scaled<SCALE>(GE::widen(g[u][k]), s), w[u][k], s, bad);
            p[u][k] = PE::narrow(pk);
          }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const long long q = q0 + (long long)(r * U + u) * kThreads;
          stream_store(P + q, p[u]);
          stream_store(W + q, w[u]);
        }
      }
    }
  } else {
    // Ragged tile (first tile of a misaligned tensor, or the last one).
    for (int u = 0; u < UNROLL; ++u) {
      const long long vb = v0 + ((long long)u * kThreads + tid) * 4;
      for (int k = 0; k < 4; ++k) {
        const long long vi = vb + k;
        if (vi >= e.phase && vi < vend) scalar_elem<MODE, PT, GT, SCALE>(e, vi - e.phase, s, bad);
      }
    }
  }
}

__device__ __forceinline__ void flush_count(uint32_t bad, unsigned long long* counter) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) bad += __shfl_xor(bad, off, 64);
  if ((threadIdx.x & 63) == 0 && bad != 0u) atomicAdd(counter, (unsigned long long)bad);
}

// The tensor of a tile: table[0..count) holds the tensors' first tiles in
// increasing order and table[count].tile0 the total, so a bisection over
// the first tiles finds the entry.  `tile` is uniform across the workgroup,
// so the search runs on scalar loads and registers.
__device__ __forceinline__ int tensor_of_tile(const Entry* table, int count, long long tile) {
  int lo = 0, hi = count;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (table[mid].tile0 <= tile) lo = mid;
    else hi = mid;
  }
  return lo;
}

// Multi-tensor launch, one tile per workgroup: the workgroups of one launch
// cover tiles tile_base .. tile_base + gridDim.x - 1 of the list.  The
// hardware hands out workgroups in index order, so the tiles in flight at
// any moment form one compact, advancing window of every stream (measured
// on MI355X: a write stream runs at about 6.8 TB/s in this order against
// about 5.5 TB/s for a persistent grid striding over the same tiles).
template <int MODE, int PT, int GT, bool COUNT, bool SCALE, int UNROLL>
__global__ void __launch_bounds__(kThreads)
elementwise_list(const Entry* __restrict__ table, int count, long long tile_base, Scalars s,
                 unsigned long long* nonfinite) {
  if (!resolve_inputs(s)) return;
  const long long tile = tile_base + blockIdx.x;
  const Entry e = table[tensor_of_tile(table, count, tile)];
  uint32_t bad = 0;
  run_tile<MODE, PT, GT, SCALE, ((COUNT || SCALE) && UNROLL > 1) ? 2 : 1, UNROLL>(e, tile - e.tile0, s, bad);
  if constexpr (COUNT) flush_count(bad, nonfinite);
}

// Single tensor, its entry passed by value (no table in device memory).
template <int MODE, int PT, int GT, bool COUNT, bool SCALE, int UNROLL>
__global__ void __launch_bounds__(kThreads)
elementwise_one(Entry e, long long tile_base, Scalars s, unsigned long long* nonfinite) {
  if (!resolve_inputs(s)) return;
  uint32_t bad = 0;
  run_tile<MODE, PT, GT, SCALE, ((COUNT || SCALE) && UNROLL > 1) ? 2 : 1, UNROLL>(e, tile_base + blockIdx.x, s, bad);
  if constexpr (COUNT) flush_count(bad, nonfinite);
}

// ---------------------------------------------------------------------------
// Blockwise 8-bit mode.

struct BlockwiseArgs {
  const float* p;
  const float* g;
  uint8_t* m_code;
  float* m_absmax;
  uint8_t* v_code;
  float* v_absmax;
  const float* qmap_m;
  const float* qmap_v;
  uint16_t* p_out;
  long long nblocks;
};

// Midpoint search through a bucket table.
//
// The top 13 bits of a float's bit pattern (sign, exponent, 4 mantissa
// bits) pick one of 8192 buckets, a sixteenth of a binade of one sign each;
// the floats of a bucket form one contiguous numeric range (for negative
// buckets the range runs from the largest magnitude up).  base[b] is the
// number of midpoints below the bucket's smallest float.  A value's code,
// the number of midpoints strictly below it, is base[b] plus the number of
// the bucket's own midpoints below it.  When no bucket holds more than NCMP
// midpoints that is a plain count over mid[base .. base+NCMP) (midpoints
// past the bucket are above the value, and mid[255..258] = +Inf pads the
// end); fuller maps take a bisection over the bucket, whose size is the
// base of the numerically next bucket minus base[b].  Ties go to the lower
// map entry; NaN is ordered above every number.
constexpr int kBucketShift = 19;
constexpr int kBuckets = 1 << (32 - kBucketShift);
constexpr int kMidPad = 260;

__device__ __forceinline__ uint32_t bucket_of(float x) { return __float_as_uint(x) >> kBucketShift; }

// The numerically next bucket (kBuckets, a pad of 255, after the last
// positive one; the first positive one after the smallest negative one).
__device__ __forceinline__ uint32_t bucket_next(uint32_t b) {
  constexpr uint32_t h = (uint32_t)kBuckets / 2;
  return b + 1 < h ? b + 1 : (b + 1 == h ? (uint32_t)kBuckets : (b == h ? 0u : b - 1));
}

template <int NCMP, bool SLOW>
__device__ __forceinline__ uint32_t search_mid(const float* mid, const uint8_t* base, float c) {
  const uint32_t b = bucket_of(c);
  uint32_t lo = base[b];
  if constexpr (NCMP > 0) {
    uint32_t code = lo;
#pragma unroll
    for (int k = 0; k < NCMP; ++k) code += mid[lo + k] < c ? 1u : 0u;
    lo = code;
  } else {
    const uint32_t nb = base[bucket_next(b)];
    uint32_t n = nb > lo ? nb - lo : 0u;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const uint32_t half = n >> 1;
      const bool lt = mid[lo + half] < c;
      lo = lt ? lo + half + 1 : lo;
      n = lt ? n - half - 1 : half;
    }
  }
  if constexpr (SLOW) return (c != c) ? 255u : lo;
  else return lo;
}

// c / d for the block normaliser d (a positive normal binary32, or +Inf or
// NaN on the slow path): the double product with rd = 1/d rounded to
// double, rounded once to binary32, is the correctly rounded quotient (the
// quotient of two binary32 numbers is either one itself or at least 2^-49
// relative away from every binary32 midpoint, while the product is within
// 2^-52).  The one case that argument leaves open is a quotient exactly on
// a midpoint of the subnormal range: the slow path takes the hardware
// division for nonzero products below the normal range.  The fast path is
// used when no map midpoint lies within 2^-125 of zero (every quotient in
// that range then gets the same code) and d is finite.
template <bool SLOW>
__device__ __forceinline__ float div_block(float x, float d, double rd) {
  const double q = (double)x * rd;
  float c = (float)q;
  if constexpr (SLOW) {
    if (__builtin_expect(q != 0.0 && __builtin_fabs(q) < 0x1p-126, 0)) c = __fdiv_rn(x, d);
    if (__builtin_expect(!(__builtin_fabsf(d) < __builtin_inff()), 0)) c = __fdiv_rn(x, d);
  }
  return c;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off, 64));
  return x;
}

// Codes of four values normalised by d, packed little-endian in 32 bits.
template <int NCMP, bool SLOW>
__device__ __forceinline__ uint32_t codes4(const float* x, float d, double rd, const float* mid, const uint8_t* base) {
  uint32_t out = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) out |= search_mid<NCMP, SLOW>(mid, base, div_block<SLOW>(x[k], d, rd)) << (8 * k);
  return out;
}

template <bool SLOW>
__device__ __forceinline__ uint32_t codes4_dispatch(int ncmp, const float* x, float d, double rd, const float* mid,
                                                    const uint8_t* base) {
  switch (ncmp) {   // uniform across the workgroup
    case 1: return codes4<1, SLOW>(x, d, rd, mid, base);
    case 2: return codes4<2, SLOW>(x, d, rd, mid, base);
    case 3: return codes4<3, SLOW>(x, d, rd, mid, base);
    case 4: return codes4<4, SLOW>(x, d, rd, mid, base);
    default: return codes4<0, SLOW>(x, d, rd, mid, base);
  }
}

// Per-map search set-up in LDS: the padded midpoints, the bucket table, the
// compare count of the fullest bucket (0 = bisection) and whether any
// midpoint lies within 2^-125 of zero (then the normaliser keeps its guard).
struct MapTables {
  float mid[kMidPad];
  uint8_t base[kBuckets + 4];
};

// The bucket table as a histogram and one scan: each midpoint adds one to
// its bucket's byte counter (four counters per LDS word; at most 255
// midpoints, so no counter carries into the next), and an exclusive scan in
// numeric bucket order (the negative buckets from the most negative, then
// the positive ones) turns the counts into base[].  A midpoint of -0 counts
// with +0: it compares like +0 with every value.  NaN midpoints (outside the
// ascending-map contract) are never below a value and are not counted.
// Thread t owns the 32 buckets of numeric positions 32t..32t+31, so the two
// halves of the workgroup scan the two signs and each wavefront's order is
// uniform.
__device__ __forceinline__ void build_map(const float* lut, MapTables& t, uint32_t* red, int& ncmp, bool& guard) {
  static_assert(kThreads == 256 && kBuckets == 32 * kThreads, "one thread per 32 buckets");
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t* cnt = reinterpret_cast<uint32_t*>(t.base);
  for (int j = tid; j < kMidPad; j += kThreads)
    t.mid[j] = j < 255 ? (lut[j] + lut[j + 1]) * 0.5f : __builtin_inff();
  for (int w = tid; w < (kBuckets + 4) / 4; w += kThreads) cnt[w] = 0u;
  __syncthreads();
  uint32_t near_zero = 0;
  if (tid < 255) {
    const float m = t.mid[tid];
    near_zero = __builtin_fabsf(m) < 0x1p-125f ? 1u : 0u;
    if (m == m) {
      const uint32_t b = __float_as_uint(m) == 0x80000000u ? 0u : bucket_of(m);
      atomicAdd(&cnt[b >> 2], 1u << (8 * (b & 3u)));
    }
  }
  __syncthreads();
  const bool neg = tid < kThreads / 2;
  const uint32_t w0 = neg ? (uint32_t)(kBuckets - 32 * (tid + 1)) / 4 : (uint32_t)(32 * (tid - kThreads / 2)) / 4;
  uint32_t words[8], total = 0, fullest = 0;
#pragma unroll
  for (int q = 0; q < 8; ++q) words[q] = cnt[w0 + q];
#pragma unroll
  for (int k = 0; k < 32; ++k) {
    const uint32_t c = (words[k >> 2] >> (8 * (k & 3))) & 0xFFu;
    total += c;
    fullest = max(fullest, c);
  }
  uint32_t incl = total;                           // inclusive scan over the wavefront
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = (uint32_t)__shfl_up((int)incl, d, 64);
    incl += lane >= d ? y : 0u;
  }
  fullest = wave_max_u32(fullest);
  near_zero = wave_max_u32(near_zero);
  if (lane == 63) red[tid >> 6] = incl | (fullest << 12) | (near_zero << 31);
  __syncthreads();
  uint32_t run = incl - total, f = 0, nz = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    const uint32_t r = red[w];
    run += w < (tid >> 6) ? (r & 0xFFFu) : 0u;
    f = max(f, (r >> 12) & 0xFFFu);
    nz |= r >> 31;
  }
  uint32_t out[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (neg) {                                       // numeric order runs down the bucket index
#pragma unroll
    for (int k = 31; k >= 0; --k) {
      out[k >> 2] |= run << (8 * (k & 3));
      run += (words[k >> 2] >> (8 * (k & 3))) & 0xFFu;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      out[k >> 2] |= run << (8 * (k & 3));
      run += (words[k >> 2] >> (8 * (k & 3))) & 0xFFu;
    }
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) cnt[w0 + q] = out[q];
  if (tid == 0) cnt[kBuckets / 4] = 0xFFFFFFFFu;   // base[kBuckets..+3] = 255
  guard = nz != 0;
  ncmp = f == 0 ? 1 : (f <= 4 ? (int)f : 0);
  __syncthreads();
}

// The search tables of one map pair: both maps, their midpoint and bucket
// tables, and each map's compare count and near-zero guard.  The ordered
// launch reads them from global memory, built once per call.
struct alignas(16) BwTables {
  float lut_m[256], lut_v[256];
  MapTables tab_m, tab_v;
  int ncmp_m, ncmp_v, guard_m, guard_v;
};
constexpr int kBwTabVec = (int)(sizeof(BwTables) / 16);
static_assert(sizeof(BwTables) % 16 == 0, "copied in 16-byte vectors");

// One workgroup builds the tables of the map pair into `out`.
__global__ void __launch_bounds__(kThreads) blockwise_tables(const float* qmap_m, const float* qmap_v, BwTables* out) {
  __shared__ BwTables T;
  __shared__ uint32_t red[2][kThreads / 64];
  const int tid = threadIdx.x;
  T.lut_m[tid] = qmap_m[tid];
  T.lut_v[tid] = qmap_v[tid];
  __syncthreads();
  int nm, nv;
  bool gm, gv;
  build_map(T.lut_m, T.tab_m, red[0], nm, gm);
  build_map(T.lut_v, T.tab_v, red[1], nv, gv);
  if (tid == 0) {
    T.ncmp_m = nm;
    T.ncmp_v = nv;
    T.guard_m = gm ? 1 : 0;
    T.guard_v = gv ? 1 : 0;
  }
  __syncthreads();
  const uint4* src = reinterpret_cast<const uint4*>(&T);
  uint4* dst = reinterpret_cast<uint4*>(out);
  for (int i = tid; i < kBwTabVec; i += kThreads) dst[i] = src[i];
}

// One 256-thread workgroup per 2048-element block at a time (eight values
// per thread), in one of two launches:
// - ORDERED: workgroup w takes blocks w*per_group .. w*per_group+per_group-1
//   in dispatch order, so the blocks in flight form one compact window, and
//   copies the tables that blockwise_tables built for the call into LDS;
// - persistent: a grid of `stride` workgroups, workgroup w taking blocks w,
//   w+stride, ..., each building the tables in LDS once.
// The loads of a workgroup's next block are issued before the current one
// is reduced and encoded.  The block absmax goes through one of two LDS
// slots, the slots alternating between consecutive blocks, so one barrier
// per block suffices: a wavefront can only rewrite a slot after every
// wavefront has passed the barrier of the block in between, that is after
// every read of the slot.  Four wavefronts per SIMD are asked of the
// register allocator: with fewer the loads in flight do not cover the
// memory latency.  The block step is a kernel argument in both launches: a
// step the compiler sees as the constant 1 makes it keep per-thread
// induction pointers, which costs registers.
template <bool COUNT, bool SCALE, bool ORDERED>
__global__ void __launch_bounds__(kThreads, 4)
blockwise_kernel(BlockwiseArgs a, Scalars s, unsigned long long* nonfinite, const BwTables* tabs,
                 long long per_group, long long stride) {
  __shared__ BwTables T;
  __shared__ uint32_t wave_max[2][2][kThreads / 64];   // [slot][moment][wavefront]
  if (!resolve_inputs(s)) return;   // uniform: before any barrier
  const int tid = threadIdx.x;
  long long b0, bend;
  int ncmp_m, ncmp_v;
  bool guard_m, guard_v;
  if constexpr (ORDERED) {
    b0 = (long long)blockIdx.x * per_group;
    bend = b0 + per_group < a.nblocks ? b0 + per_group : a.nblocks;
    const uint4* src = reinterpret_cast<const uint4*>(tabs);
    uint4* dst = reinterpret_cast<uint4*>(&T);
    for (int i = tid; i < kBwTabVec; i += kThreads) dst[i] = src[i];
  } else {
    b0 = blockIdx.x;
    bend = a.nblocks;
    T.lut_m[tid] = a.qmap_m[tid];
    T.lut_v[tid] = a.qmap_v[tid];
    __syncthreads();
    build_map(T.lut_m, T.tab_m, wave_max[0][0], ncmp_m, guard_m);
    build_map(T.lut_v, T.tab_v, wave_max[0][1], ncmp_v, guard_v);
  }

  // The 1e-30 lower clamp of the normaliser, as a binary32 bit pattern.
  const uint32_t floor_bits = __float_as_uint((float)1e-30);
  uint32_t bad = 0;
  // Inputs of one block for this thread: elements base + h*1024 + 4*tid + k.
  struct BlockIn {
    f32x4 p[2], g[2];
    uint32_t mc[2], vc[2];
    float am, av;
  };
  auto load_block = [&](long long blk, BlockIn& in) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const long long e0 = blk * kBlock + h * 1024 + tid * 4;
      in.p[h] = stream_load(reinterpret_cast<const f32x4*>(a.p + e0));
      in.g[h] = stream_load(reinterpret_cast<const f32x4*>(a.g + e0));
      in.mc[h] = *reinterpret_cast<const uint32_t*>(a.m_code + e0);
      in.vc[h] = *reinterpret_cast<const uint32_t*>(a.v_code + e0);
    }
    in.am = a.m_absmax[blk];
    in.av = a.v_absmax[blk];
  };
  BlockIn cur, nxt;
  if (b0 < bend) load_block(b0, cur);
  if constexpr (ORDERED) {
    __syncthreads();   // the tables copied into LDS
    ncmp_m = T.ncmp_m;
    ncmp_v = T.ncmp_v;
    guard_m = T.guard_m != 0;
    guard_v = T.guard_v != 0;
  }
  int slot = 0;
  for (long long b = b0; b < bend; b += stride, slot ^= 1) {
    const long long base = b * kBlock;
    float m1[8], v1[8];
    uint32_t pbad = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const long long e0 = base + h * 1024 + tid * 4;
      float po[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float m = T.lut_m[(cur.mc[h] >> (8 * k)) & 0xFFu] * cur.am;
        const float v = T.lut_v[(cur.vc[h] >> (8 * k)) & 0xFFu] * cur.av;
        float p1;
        adamw(cur.p[h][k], scaled<SCALE>(cur.g[h][k], s), s.beta1 * m, v, s, p1, m1[h * 4 + k], v1[h * 4 + k]);
        if constexpr (COUNT) pbad |= (__builtin_isfinite(p1) ? 0u : 1u) << (h * 4 + k);
        po[k] = p1;
      }
      uint2 out;
      out.x = bf16_encode2(po[0], po[1]);
      out.y = bf16_encode2(po[2], po[3]);
      *reinterpret_cast<uint2*>(a.p_out + e0) = out;
    }
    // The next block's loads go out before this block's reduction and
    // encoding, so their latency hides behind that work.
    if (b + stride < bend) load_block(b + stride, nxt);
    // Block absmax: on non-negative floats (and NaN with the sign cleared)
    // the unsigned order of the bit patterns is the numeric order, with NaN
    // above everything, so an integer max propagates NaN as the reference's
    // amax does.
    uint32_t xm = 0, xv = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      xm = max(xm, __float_as_uint(m1[k]) & 0x7FFFFFFFu);
      xv = max(xv, __float_as_uint(v1[k]) & 0x7FFFFFFFu);
    }
    xm = wave_max_u32(xm);
    xv = wave_max_u32(xv);
    if ((tid & 63) == 0) {
      wave_max[slot][0][tid >> 6] = xm;
      wave_max[slot][1][tid >> 6] = xv;
    }
    __syncthreads();
    uint32_t Am = wave_max[slot][0][0], Av = wave_max[slot][1][0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
      Am = max(Am, wave_max[slot][0][w]);
      Av = max(Av, wave_max[slot][1][w]);
    }
    const float dm = __uint_as_float(max(Am, floor_bits));
    const float dv = __uint_as_float(max(Av, floor_bits));
    const double rdm = 1.0 / (double)dm;   // correctly rounded double division
    const double rdv = 1.0 / (double)dv;
    // Inf or NaN in a block (absmax at or above the Inf pattern) takes the
    // slow path, which also orders NaN quotients above every midpoint.
    const bool slow_m = guard_m || Am >= kInfBits, slow_v = guard_v || Av >= kInfBits;
    if constexpr (COUNT) {
      // An element counts once if p', m' or v' is Inf or NaN.  p' is tested
      // as it is formed (one bit per element); m' and v' are all finite
      // unless the block absmax is at or above the Inf pattern, so only such
      // blocks test them (this keeps the counting kernel free of spills).
      if (Am >= kInfBits || Av >= kInfBits) {
#pragma unroll
        for (int k = 0; k < 8; ++k) pbad |= nonfinite3(1.0f, m1[k], v1[k]) << k;
      }
      bad += __builtin_popcount(pbad);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t cm = slow_m ? codes4_dispatch<true>(ncmp_m, m1 + 4 * h, dm, rdm, T.tab_m.mid, T.tab_m.base)
                                 : codes4_dispatch<false>(ncmp_m, m1 + 4 * h, dm, rdm, T.tab_m.mid, T.tab_m.base);
      const uint32_t cv = slow_v ? codes4_dispatch<true>(ncmp_v, v1 + 4 * h, dv, rdv, T.tab_v.mid, T.tab_v.base)
                                 : codes4_dispatch<false>(ncmp_v, v1 + 4 * h, dv, rdv, T.tab_v.mid, T.tab_v.base);
      const long long e0 = base + h * 1024 + tid * 4;
      *reinterpret_cast<uint32_t*>(a.m_code + e0) = cm;
      *reinterpret_cast<uint32_t*>(a.v_code + e0) = cv;
    }
    if (tid == 0) {
      a.m_absmax[b] = __uint_as_float(Am);
      a.v_absmax[b] = __uint_as_float(Av);
    }
    cur = nxt;
  }
  if constexpr (COUNT) flush_count(bad, nonfinite);
}

// ---------------------------------------------------------------------------
// Gradient pre-pass: the sum of the squares of all gradients in double and
// the number of non-finite gradients.  A persistent grid walks the same tile
// table as the update (only g, n, phase and tile0 are used); each workgroup
// writes one partial, and one workgroup adds the partials in index order, so
// the result depends only on the list and the grid size.

__device__ __forceinline__ void stats_add(float x, double& acc, uint32_t& bad) {
  const double d = (double)x;
  acc = __builtin_fma(d, d, acc);   // d*d is exact in double: one rounding per term
  bad += __builtin_isfinite(x) ? 0u : 1u;
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// NT: nontemporal loads, for lists too large for the last-level cache (the
// step that follows reads the gradients again; a list that fits the cache
// keeps plain loads so that it stays there).
template <int GT, bool NT>
__device__ __forceinline__ void stats_tile(const Entry& e, long long tile, double& acc, uint32_t& bad) {
  using GE = Elem<GT>;
  using GV = typename GE::vec4;
  const long long v0 = tile * kTile;
  const long long vend = e.n + e.phase;
  const int tid = threadIdx.x;
  const typename GE::scalar* g = static_cast<const typename GE::scalar*>(e.g);
  if (v0 >= e.phase && v0 + kTile <= vend) {
    const GV* G = reinterpret_cast<const GV*>(g - e.phase);
    const long long q0 = v0 / 4 + tid;
    GV x[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const GV* a = G + q0 + (long long)u * kThreads;
      x[u] = NT ? __builtin_nontemporal_load(a) : *a;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) stats_add(GE::widen(x[u][k]), acc, bad);
  } else {
    for (int u = 0; u < kUnroll; ++u) {
      const long long vb = v0 + ((long long)u * kThreads + tid) * 4;
      for (int k = 0; k < 4; ++k) {
        const long long vi = vb + k;
        if (vi >= e.phase && vi < vend) stats_add(GE::widen(g[vi - e.phase]), acc, bad);
      }
    }
  }
}

template <int GT, bool NT>
__global__ void __launch_bounds__(kThreads)
grad_stats_list(const Entry* __restrict__ table, long long total_tiles, double* part_sum,
                unsigned long long* part_bad) {
  __shared__ double wsum[kThreads / 64];
  __shared__ unsigned long long wbad[kThreads / 64];
  double acc = 0.0;
  uint32_t bad = 0;
  int t = 0;
  for (long long tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    while (tile >= table[t + 1].tile0) ++t;
    const Entry e = table[t];
    stats_tile<GT, NT>(e, tile - e.tile0, acc, bad);
  }
  const int tid = threadIdx.x;
  acc = wave_sum_f64(acc);
  const unsigned long long b = wave_sum_u64(bad);
  if ((tid & 63) == 0) {
    wsum[tid >> 6] = acc;
    wbad[tid >> 6] = b;
  }
  __syncthreads();
  if (tid == 0) {
    double sacc = wsum[0];
    unsigned long long bacc = wbad[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
      sacc += wsum[w];
      bacc += wbad[w];
    }
    part_sum[blockIdx.x] = sacc;
    part_bad[blockIdx.x] = bacc;
  }
}

// One workgroup: the partials in index order, then the outputs.  The clip
// coefficient is min(1, max_norm / (sqrt(sumsq) + 1e-6)) in double (a NaN
// stays NaN), rounded once to binary32.
__global__ void __launch_bounds__(kThreads)
grad_stats_finalize(const double* __restrict__ part_sum, const unsigned long long* __restrict__ part_bad,
                    int nparts, double max_norm, double* sumsq, unsigned long long* nonfinite, float* clip) {
  __shared__ double wsum[kThreads / 64];
  __shared__ unsigned long long wbad[kThreads / 64];
  const int tid = threadIdx.x;
  double sacc = 0.0;
  unsigned long long bacc = 0;
  for (int i = tid; i < nparts; i += kThreads) {
    sacc += part_sum[i];
    bacc += part_bad[i];
  }
  sacc = wave_sum_f64(sacc);
  bacc = wave_sum_u64(bacc);
  if ((tid & 63) == 0) {
    wsum[tid >> 6] = sacc;
    wbad[tid >> 6] = bacc;
  }
  __syncthreads();
  if (tid == 0) {
    double total = wsum[0];
    unsigned long long nb = wbad[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
      total += wsum[w];
      nb += wbad[w];
    }
    *sumsq = total;
    if (nonfinite != nullptr) *nonfinite = nb;
    if (clip != nullptr) {
      const double coef = max_norm / (__builtin_sqrt(total) + 1e-6);
      *clip = coef != coef ? (float)coef : (float)(coef < 1.0 ? coef : 1.0);
    }
  }
}

// ---------------------------------------------------------------------------
// Exports for tests: every code of every lane, and the square root, on the
// device.

__global__ void __launch_bounds__(kThreads) sqrt_kernel(const float* in, float* out, long long n) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n; i += (long long)gridDim.x * kThreads)
    out[i] = sqrt_rn(in[i]);
}

__global__ void __launch_bounds__(kThreads)
codec_kernel(int lane_kind, int dir, const void* in, void* out, long long n) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n; i += (long long)gridDim.x * kThreads) {
    if (dir == 0) {
      const float x = static_cast<const float*>(in)[i];
      uint32_t c = lane_kind == 0   ? e4_encode_m(x)
                   : lane_kind == 1 ? e4_encode_r(x)
                   : lane_kind == 2 ? f16_encode(x)
                                    : bf16_encode(x);
      static_cast<uint16_t*>(out)[i] = (uint16_t)c;
    } else {
      const uint32_t c = static_cast<const uint16_t*>(in)[i];
      float x = lane_kind == 0   ? e4_decode_m(c)
                : lane_kind == 1 ? e4_decode_r(c << 16)
                : lane_kind == 2 ? f16_decode(c)
                                 : __uint_as_float(c << 16);
      static_cast<float*>(out)[i] = x;
    }
  }
}

}  // namespace pa
