// kernels.hpp -- gfx950 kernels of the packed-AdamW step.
//
// Elementwise modes (packed E4, packed FP16, FP32): one persistent launch
// walks a table of tensors cut into 4096-element tiles.  Each thread moves
// 16-byte vectors of parameter, gradient and state (one read and one write
// per word), keeps the whole update in registers, and never touches LDS.
// The table is read with scalar loads; a workgroup's tensor cursor only moves
// forward, so finding the tensor of a tile costs nothing per element.
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
// each rounded once).
struct Scalars {
  float beta1, one_m_beta1, beta2, one_m_beta2;
  float bc2, lr_over_bc1, decay, eps;
  float beta1_x2p112;   // beta1 * 2^112, exact (pairs with e4_decode_m_unscaled)
  float pad_;
  double inv_bc2;       // 1/bc2 rounded to double, for the exact quotient v'/bc2
};

// One tensor of an elementwise launch.  Every buffer of a tensor shares one
// 16-byte phase; `phase` is that phase in elements, so element i sits at
// virtual index i + phase and virtual indices 4k..4k+3 form one aligned
// 16-byte vector.
struct Entry {
  float* p;
  const float* g;
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
constexpr int kTile = kThreads * 4 * kUnroll;   // elements per tile
constexpr int kBlock = 2048;                    // blockwise quantisation block

enum { kModeFp32 = 0, kModeE4 = 1, kModeF16 = 2 };

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
template <int MODE>
__device__ __forceinline__ void scalar_elem(const Entry& e, long long i, const Scalars& s, uint32_t& bad) {
  float p = e.p[i];
  const float g = e.g[i];
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
  e.p[i] = p;
}

// Tile `tile` (local to tensor e).
template <int MODE>
__device__ __forceinline__ void run_tile(const Entry& e, long long tile, const Scalars& s, uint32_t& bad) {
  const long long v0 = tile * kTile;
  const long long vend = e.n + e.phase;
  const int tid = threadIdx.x;
  if (v0 >= e.phase && v0 + kTile <= vend) {
    // Whole tile inside the tensor: unguarded 16-byte vectors.
    const long long q0 = v0 / 4 + tid;
    f32x4* P = reinterpret_cast<f32x4*>(e.p - e.phase);
    const f32x4* G = reinterpret_cast<const f32x4*>(e.g - e.phase);
    if constexpr (MODE == kModeFp32) {
      f32x4* M = reinterpret_cast<f32x4*>(static_cast<float*>(e.s0) - e.phase);
      f32x4* V = reinterpret_cast<f32x4*>(e.s1 - e.phase);
      f32x4 p[kUnroll], g[kUnroll], m[kUnroll], v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const long long q = q0 + (long long)u * kThreads;
        p[u] = stream_load(P + q);
        g[u] = stream_load(G + q);
        m[u] = stream_load(M + q);
        v[u] = stream_load(V + q);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float pk = p[u][k], mk = m[u][k], vk = v[u][k];
          fp32_elem(pk, g[u][k], mk, vk, s, bad);
          p[u][k] = pk;
          m[u][k] = mk;
          v[u][k] = vk;
        }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const long long q = q0 + (long long)u * kThreads;
        stream_store(P + q, p[u]);
        stream_store(M + q, m[u]);
        stream_store(V + q, v[u]);
      }
    } else {
      u32x4* W = reinterpret_cast<u32x4*>(static_cast<uint32_t*>(e.s0) - e.phase);
      f32x4 p[kUnroll], g[kUnroll];
      u32x4 w[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const long long q = q0 + (long long)u * kThreads;
        p[u] = stream_load(P + q);
        g[u] = stream_load(G + q);
        w[u] = stream_load(W + q);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float pk = p[u][k];
          w[u][k] = packed_elem<MODE>(pk, g[u][k], w[u][k], s, bad);
          p[u][k] = pk;
        }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const long long q = q0 + (long long)u * kThreads;
        stream_store(P + q, p[u]);
        stream_store(W + q, w[u]);
      }
    }
  } else {
    // Ragged tile (first tile of a misaligned tensor, or the last one).
    for (int u = 0; u < kUnroll; ++u) {
      const long long vb = v0 + ((long long)u * kThreads + tid) * 4;
      for (int k = 0; k < 4; ++k) {
        const long long vi = vb + k;
        if (vi >= e.phase && vi < vend) scalar_elem<MODE>(e, vi - e.phase, s, bad);
      }
    }
  }
}

__device__ __forceinline__ void flush_count(uint32_t bad, unsigned long long* counter) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) bad += __shfl_xor(bad, off, 64);
  if ((threadIdx.x & 63) == 0 && bad != 0u) atomicAdd(counter, (unsigned long long)bad);
}

// Persistent multi-tensor launch.  table[count].tile0 holds the total tile
// count (a sentinel), so the cursor never runs past the table.
template <int MODE, bool COUNT>
__global__ void __launch_bounds__(kThreads)
elementwise_list(const Entry* __restrict__ table, long long total_tiles, Scalars s,
                 unsigned long long* nonfinite) {
  uint32_t bad = 0;
  int t = 0;
  for (long long tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) {
    while (tile >= table[t + 1].tile0) ++t;
    const Entry e = table[t];
    run_tile<MODE>(e, tile - e.tile0, s, bad);
  }
  if constexpr (COUNT) flush_count(bad, nonfinite);
}

// Single tensor, its entry passed by value (no table in device memory).
template <int MODE, bool COUNT>
__global__ void __launch_bounds__(kThreads)
elementwise_one(Entry e, long long total_tiles, Scalars s, unsigned long long* nonfinite) {
  uint32_t bad = 0;
  for (long long tile = blockIdx.x; tile < total_tiles; tile += gridDim.x) run_tile<MODE>(e, tile, s, bad);
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

// The 255 midpoints are kept in LDS in breadth-first (Eytzinger) order:
// node t has children 2t+1 and 2t+2, and an in-order walk of the 255 nodes
// gives the midpoints ascending.  Level l of the tree is the 2^l consecutive
// entries starting at 2^l - 1, so every step of a search reads from one
// short contiguous run of LDS words (few bank conflicts), unlike a bisection
// of the sorted array whose late steps all land in a handful of banks.
// Node t at level l, position p within the level, holds sorted midpoint
// (2p + 1) * 2^(7 - l) - 1.
__device__ __forceinline__ int eytzinger_sorted_index(int t) {
  const int l = 31 - __builtin_clz(t + 1);   // level of node t
  const int p = t + 1 - (1 << l);            // position within the level
  return (2 * p + 1) * (1 << (7 - l)) - 1;
}

// Number of midpoints strictly below c (ties go to the lower map entry):
// descend right exactly when the node's midpoint is below c; the leaf
// reached, counted from the left, is that number.  NaN is ordered above
// every number.
__device__ __forceinline__ uint32_t search_mid(const float* tree, float c) {
  uint32_t t = 0;
#pragma unroll
  for (int level = 0; level < 8; ++level) t = 2 * t + 1 + (tree[t] < c ? 1u : 0u);
  return (c != c) ? 255u : t - 255u;
}

// c / d for the block normaliser d (a positive normal binary32): the double
// product with rd = 1/d rounded to double, rounded once to binary32, is the
// correctly rounded quotient (the quotient of two binary32 numbers is either
// one itself or at least 2^-49 relative away from every binary32 midpoint,
// while the product is within 2^-52).  The one case that argument leaves
// open is a quotient exactly on a midpoint of the subnormal range, so
// nonzero products below the normal range take the hardware division
// instead (a zero product is exact: x is zero or d is Inf).
__device__ __forceinline__ float div_block(float x, float d, double rd) {
  const double q = (double)x * rd;
  float c = (float)q;
  if (__builtin_expect(q != 0.0 && __builtin_fabs(q) < 0x1p-126, 0)) c = __fdiv_rn(x, d);
  return c;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = max(x, (uint32_t)__shfl_xor((int)x, off, 64));
  return x;
}

template <bool COUNT>
__global__ void __launch_bounds__(kThreads)
blockwise_kernel(BlockwiseArgs a, Scalars s, unsigned long long* nonfinite) {
  __shared__ float lut_m[256], lut_v[256], tree_m[256], tree_v[256];
  __shared__ uint32_t wave_max[2][kThreads / 64];
  const int tid = threadIdx.x;
  lut_m[tid] = a.qmap_m[tid];
  lut_v[tid] = a.qmap_v[tid];
  __syncthreads();
  if (tid < 255) {
    // midpoint j = (q_j + q_{j+1}) * 0.5 in binary32, stored at its tree node
    const int j = eytzinger_sorted_index(tid);
    tree_m[tid] = (lut_m[j] + lut_m[j + 1]) * 0.5f;
    tree_v[tid] = (lut_v[j] + lut_v[j + 1]) * 0.5f;
  } else {
    tree_m[tid] = tree_v[tid] = __builtin_inff();
  }
  __syncthreads();

  // The 1e-30 lower clamp of the normaliser, as a binary32 bit pattern.
  const uint32_t floor_bits = __float_as_uint((float)1e-30);
  uint32_t bad = 0;
  for (long long b = blockIdx.x; b < a.nblocks; b += gridDim.x) {
    const long long base = b * kBlock;
    const float am = a.m_absmax[b];
    const float av = a.v_absmax[b];
    float m1[8], v1[8];
    uint32_t mc[2], vc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const long long e0 = base + h * 1024 + tid * 4;
      const float4 P = *reinterpret_cast<const float4*>(a.p + e0);
      const float4 G = *reinterpret_cast<const float4*>(a.g + e0);
      mc[h] = *reinterpret_cast<const uint32_t*>(a.m_code + e0);
      vc[h] = *reinterpret_cast<const uint32_t*>(a.v_code + e0);
      uint32_t bf[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float m = lut_m[(mc[h] >> (8 * k)) & 0xFFu] * am;
        const float v = lut_v[(vc[h] >> (8 * k)) & 0xFFu] * av;
        float p1;
        adamw(reinterpret_cast<const float*>(&P)[k], reinterpret_cast<const float*>(&G)[k], s.beta1 * m, v, s,
              p1, m1[h * 4 + k], v1[h * 4 + k]);
        bad += nonfinite3(p1, m1[h * 4 + k], v1[h * 4 + k]);
        bf[k] = bf16_encode(p1);
      }
      uint2 out;
      out.x = bf[0] | (bf[1] << 16);
      out.y = bf[2] | (bf[3] << 16);
      *reinterpret_cast<uint2*>(a.p_out + e0) = out;
    }
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
      wave_max[0][tid >> 6] = xm;
      wave_max[1][tid >> 6] = xv;
    }
    __syncthreads();
    uint32_t Am = wave_max[0][0], Av = wave_max[1][0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) {
      Am = max(Am, wave_max[0][w]);
      Av = max(Av, wave_max[1][w]);
    }
    __syncthreads();   // wave_max is rewritten by the next block
    const float dm = __uint_as_float(max(Am, floor_bits));
    const float dv = __uint_as_float(max(Av, floor_bits));
    const double rdm = 1.0 / (double)dm;   // correctly rounded double division
    const double rdv = 1.0 / (double)dv;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t cm = 0, cv = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cm |= search_mid(tree_m, div_block(m1[h * 4 + k], dm, rdm)) << (8 * k);
        cv |= search_mid(tree_v, div_block(v1[h * 4 + k], dv, rdv)) << (8 * k);
      }
      const long long e0 = base + h * 1024 + tid * 4;
      *reinterpret_cast<uint32_t*>(a.m_code + e0) = cm;
      *reinterpret_cast<uint32_t*>(a.v_code + e0) = cv;
    }
    if (tid == 0) {
      a.m_absmax[b] = __uint_as_float(Am);
      a.v_absmax[b] = __uint_as_float(Av);
    }
  }
  if constexpr (COUNT) flush_count(bad, nonfinite);
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
      uint32_t c = lane_kind == 0 ? e4_encode_m(x) : lane_kind == 1 ? e4_encode_r(x) : f16_encode(x);
      static_cast<uint16_t*>(out)[i] = (uint16_t)c;
    } else {
      const uint32_t c = static_cast<const uint16_t*>(in)[i];
      float x = lane_kind == 0 ? e4_decode_m(c) : lane_kind == 1 ? e4_decode_r(c << 16) : f16_decode(c);
      static_cast<float*>(out)[i] = x;
    }
  }
}

}  // namespace pa
