// probe_copy.hip -- bandwidth probes used by the benchmark (libpa_probe.so).
//
// Not part of the optimizer: a plain 16-byte-vector copy of a known number
// of bytes (to calibrate the HBM byte counters, and as the copy ceiling), a
// probe with the packed step's traffic shape, three 16-byte streams read
// and two written per thread-iteration (12 bytes in, 8 out per element),
// with no arithmetic to speak of, and the ceilings of the step's own access
// forms: nontemporal reads, nontemporal writes, and the step's traffic with
// those forms, with and without the step's amount of arithmetic.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads) copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        long long n16) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n16; i += (long long)gridDim.x * kThreads)
    dst[i] = src[i];
}

__global__ void __launch_bounds__(kThreads)
stream5_kernel(uint4* __restrict__ a, const uint4* __restrict__ b, uint4* __restrict__ c, long long n16) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n16; i += (long long)gridDim.x * kThreads) {
    uint4 x = a[i], y = b[i], z = c[i];
    x.x ^= y.x; x.y ^= y.y; x.z ^= y.z; x.w ^= y.w;
    z.x += y.x; z.y += y.y; z.z += y.z; z.w += y.w;
    a[i] = x;
    c[i] = z;
  }
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kU = 4;   // 16-byte vectors per stream per thread-iteration

// Nontemporal 16-byte reads of n16 vectors, summed so that nothing is dropped.
__global__ void __launch_bounds__(kThreads) read_nt_kernel(const f32x4* __restrict__ a, long long n16, float* sink) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const long long stride = (long long)gridDim.x * kThreads * kU;
  for (long long i = (long long)blockIdx.x * kThreads * kU + threadIdx.x; i < n16; i += stride)
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (i + u * kThreads < n16) acc += __builtin_nontemporal_load(a + i + u * kThreads);
  if (acc.x == 1234.5f && acc.y == 6.78f) sink[0] = acc.z;   // practically never
}

// Nontemporal 16-byte writes of n16 vectors.
__global__ void __launch_bounds__(kThreads) write_nt_kernel(f32x4* __restrict__ a, long long n16) {
  const f32x4 v = {1.f, 2.f, 3.f, 4.f};
  const long long stride = (long long)gridDim.x * kThreads * kU;
  for (long long i = (long long)blockIdx.x * kThreads * kU + threadIdx.x; i < n16; i += stride)
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (i + u * kThreads < n16) __builtin_nontemporal_store(v, a + i + u * kThreads);
}

// The packed step's traffic with its load and store forms: p, g, w read and
// p, w written in place, nontemporal 16-byte accesses, four vectors per
// stream in flight per thread, and K dependent multiply-adds (2K binary32
// instructions) per value on the two written streams.
template <int K>
__global__ void __launch_bounds__(kThreads) mix_kernel(f32x4* __restrict__ p, const f32x4* __restrict__ g,
                                                       f32x4* __restrict__ w, long long n16) {
  const long long stride = (long long)gridDim.x * kThreads * kU;
  for (long long i = (long long)blockIdx.x * kThreads * kU + threadIdx.x; i < n16; i += stride) {
    f32x4 x[kU], y[kU], z[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const bool ok = i + u * kThreads < n16;
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      x[u] = ok ? __builtin_nontemporal_load(p + i + u * kThreads) : zero;
      y[u] = ok ? __builtin_nontemporal_load(g + i + u * kThreads) : zero;
      z[u] = ok ? __builtin_nontemporal_load(w + i + u * kThreads) : zero;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        x[u] = x[u] * 0.999f + y[u];
        z[u] = z[u] * 1.001f - y[u];
      }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (i + u * kThreads < n16) {
        __builtin_nontemporal_store(x[u] - 0.001f * y[u], p + i + u * kThreads);
        __builtin_nontemporal_store(z[u] * 0.9f + y[u], w + i + u * kThreads);
      }
  }
}

}  // namespace

extern "C" {

// Nontemporal read of n16 16-byte vectors (16-byte aligned); sink: one
// device float.  Returns 0 or -1.
int pa_probe_read(const void* a, size_t n16, void* sink, int grid, void* stream) {
  if (!a || !sink || grid < 1 || (reinterpret_cast<uintptr_t>(a) & 15)) return -1;
  hipLaunchKernelGGL(read_nt_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const f32x4*>(a), (long long)n16, static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// Nontemporal write of n16 16-byte vectors (16-byte aligned).
int pa_probe_write(void* a, size_t n16, int grid, void* stream) {
  if (!a || grid < 1 || (reinterpret_cast<uintptr_t>(a) & 15)) return -1;
  hipLaunchKernelGGL(write_nt_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<f32x4*>(a), (long long)n16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The packed step's traffic (see mix_kernel) over n16 16-byte vectors per
// stream, with valu_per_value = 0 or 80 binary32 instructions per value.
int pa_probe_mix(void* p, const void* g, void* w, size_t n16, int valu_per_value, int grid, void* stream) {
  if (!p || !g || !w || grid < 1 || ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(g) |
                                      reinterpret_cast<uintptr_t>(w)) & 15))
    return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  f32x4* P = static_cast<f32x4*>(p);
  const f32x4* G = static_cast<const f32x4*>(g);
  f32x4* W = static_cast<f32x4*>(w);
  if (valu_per_value == 0)
    hipLaunchKernelGGL(mix_kernel<0>, dim3(grid), dim3(kThreads), 0, st, P, G, W, (long long)n16);
  else if (valu_per_value == 80)
    hipLaunchKernelGGL(mix_kernel<20>, dim3(grid), dim3(kThreads), 0, st, P, G, W, (long long)n16);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -1;
}


// Copy `bytes` (a multiple of 16, both pointers 16-byte aligned) from src to
// dst on `stream` with `grid` workgroups of 256 threads.  Returns 0 or -1.
int pa_probe_copy(const void* src, void* dst, size_t bytes, int grid, void* stream) {
  if (!src || !dst || bytes % 16 || grid < 1 || (reinterpret_cast<uintptr_t>(src) & 15) ||
      (reinterpret_cast<uintptr_t>(dst) & 15))
    return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), (long long)(bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// a[i] ^= b[i]; c[i] += b[i] over n16 16-byte vectors: 48 bytes read and 32
// written per vector, the packed step's 12 + 8 bytes per element.
int pa_probe_stream5(void* a, const void* b, void* c, size_t n16, int grid, void* stream) {
  if (!a || !b || !c || grid < 1) return -1;
  hipLaunchKernelGGL(stream5_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(a), static_cast<const uint4*>(b), static_cast<uint4*>(c), (long long)n16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // extern "C"
