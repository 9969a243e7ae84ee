// probe_copy.hip -- bandwidth probes used by the benchmark (libpa_probe.so).
//
// Not part of the optimizer: a plain 16-byte-vector copy of a known number
// of bytes (to calibrate the HBM byte counters), and the ceilings of the
// packed step's traffic on this HBM: a read-only stream, a write-only
// stream, and the step's own mix (three 16-byte streams read, two written in
// place, 12 bytes in and 8 out per element) with and without the step's
// amount of arithmetic.  Every probe takes one tile per workgroup in tile
// order, the order the step itself uses; the tile sizes are the fastest
// found for each form (reads: 8 KB per workgroup, nontemporal; writes: 4 KB
// per workgroup, plain stores; the mix: 16 KB per stream per workgroup,
// nontemporal both ways).  A copy through the HIP runtime (hipMemcpyAsync,
// device to device) is exported as well, as a reference that is not code
// of this library.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Workgroups of one probe launch: the dispatch packet counts work items in
// 32 bits, so larger streams take several launches.
constexpr long long kMaxGrid = 1LL << 22;

__global__ void __launch_bounds__(kThreads) copy_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                        long long n16) {
  for (long long i = (long long)blockIdx.x * kThreads + threadIdx.x; i < n16; i += (long long)gridDim.x * kThreads)
    dst[i] = src[i];
}

// Nontemporal reads of two vectors per thread, summed so nothing is dropped.
__global__ void __launch_bounds__(kThreads) read_kernel(const f32x4* __restrict__ a, long long n16, long long base,
                                                        float* sink) {
  const long long i = (base + blockIdx.x) * (2 * kThreads) + threadIdx.x;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (i < n16) acc += __builtin_nontemporal_load(a + i);
  if (i + kThreads < n16) acc += __builtin_nontemporal_load(a + i + kThreads);
  if (acc.x == 1234.5f && acc.y == 6.78f) sink[0] = acc.z;   // practically never
}

// One 16-byte store per thread.
__global__ void __launch_bounds__(kThreads) write_kernel(f32x4* __restrict__ a, long long n16, long long base) {
  const f32x4 v = {1.f, 2.f, 3.f, 4.f};
  const long long i = (base + blockIdx.x) * kThreads + threadIdx.x;
  if (i < n16) a[i] = v;
}

// The packed step's traffic: p, g, w read and p, w written in place, four
// vectors per stream per thread, nontemporal, and K dependent multiply-adds
// (2K binary32 instructions) per value on the two written streams.
template <int K>
__global__ void __launch_bounds__(kThreads) mix_kernel(f32x4* __restrict__ p, const f32x4* __restrict__ g,
                                                       f32x4* __restrict__ w, long long n16, long long base) {
  constexpr int kU = 4;
  const long long i = (base + blockIdx.x) * (kU * kThreads) + threadIdx.x;
  f32x4 x[kU], y[kU], z[kU];
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const long long j = i + (long long)u * kThreads;
    const bool ok = j < n16;
    x[u] = ok ? __builtin_nontemporal_load(p + j) : zero;
    y[u] = ok ? __builtin_nontemporal_load(g + j) : zero;
    z[u] = ok ? __builtin_nontemporal_load(w + j) : zero;
  }
#pragma unroll
  for (int u = 0; u < kU; ++u)
#pragma unroll
    for (int k = 0; k < K; ++k) {
      x[u] = x[u] * 0.999f + y[u];
      z[u] = z[u] * 1.001f - y[u];
    }
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const long long j = i + (long long)u * kThreads;
    if (j < n16) {
      __builtin_nontemporal_store(x[u] - 0.001f * y[u], p + j);
      __builtin_nontemporal_store(z[u] * 0.9f + y[u], w + j);
    }
  }
}

// Launches of `per` vectors per workgroup over n16 vectors.
template <typename F>
int tiles(long long n16, long long per, F&& launch) {
  const long long total = (n16 + per - 1) / per;
  for (long long base = 0; base < total; base += kMaxGrid) {
    const long long grid = total - base < kMaxGrid ? total - base : kMaxGrid;
    launch(dim3((unsigned)grid), base);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

bool a16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" {

// Nontemporal read of n16 16-byte vectors (16-byte aligned); sink: one
// device float.  Returns 0 or -1.
int pa_probe_read(const void* a, size_t n16, void* sink, void* stream) {
  if (!a || !sink || !a16(a)) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return tiles((long long)n16, 2 * kThreads, [&](dim3 grid, long long base) {
    hipLaunchKernelGGL(read_kernel, grid, dim3(kThreads), 0, st, static_cast<const f32x4*>(a), (long long)n16, base,
                       static_cast<float*>(sink));
  });
}

// Write of n16 16-byte vectors (16-byte aligned).
int pa_probe_write(void* a, size_t n16, void* stream) {
  if (!a || !a16(a)) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  return tiles((long long)n16, kThreads, [&](dim3 grid, long long base) {
    hipLaunchKernelGGL(write_kernel, grid, dim3(kThreads), 0, st, static_cast<f32x4*>(a), (long long)n16, base);
  });
}

// The packed step's traffic (see mix_kernel) over n16 16-byte vectors per
// stream, with valu_per_value = 0 or 80 binary32 instructions per value.
int pa_probe_mix(void* p, const void* g, void* w, size_t n16, int valu_per_value, void* stream) {
  if (!p || !g || !w || !a16(p) || !a16(g) || !a16(w)) return -1;
  if (valu_per_value != 0 && valu_per_value != 80) return -1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  f32x4* P = static_cast<f32x4*>(p);
  const f32x4* G = static_cast<const f32x4*>(g);
  f32x4* W = static_cast<f32x4*>(w);
  return tiles((long long)n16, 4 * kThreads, [&](dim3 grid, long long base) {
    if (valu_per_value == 0)
      hipLaunchKernelGGL(mix_kernel<0>, grid, dim3(kThreads), 0, st, P, G, W, (long long)n16, base);
    else
      hipLaunchKernelGGL(mix_kernel<20>, grid, dim3(kThreads), 0, st, P, G, W, (long long)n16, base);
  });
}

// Copy `bytes` (a multiple of 16, both pointers 16-byte aligned) from src to
// dst on `stream` with `grid` workgroups of 256 threads (the calibration
// copy of the byte counters).  Returns 0 or -1.
int pa_probe_copy(const void* src, void* dst, size_t bytes, int grid, void* stream) {
  if (!src || !dst || bytes % 16 || grid < 1 || !a16(src) || !a16(dst)) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), (long long)(bytes / 16));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// The HIP runtime's own device-to-device copy of `bytes` (not code of this
// library: a reference rate for one read and one write stream).
int pa_probe_runtime_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return -1;
  return hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, static_cast<hipStream_t>(stream)) == hipSuccess
             ? 0
             : -1;
}

}  // extern "C"
