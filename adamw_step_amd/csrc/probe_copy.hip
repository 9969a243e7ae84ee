// probe_copy.hip -- bandwidth probes used by the benchmark (libpa_probe.so).
//
// Not part of the optimizer: a plain 16-byte-vector copy of a known number
// of bytes (to calibrate the HBM byte counters, and as the copy ceiling) and
// a probe with the packed step's traffic shape, three 16-byte streams read
// and two written per thread-iteration (12 bytes in, 8 out per element),
// with no arithmetic to speak of.

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

}  // namespace

extern "C" {

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
