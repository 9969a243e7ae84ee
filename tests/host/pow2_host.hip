// Host build of the GPU path's double-double level decision, for the CPU
// tests: pa::pow2_rn32_dd uses only IEEE double operations, so the host
// build gives what the device gives.  Built by the tests with hipcc
// (host side only, no contraction, as the library).
#include <stddef.h>

#include "pow2.hpp"

extern "C" void pow2_rn32_dd_host(const double* x, float* out, size_t n) {
  for (size_t i = 0; i < n; ++i) out[i] = pa::pow2_rn32_dd(x[i]);
}
