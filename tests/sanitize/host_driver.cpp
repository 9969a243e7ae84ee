// Drives the C ABI's host-side validation under AddressSanitizer and
// UndefinedBehaviorSanitizer, without a GPU: every call below is rejected
// before any device work, or fails cleanly at the first device query.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "../../include/pa.h"

int main() {
  pa_hyper h{1e-3, 0.9, 0.999, 1e-8, 0.01, nullptr};
  const uintptr_t F = 0x7F0000000000ull;   // never dereferenced
  auto P = [](uintptr_t a) { return reinterpret_cast<float*>(a); };
  int bad = 0;
  auto expect = [&](int got, int want, const char* what) {
    if (got != want) {
      std::printf("%s: got %d want %d\n", what, got, want);
      ++bad;
    }
  };
  expect(pa_step(7, P(F), P(F + 4096), reinterpret_cast<void*>(F + 8192), 64, &h, 1, nullptr), PA_ERR_ARG, "mode");
  expect(pa_step(1, P(F), P(F + 4096), reinterpret_cast<void*>(F + 8192), 64, &h, 0, nullptr), PA_ERR_ARG, "step");
  expect(pa_step(1, P(F + 2), P(F + 4098), reinterpret_cast<void*>(F + 8194), 64, &h, 1, nullptr), PA_ERR_ALIGN, "align");
  expect(pa_step(1, P(F), P(F + 4096), reinterpret_cast<void*>(F + 64), 64, &h, 1, nullptr), PA_ERR_ALIAS, "alias");
  pa_fp32_state fs{P(F + 65536), P(F + 65536 + 128)};
  expect(pa_step(0, P(F), P(F + 4096), &fs, 64, &h, 1, nullptr), PA_ERR_ALIAS, "fp32 alias");
  pa_blockwise_state bs{reinterpret_cast<uint8_t*>(F + (1 << 20)), P(F + (2 << 20)),
                        reinterpret_cast<uint8_t*>(F + (3 << 20)), P(F + (4 << 20)),
                        P(F + (5 << 20)), P(F + (6 << 20)), reinterpret_cast<uint16_t*>(F + (7 << 20))};
  expect(pa_step(3, P(F), P(F + (1 << 19)), &bs, 2049, &h, 1, nullptr), PA_ERR_SHAPE, "shape");
  expect(pa_step_typed(1, 1, 2, P(F), P(F + 4096), reinterpret_cast<void*>(F + 8192), 64, &h, 1, nullptr),
         PA_ERR_ARG, "typed pair");
  expect(pa_step_typed(1, 1, 1, P(F + 2), P(F + 4098), reinterpret_cast<void*>(F + 8200), 64, &h, 1, nullptr),
         PA_ERR_ALIGN, "typed phase");
  // a list with an overlap between two tensors' state
  std::vector<float*> ps{P(F), P(F + 4096)};
  std::vector<const float*> gs{P(F + 8192), P(F + 12288)};
  std::vector<void*> ss{reinterpret_cast<void*>(F + 16384), reinterpret_cast<void*>(F + 16384 + 64)};
  std::vector<size_t> ns{64, 64};
  int rc = pa_step_list(1, 2, ps.data(), gs.data(), ss.data(), ns.data(), &h, 1, nullptr);
  if (rc != PA_ERR_ALIAS && rc != PA_ERR_DEVICE) {   // without a GPU the device query may come first
    std::printf("list alias: got %d\n", rc);
    ++bad;
  }
  // gradient pre-pass: argument rules checked before any device work
  const void* gl[1] = {reinterpret_cast<void*>(F)};
  size_t gn[1] = {64};
  expect(pa_grad_stats_list(7, 1, gl, gn, 0.0, reinterpret_cast<double*>(F + 4096), nullptr, nullptr, nullptr),
         PA_ERR_ARG, "stats dtype");
  expect(pa_grad_stats_list(0, 1, gl, gn, 0.0, reinterpret_cast<double*>(F + 4100), nullptr, nullptr, nullptr),
         PA_ERR_ALIGN, "stats align");
  expect(pa_grad_stats_list(0, 1, gl, gn, 1.0, reinterpret_cast<double*>(F + 4096),
                            reinterpret_cast<unsigned long long*>(F + 4096), nullptr, nullptr),
         PA_ERR_ALIAS, "stats alias");
  // TurboAdam step: configuration and beta rules checked before any device work
  pa_turbo_state ts{1, 1, 0, reinterpret_cast<uint8_t*>(F + (1 << 21)), reinterpret_cast<uint16_t*>(F + (1 << 22)),
                    nullptr, reinterpret_cast<uint8_t*>(F + (1 << 23)), reinterpret_cast<uint16_t*>(F + (1 << 24)),
                    nullptr, P(F + (1 << 25))};
  pa_turbo_config tc{5, 1.1, 1, 0, 0, 0};
  float* tp[1] = {P(F)};
  const float* tg[1] = {P(F + (1 << 20))};
  size_t tn[1] = {4096};
  expect(pa_turbo_step_list(1, tp, tg, &ts, tn, &h, &tc, 1, reinterpret_cast<void*>(F + (1 << 26)), 1 << 20, nullptr),
         PA_ERR_ARG, "turbo bits");
  pa_turbo_config tcb{3, 1.1, 1, 96, 32, 0};
  expect(pa_turbo_step_list(1, tp, tg, &ts, tn, &h, &tcb, 1, reinterpret_cast<void*>(F + (1 << 26)), 1 << 20, nullptr),
         PA_ERR_ARG, "turbo block");
  pa_turbo_config tcg{6, 1.1, 1, 64, 128, 0};
  expect(pa_turbo_step_list(1, tp, tg, &ts, tn, &h, &tcg, 1, reinterpret_cast<void*>(F + (1 << 26)), 1 << 20, nullptr),
         PA_ERR_ARG, "turbo group");
  if (pa_turbo_layout_bytes(1, 1, 3, 32, 8, 1000) != 4 * 63 + 2 * 125 + 12 + 4 * 94 + 4 * 32) ++bad;
  pa_hyper hb{1e-3, 0.99, 0.98, 1e-8, 0.01, nullptr, nullptr, nullptr};
  pa_turbo_config tc4{4, 1.1, 1, 0, 0, 0};
  expect(pa_turbo_step_list(1, tp, tg, &ts, tn, &hb, &tc4, 1, reinterpret_cast<void*>(F + (1 << 26)), 1 << 20, nullptr),
         PA_ERR_ARG, "turbo betas");
  void* tpv[1] = {P(F)};
  const void* tgv[1] = {P(F + (1 << 20))};
  expect(pa_turbo_step_list_typed(PA_DT_F32, PA_DT_BF16, 1, tpv, tgv, &ts, tn, &h, &tc4, 1,
                                  reinterpret_cast<void*>(F + (1 << 26)), 1 << 20, nullptr),
         PA_ERR_ARG, "turbo typed pair");
  expect(pa_turbo_step_list_typed(PA_DT_BF16, PA_DT_BF16, 1, tpv, tgv, &ts, tn, &hb, &tc4, 1,
                                  reinterpret_cast<void*>(F + (1 << 26)), 1 << 20, nullptr),
         PA_ERR_ARG, "turbo typed betas");
  if (pa_turbo_state_bytes(1, 1, 4, 131072) != 106508 || pa_turbo_workspace_bytes(1, &ts, tn) != 136) ++bad;
  pa_format pf;
  for (int m = 0; m < 4; ++m) expect(pa_format_info(m, &pf), PA_OK, "format");
  expect(pa_format_info(9, &pf), PA_ERR_ARG, "format mode");
  if (pa_state_bytes(1, 1000) != 4000 || pa_state_bytes(0, 1000) != 8000) ++bad;
  for (int s = 1; s >= -8; --s) (void)pa_status_string(s);
  (void)pa_last_hip_error();
  pa_release_plans();
  std::printf("host driver %s\n", bad ? "FAILED" : "ok");
  return bad ? 1 : 0;
}
