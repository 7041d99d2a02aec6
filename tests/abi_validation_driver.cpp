// Host-side driver for the sanitizer build of the C ABI's validation layer:
// every call below fails validation (or is an empty batch), which returns
// before the first HIP call, so it runs without a GPU.  Built and run by
// tests/test_host_sanitizers.py with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code; any report fails the test.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "muon.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
    ++failures;
  }
}

int main() {
  char* W = reinterpret_cast<char*>(0x10000000);
  char* G = reinterpret_cast<char*>(0x20000000);
  float* M = reinterpret_cast<float*>(0x30000000);
  char* WS = reinterpret_cast<char*>(0x40000000);
  const double a = 3.4445, b = -4.775, c = 2.0315;
  const double inf = 1.0 / 0.0, nan = 0.0 / 0.0;

  // workspace sizes, including shapes whose products overflow 64 bits
  expect(muon_workspace_bytes(1, 0, 5, 0) == 0, 1, "ws rows 0");
  expect(muon_workspace_bytes(-1, 5, 5, 0) == 0, 1, "ws count -1");
  expect(muon_workspace_bytes(1, 5, 5, 9) == 0, 1, "ws dtype");
  expect(muon_workspace_bytes(INT64_MAX, MUON_MAX_DIM, MUON_MAX_DIM, 0) == 0, 1, "ws overflow");
  expect(muon_workspace_bytes(7, 3072, 768, 1) > 0, 1, "ws valid");

  // muon_step: every argument error
  expect(muon_step(nullptr, G, M, 64, 128, 0, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "null W");
  expect(muon_step(W, G, M, 0, 128, 0, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr, nullptr),
         MUON_ERR_INVALID_SHAPE, "rows 0");
  expect(muon_step(W, G, M, 64, MUON_MAX_DIM + 1, 0, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr,
                   nullptr), MUON_ERR_INVALID_SHAPE, "cols too large");
  expect(muon_step(W, G, M, 64, 128, 5, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr, nullptr),
         MUON_ERR_UNSUPPORTED_DTYPE, "dtype");
  expect(muon_step(W, G, M, 64, 128, 0, nan, 0.95, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "lr nan");
  expect(muon_step(W, G, M, 64, 128, 0, 0.02, inf, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "momentum inf");
  expect(muon_step(W, G, M, 64, 128, 0, 0.02, 0.95, 0.1, -1, a, b, c, 0, WS, 1 << 30, nullptr, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "ns -1");
  expect(muon_step(W, G, M, 64, 128, 0, 0.02, 0.95, 0.1, MUON_MAX_NS_STEPS + 1, a, b, c, 0, WS, 1 << 30,
                   nullptr, nullptr), MUON_ERR_INVALID_ARGUMENT, "ns too many");
  expect(muon_step(W, G, M, 64, 128, 0, 0.02, 0.95, 0.1, 5, a, b, c, 77, WS, 1 << 30, nullptr, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "variant");
  expect(muon_step(W, G, M, 64, 128, 0, 0.02, 0.95, 0.1, 5, a, b, c, 0, nullptr, 1 << 30, nullptr, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "null workspace");
  expect(muon_step(W, G, M, 64, 128, 0, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 16, nullptr, nullptr),
         MUON_ERR_WORKSPACE_TOO_SMALL, "workspace small");
  expect(muon_step(W, W + 64, M, 64, 128, 0, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "W and G overlap");
  expect(muon_step(W, G, M, 64, 128, 0, 0.02, 0.95, 0.1, 5, a, b, c, 0, W + 16, 1 << 30, nullptr, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "workspace overlaps W");

  // batched and grouped: counts, both or neither form, overflowing products
  expect(muon_step_batched(nullptr, nullptr, nullptr, 0, 64, 64, 1, 0.02, 0.95, 0.1, 5, a, b, c, 0, nullptr, 0,
                           nullptr, nullptr), MUON_OK, "batched empty");
  expect(muon_step_batched(nullptr, nullptr, nullptr, -1, 64, 64, 1, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS,
                           1 << 30, nullptr, nullptr), MUON_ERR_INVALID_ARGUMENT, "batched count -1");
  std::vector<muon_group> gs(11);
  for (size_t i = 0; i < gs.size(); ++i) {
    gs[i] = muon_group{int64_t(1 + i), int64_t(64 + 3 * i), int64_t(96 + 5 * i), nullptr, nullptr, nullptr,
                       W + (i << 24), G + (i << 24), M + (i << 22)};
  }
  expect(muon_workspace_bytes_grouped(gs.data(), int(gs.size()), 1) > 0, 1, "grouped ws");
  expect(muon_step_grouped(gs.data(), int(gs.size()), 1, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 16, nullptr,
                           nullptr), MUON_ERR_WORKSPACE_TOO_SMALL, "grouped workspace small");
  gs[10].W_table = reinterpret_cast<void* const*>(W);   // both forms in one group
  expect(muon_step_grouped(gs.data(), int(gs.size()), 1, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr,
                           nullptr), MUON_ERR_INVALID_ARGUMENT, "grouped both forms");
  gs[10].W_table = nullptr;
  gs[3].count = INT64_MAX / 2;
  expect(muon_step_grouped(gs.data(), int(gs.size()), 1, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr,
                           nullptr), MUON_ERR_INVALID_SHAPE, "grouped count overflow");
  gs[3].count = 2;
  gs[5].rows = MUON_MAX_DIM;
  gs[5].cols = MUON_MAX_DIM;
  gs[5].count = int64_t(1) << 40;
  expect(muon_step_grouped(gs.data(), int(gs.size()), 1, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr,
                           nullptr), MUON_ERR_INVALID_SHAPE, "grouped too many blocks");
  expect(muon_step_grouped(nullptr, 3, 1, 0.02, 0.95, 0.1, 5, a, b, c, 0, WS, 1 << 30, nullptr, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "grouped null array");
  expect(muon_step_grouped_noalloc(gs.data(), int(gs.size()), 1, 0.02, 0.95, 0.1, 5, a, b, c, 0, nullptr,
                                   nullptr), MUON_ERR_INVALID_SHAPE, "noalloc too many blocks");
  muon_group big{8, 1024, 4096, nullptr, nullptr, nullptr, W, G, M};
  expect(muon_step_grouped_noalloc(&big, 1, 1, 0.02, 0.95, 0.1, 5, a, b, c, 0, nullptr, nullptr),
         MUON_ERR_WORKSPACE_TOO_SMALL, "noalloc beyond its array");

  // AdamW
  expect(muon_adamw_step(W, G, M, M + (1 << 20), 1000, 1, 0.01, 1.0, 0.95, 1e-10, 0.0, 1, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "adamw beta1 1");
  expect(muon_adamw_step(W, G, M, M + (1 << 20), 1000, 1, 0.01, 0.8, 0.95, -1.0, 0.0, 1, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "adamw eps < 0");
  expect(muon_adamw_step(W, G, M, M + (1 << 20), 1000, 1, 0.01, 0.8, 0.95, 1e-10, 0.0, 0, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "adamw step 0");
  expect(muon_adamw_step(W, G, M, M + (1 << 20), -5, 1, 0.01, 0.8, 0.95, 1e-10, 0.0, 1, nullptr),
         MUON_ERR_INVALID_SHAPE, "adamw n < 0");
  expect(muon_adamw_step(W, G, M, M + (1 << 20), 0, 1, 0.01, 0.8, 0.95, 1e-10, 0.0, 1, nullptr), MUON_OK,
         "adamw empty");
  std::vector<muon_adamw_tensor> ts(40);
  for (size_t i = 0; i < ts.size(); ++i)
    ts[i] = muon_adamw_tensor{W + (i << 20), G + (i << 20), M + (i << 20), M + (int64_t(1) << 26) + (i << 20),
                              1000, 0.01, 0.001};
  ts[39].P = ts[0].P;   // two tensors share their parameters
  expect(muon_adamw_step_grouped(ts.data(), int64_t(ts.size()), 1, 0.8, 0.95, 1e-10, 3, nullptr),
         MUON_ERR_INVALID_ARGUMENT, "adamw grouped overlap");

  // names and profile arguments
  for (int s = -2; s < 8; ++s)
    if (!muon_status_string(s)) ++failures;
  for (int p = -1; p <= MUON_NUM_PHASES; ++p)
    if (!muon_phase_name(p)) ++failures;
  expect(muon_profile_read(nullptr, nullptr, 3), MUON_ERR_INVALID_ARGUMENT, "profile null");

  std::printf("%s\n", failures ? "FAILED" : "ALL_VALIDATION_CASES_OK");
  return failures ? 1 : 0;
}
