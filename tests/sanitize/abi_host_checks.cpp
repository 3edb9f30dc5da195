// Host-only exercise of the C ABI's argument validation and error paths, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code of plan.hip (see
// tests/test_host_sanitizers.py). Runs on a machine without a GPU: every call here must
// return its documented status without touching invalid memory. Exit status 0 = all
// statuses as expected; the sanitizers abort the process on a finding.
#include <cstdio>
#include <cstring>

#include "nys_attn.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    std::fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want,
                 nys_attn_last_error());
    ++failures;
  }
}

int main() {
  nys_attn_plan* plan = reinterpret_cast<nys_attn_plan*>(0x1);
  // create: every argument check, and *plan reset to NULL
  const int bad[][8] = {
      {1, 1, 64, 32, 8, 33, 6, -1}, {-1, 1, 64, 32, 8, 33, 6, 1}, {1, 1, 0, 32, 8, 33, 6, 1},
      {1, 1, 64, 32, 0, 33, 6, 1},  {1, 1, 64, 32, 128, 33, 6, 1}, {1, 1, 64, 32, 8, 32, 6, 1},
      {1, 1, 64, 32, 8, 33, -1, 1}, {1, 1, 64, 32, 8, 33, 101, 1}, {1, 1, 64, 0, 8, 33, 6, 1}};
  for (const auto& a : bad) {
    plan = reinterpret_cast<nys_attn_plan*>(0x1);
    expect("create (invalid)", nys_attn_create(&plan, a[0], a[1], a[2], a[3], a[4], a[5], a[6],
                                               static_cast<nys_dtype>(a[7])),
           NYS_E_ARG);
    if (plan != nullptr) {
      std::fprintf(stderr, "create left *plan set on failure\n");
      ++failures;
    }
  }
  expect("create (d = 48)", nys_attn_create(&plan, 1, 1, 64, 48, 8, 33, 6, NYS_BF16),
         NYS_E_UNSUPPORTED);
  expect("create (m = 512)", nys_attn_create(&plan, 1, 1, 1024, 32, 512, 33, 6, NYS_BF16),
         NYS_E_UNSUPPORTED);
  expect("create (NULL out)", nys_attn_create(nullptr, 1, 1, 64, 32, 8, 33, 6, NYS_BF16),
         NYS_E_ARG);
  // a valid shape reaches the device check: no device here
  const nys_status st = nys_attn_create(&plan, 2, 4, 512, 64, 64, 33, 6, NYS_BF16);
  if (st != NYS_E_DEVICE && st != NYS_OK) expect("create (no device)", st, NYS_E_DEVICE);
  if (st == NYS_OK) nys_attn_destroy(plan);
  // NULL plans
  int dummy[4] = {0, 0, 0, 0};
  expect("forward (NULL plan)",
         nys_attn_forward(nullptr, dummy, dummy, dummy, nullptr, dummy, nullptr), NYS_E_ARG);
  expect("forward_debug (NULL plan)",
         nys_attn_forward_debug(nullptr, dummy, dummy, dummy, nullptr, dummy, nullptr, nullptr),
         NYS_E_ARG);
  expect("forward_varlen (NULL plan)",
         nys_attn_forward_varlen(nullptr, dummy, dummy, dummy, nullptr, nullptr, dummy, nullptr,
                                 nullptr),
         NYS_E_ARG);
  expect("backward (NULL plan)",
         nys_attn_backward(nullptr, dummy, dummy, dummy, nullptr, nullptr, dummy, dummy, dummy,
                           dummy, nullptr, nullptr),
         NYS_E_ARG);
  expect("profile_enable (NULL plan)", nys_attn_profile_enable(nullptr, 4), NYS_E_ARG);
  int n_calls = 0;
  float ms[4];
  expect("profile_read (NULL plan)", nys_attn_profile_read(nullptr, ms, 1, &n_calls), NYS_E_ARG);
  if (nys_attn_workspace_bytes(nullptr) != 0) {
    std::fprintf(stderr, "workspace_bytes(NULL) != 0\n");
    ++failures;
  }
  nys_attn_destroy(nullptr);
  // the allocation-free forward validates before any device call
  expect("noalloc (bad dtype)",
         nys_attn_forward_noalloc(1, 1, 64, 32, 8, 33, 6, static_cast<nys_dtype>(7), dummy,
                                  dummy, dummy, nullptr, dummy, nullptr),
         NYS_E_ARG);
  expect("noalloc (m > 256)",
         nys_attn_forward_noalloc(1, 1, 1024, 32, 512, 33, 6, NYS_BF16, dummy, dummy, dummy,
                                  nullptr, dummy, nullptr),
         NYS_E_UNSUPPORTED);
  // projections and mixed-chunk attention: argument checks
  expect("proj_qkv (d = 48)",
         nys_proj_qkv(dummy, dummy, dummy, dummy, dummy, 1, 1, 64, 48, 64, nullptr),
         NYS_E_UNSUPPORTED);
  expect("proj_out (n = 0)", nys_proj_out(dummy, dummy, dummy, 1, 1, 0, 64, 64, nullptr),
         NYS_E_ARG);
  if (nys_flash_workspace_bytes(1, 1, 64, 64, 100, 0) != 0) {
    std::fprintf(stderr, "flash_workspace_bytes accepted chunk 100\n");
    ++failures;
  }
  if (nys_flash_workspace_bytes(2, 2, 1000, 64, 128, 1) == 0) {
    std::fprintf(stderr, "flash_workspace_bytes refused a valid shape\n");
    ++failures;
  }
  expect("flash (causal = 2)",
         nys_flash_attention(dummy, dummy, dummy, dummy, 1, 1, 64, 64, 64, 2, dummy, 64, nullptr),
         NYS_E_ARG);
  expect("flash (small workspace)",
         nys_flash_attention(dummy, dummy, dummy, dummy, 1, 1, 64, 64, 64, 0, dummy, 16, nullptr),
         NYS_E_ARG);
  if (std::strlen(nys_attn_last_error()) == 0) {
    std::fprintf(stderr, "last_error empty after a failure\n");
    ++failures;
  }
  std::printf("abi host checks: %d failure(s)\n", failures);
  return failures == 0 ? 0 : 1;
}
