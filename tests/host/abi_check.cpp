// Host-side run of the C ABI's argument validation and workspace sizing,
// linked against a copy of the library built with the host address and
// undefined-behaviour sanitizers: every call here is rejected (or is a
// no-op) before any device work, so no GPU is needed. Extreme sizes
// (negative, zero, INT64 extremes) must give a status or SIZE_MAX, never an
// overflow, an out-of-bounds access or a crash.
// Usage: abi_check. Prints "ok <checks>" or the first mismatch and exits 1.
#include <stdint.h>
#include <stdio.h>

#include "itl.h"

static int n_checks = 0;
static int n_fail = 0;

#define EXPECT(cond)                                                        \
  do {                                                                      \
    ++n_checks;                                                             \
    if (!(cond)) {                                                          \
      printf("failed: %s (line %d; last error: %s)\n", #cond, __LINE__,    \
             itl_last_error());                                             \
      ++n_fail;                                                             \
    }                                                                       \
  } while (0)

int main() {
  const int64_t big = INT64_MAX, small = INT64_MIN;
  void* p16 = (void*)(uintptr_t)256;  // never dereferenced: every call below fails validation first
  float* f16 = (float*)(uintptr_t)256;
  const int32_t* t16 = (const int32_t*)(uintptr_t)256;
  const int64_t sizes[] = {small, -1, 0, 1, 63, 64, 65, 4096, (int64_t)1 << 31, (int64_t)1 << 40, (int64_t)1 << 62, big};

  // workspace sizing: SIZE_MAX or a finite size, whatever the inputs
  for (int64_t a : sizes)
    for (int64_t b : sizes) {
      const size_t w1 = itl_lmhead_logprob_workspace_bytes(a, b);
      EXPECT(a >= 0 && b > 0 && a <= ((int64_t)1 << 31) && b <= ((int64_t)1 << 31) ? true : w1 == SIZE_MAX);
      const size_t w2 = itl_reinforce_zero_loss_workspace_bytes(a, (int32_t)(b > INT32_MAX ? -1 : b));
      (void)w2;
      for (int64_t d : sizes) {
        const size_t w3 = itl_reinforce_zero_backward_workspace_bytes(a, d, b, ITL_BF16);
        if (a < 0 || d <= 0 || b <= 0 || d % 64 != 0 || d >= ((int64_t)1 << 22)) EXPECT(w3 == SIZE_MAX);
        else if (a < ((int64_t)1 << 30) && b < ((int64_t)1 << 30)) EXPECT(w3 != SIZE_MAX && w3 < ((size_t)1 << 52));
      }
      (void)itl_mismatch_stats_workspace_bytes(a);
    }

  // the head entry points: bad shapes, dtypes and pointers are rejected
  for (int64_t n : sizes)
    for (int64_t d : sizes)
      for (int64_t v : sizes) {
        const bool bad = n < 0 || d <= 0 || v <= 0;
        itl_status s = itl_lmhead_logprob(nullptr, nullptr, ITL_BF16, n, d, v, nullptr, nullptr, nullptr, nullptr,
                                          0, nullptr);
        EXPECT(bad ? s == ITL_ERR_INVALID_ARG : s != ITL_OK || n == 0);
        s = itl_lmhead_logprob_keep_logits(nullptr, nullptr, ITL_F32, n, d, v, nullptr, nullptr, nullptr, nullptr,
                                           0, nullptr, 0, nullptr);
        EXPECT(bad ? s == ITL_ERR_INVALID_ARG : s != ITL_OK || n == 0);
        s = itl_lmhead_logprob_noalloc(nullptr, nullptr, ITL_BF16, n, d, v, nullptr, nullptr, nullptr, nullptr);
        EXPECT(bad ? s == ITL_ERR_INVALID_ARG : s != ITL_OK || n == 0);
        s = itl_reinforce_zero_backward(p16, nullptr, ITL_BF16, n, d, v, t16, f16, f16, f16, f16, p16, 0, nullptr);
        EXPECT(s != ITL_OK);
        s = itl_reinforce_zero_backward_from_logits(p16, p16, ITL_BF16, n, d, v, t16, f16, f16, nullptr, 0, f16,
                                                    f16, p16, 0, nullptr);
        EXPECT(n <= 0 ? true : s != ITL_OK);
        s = itl_lmhead_logprob_fp8(nullptr, nullptr, nullptr, nullptr, n, d, v, nullptr, nullptr, nullptr, nullptr, 0,
                                   nullptr);
        EXPECT(bad ? s == ITL_ERR_INVALID_ARG : s != ITL_OK || n == 0);
        s = itl_lmhead_logprob_mxfp4(nullptr, nullptr, nullptr, nullptr, n, d, v, nullptr, nullptr, nullptr, nullptr,
                                     0, nullptr);
        EXPECT(bad ? s == ITL_ERR_INVALID_ARG : s != ITL_OK || n == 0);
        s = itl_quantize_rows_fp8(nullptr, ITL_BF16, n, d, nullptr, nullptr, nullptr);
        EXPECT(n < 0 || d <= 0 ? s == ITL_ERR_INVALID_ARG : s != ITL_OK || n == 0);
        s = itl_quantize_rows_mxfp4(nullptr, ITL_BF16, n, d, nullptr, nullptr, nullptr);
        EXPECT(n < 0 || d <= 0 ? s == ITL_ERR_INVALID_ARG : s != ITL_OK || n == 0);
      }
  EXPECT(itl_lmhead_logprob(p16, p16, (itl_dtype)7, 4, 64, 10, t16, f16, nullptr, p16, 1 << 20, nullptr) ==
         ITL_ERR_UNSUPPORTED);

  // the loss, the advantage and the diagnostics
  for (int64_t n : sizes)
    for (int64_t r : sizes) {
      const int32_t r32 = (int32_t)(r > INT32_MAX || r < INT32_MIN ? -1 : r);
      itl_status s = itl_reinforce_zero_loss(nullptr, nullptr, nullptr, nullptr, r32, n, nullptr, nullptr, nullptr,
                                             nullptr, 0, nullptr);
      EXPECT(r32 < 0 || n < 0 ? s == ITL_ERR_INVALID_ARG
                              : (r32 == 0 ? s == ITL_OK || s == ITL_ERR_UNSUPPORTED : s != ITL_OK));
      s = itl_group_advantage(nullptr, nullptr, r32, r32, nullptr, nullptr);
      EXPECT(r32 < 0 ? s == ITL_ERR_INVALID_ARG : (r32 == 0 ? s == ITL_OK : s != ITL_OK));
      s = itl_mismatch_stats(nullptr, nullptr, nullptr, n, nullptr, nullptr, 0, nullptr);
      EXPECT(s != ITL_OK);
      if (n != 0) {  // (n == 0 would go on to the device)
        s = itl_mismatch_stats(nullptr, nullptr, nullptr, n, (double*)p16, nullptr, 0, nullptr);
        EXPECT(s != ITL_OK);
      }
      s = itl_check_inputs(nullptr, n, r, nullptr, r32 < 0 ? r32 : -1, nullptr);
      EXPECT(s == ITL_ERR_INVALID_ARG);
    }

  // status strings and the build description
  for (int k = -1; k <= 6; ++k) EXPECT(itl_status_string((itl_status)k) != nullptr);
  EXPECT(itl_build_info() != nullptr && itl_build_info()[0] != 0);
  EXPECT(itl_last_error() != nullptr);

  if (n_fail) return 1;
  printf("ok %d\n", n_checks);
  return 0;
}
