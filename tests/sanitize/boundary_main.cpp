// boundary_main.cpp -- drives the library's host-side argument checks and
// launch planning (include/fa.h) in a build instrumented with AddressSanitizer
// and UndefinedBehaviorSanitizer.  Built with the host sources of the library
// (fa_api.cpp, fa_launch.cpp); the device-side launch functions are stubbed
// out here, since no call below reaches a launch: every call is invalid, or
// the host-only plan query.  Exits 0 when every status matches.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "fa.h"
#include "fa_kernel.h"

extern "C" const unsigned char fa_hsaco_data[16] = {0};
extern "C" const unsigned long fa_hsaco_size = 16;

namespace fa {
hipError_t launch_combine(DType, const float*, const float*, void*, float*, int, int, int, int, int,
                          hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_tile(const LaunchArgs&, bool, bool, int, float*, float*) { return hipErrorInvalidValue; }
hipError_t launch_bwd_delta(const BwdLaunchArgs&) { return hipErrorInvalidValue; }
hipError_t launch_bwd_wide(const BwdLaunchArgs&) { return hipErrorInvalidValue; }
}  // namespace fa

static int failures = 0;
#define EXPECT(expr, want)                                                              \
  do {                                                                                  \
    int got_ = (expr);                                                                  \
    if (got_ != (want)) {                                                               \
      fprintf(stderr, "line %d: %s = %d, expected %d\n", __LINE__, #expr, got_, (want)); \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

int main() {
  // fake, 16-byte-aligned, far-apart device addresses; never dereferenced
  void* Q = (void*)(uintptr_t)(1ull << 40);
  void* K = (void*)(uintptr_t)(2ull << 40);
  void* V = (void*)(uintptr_t)(3ull << 40);
  void* O = (void*)(uintptr_t)(4ull << 40);
  float* L = (float*)(uintptr_t)(5ull << 40);
  void* W = (void*)(uintptr_t)(6ull << 40);
  void* G = (void*)(uintptr_t)(7ull << 40);
  void* DQ = (void*)(uintptr_t)(8ull << 40);
  void* DK = (void*)(uintptr_t)(9ull << 40);
  void* DV = (void*)(uintptr_t)(10ull << 40);

  // malformed arguments
  EXPECT(fa_fwd(nullptr, K, V, O, L, 1, 128, 128, 4, 2, 128, 1, 0.1f, 0), FA_ERR_INVALID);
  EXPECT(fa_fwd(Q, K, V, O, L, 0, 128, 128, 4, 2, 128, 1, 0.1f, 0), FA_ERR_INVALID);
  EXPECT(fa_fwd(Q, K, V, O, L, 1, 128, 128, 3, 2, 128, 1, 0.1f, 0), FA_ERR_INVALID);
  EXPECT(fa_fwd(Q, K, V, O, L, 1, 128, 128, 4, 2, 128, 2, 0.1f, 0), FA_ERR_INVALID);
  EXPECT(fa_fwd(Q, K, V, O, L, 1, 128, 128, 4, 2, 128, 1, __builtin_nanf(""), 0), FA_ERR_INVALID);
  EXPECT(fa_fwd((char*)Q + 8, K, V, O, L, 1, 128, 128, 4, 2, 128, 1, 0.1f, 0), FA_ERR_INVALID);
  EXPECT(fa_fwd(Q, K, V, Q, L, 1, 128, 128, 4, 2, 128, 1, 0.1f, 0), FA_ERR_INVALID);
  // sizes whose products overflow 64 bits, and the largest ints
  EXPECT(fa_fwd(Q, K, V, O, L, 2147483647, 2147483647, 2147483647, 2147483647, 1, 128, 1, 0.1f, 0),
         FA_ERR_INVALID);
  EXPECT(fa_fwd_f16(Q, K, V, O, L, 1, 2147483647, 2147483647, 1, 1, 64, 0, 0.1f, 0),
         FA_ERR_UNSUPPORTED);
  // not implemented
  EXPECT(fa_fwd(Q, K, V, O, L, 1, 128, 128, 4, 2, 96, 1, 0.1f, 0), FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd(Q, K, V, O, L, 1, 128, 128, 4, 2, 128, 1, -0.1f, 0), FA_ERR_UNSUPPORTED);
  EXPECT(fa_fwd(Q, K, V, O, L, 1, 128, 65536 * 64, 4, 2, 128, 1, 0.1f, 0), FA_ERR_UNSUPPORTED);
  // workspace entry
  EXPECT(fa_fwd_ws(2, Q, K, V, O, L, 1, 128, 128, 4, 2, 128, 1, 0.1f, W, 1024, 0), FA_ERR_INVALID);
  EXPECT(fa_fwd_ws(0, Q, K, V, O, L, 1, 128, 128, 4, 2, 128, 1, 0.1f, (char*)W + 4, 1024, 0),
         FA_ERR_INVALID);
  EXPECT(fa_fwd_ws(0, Q, K, V, O, L, 1, 128, 128, 4, 2, 128, 1, 0.1f, Q, 1024, 0), FA_ERR_INVALID);
  EXPECT(fa_fwd_ws(0, Q, K, V, O, L, 1, 128, 128, 4, 2, 128, 1, 0.1f, W, 0, 0), FA_ERR_INVALID);
  // backward
  EXPECT(fa_bwd(0, Q, K, V, O, L, G, DQ, DK, DV, 1, 128, 128, 4, 2, 128, 1, 0.1f, nullptr, 0, 0),
         FA_ERR_WORKSPACE);
  EXPECT(fa_bwd(0, Q, K, V, O, L, G, DQ, DK, DV, 1, 128, 128, 4, 2, 128, 1, 0.1f, W, 8 * 4 * 128 - 1, 0),
         FA_ERR_WORKSPACE);
  EXPECT(fa_bwd(0, Q, K, V, O, L, G, DQ, DK, DK, 1, 128, 128, 4, 2, 128, 1, 0.1f, W, 1 << 20, 0),
         FA_ERR_INVALID);
  EXPECT(fa_bwd(0, Q, K, V, O, nullptr, G, DQ, DK, DV, 1, 128, 128, 4, 2, 128, 1, 0.1f, W, 1 << 20, 0),
         FA_ERR_INVALID);
  EXPECT(fa_bwd(0, Q, K, V, O, L, G, DQ, DK, DV, 1, 128, 128, 4, 2, 96, 1, 0.1f, W, 1 << 20, 0),
         FA_ERR_UNSUPPORTED);
  EXPECT(fa_bwd(3, Q, K, V, O, L, G, DQ, DK, DV, 1, 128, 128, 4, 2, 128, 1, 0.1f, W, 1 << 20, 0),
         FA_ERR_INVALID);
  // one batch slice of k (2^20 keys x 8 heads x 128 dims x 2 bytes) at 2 GiB
  EXPECT(fa_bwd(0, Q, K, V, O, L, G, DQ, DK, DV, 1, 128, 1 << 20, 8, 8, 128, 0, 0.1f, W, 1 << 20, 0),
         FA_ERR_UNSUPPORTED);

  // the plan over a sweep of sizes (host only)
  int kern, ranges;
  size_t ws;
  const int sizes[] = {1, 2, 17, 63, 64, 65, 200, 511, 512, 513, 1000, 4096, 32768, 1 << 20};
  for (int sq : sizes)
    for (int skv : sizes)
      for (int hq : {1, 8, 64, 256})
        for (int d : {64, 128, 192, 256})
          for (int c = 0; c < 2; ++c)
            for (int w = 0; w < 2; ++w) {
              EXPECT(fa_fwd_plan(2, sq, skv, hq, hq > 4 ? hq / 4 : 1, d, c, 256, w, &kern, &ranges, &ws),
                     FA_OK);
              if (ranges < 1 || ranges > 64 || (ranges > 1 && ws == 0) || (ranges == 1 && ws != 0)) {
                fprintf(stderr, "plan sq %d skv %d hq %d d %d: ranges %d ws %zu\n", sq, skv, hq, d,
                        ranges, ws);
                ++failures;
              }
            }
  EXPECT(fa_fwd_plan(1, 1, 1, 1, 1, 128, 0, 256, 1, nullptr, &ranges, &ws), FA_ERR_INVALID);
  for (int s = -5; s <= 1; ++s) {
    const char* m = fa_strerror(s);
    if (!m || !strlen(m)) ++failures;
  }
  printf("%s (%d failures)\n", failures ? "FAIL" : "OK", failures);
  return failures ? 1 : 0;
}
