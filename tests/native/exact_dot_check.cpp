// Host build of the library's exact dot-product sign (exact_dot.h, the same
// header the HIP kernels include), for the CPU tests: compiled with g++ by
// tests/test_exact_dot.py and called through ctypes.
#include <stdint.h>
#include <string.h>

#include "exact_dot.h"

static double bf16_value(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return static_cast<double>(f);
}

extern "C" int hst_check_dot_nonneg_f32(const float* a, const float* b, int n) {
  uint64_t w[hst::kExactLimbs];
  return hst::exact_sum_nonneg(
             [&](int c) { return static_cast<double>(a[c]) * static_cast<double>(b[c]); }, n, w)
             ? 1
             : 0;
}

extern "C" int hst_check_dot_nonneg_bf16(const uint16_t* a, const uint16_t* b, int n) {
  uint64_t w[hst::kExactLimbs];
  return hst::exact_sum_nonneg([&](int c) { return bf16_value(a[c]) * bf16_value(b[c]); }, n, w) ? 1 : 0;
}

// The accumulator's words after summing the products (for checks of the
// fixed-point value itself).
extern "C" void hst_check_dot_words_f32(const float* a, const float* b, int n, uint64_t* out) {
  hst::exact_sum_nonneg([&](int c) { return static_cast<double>(a[c]) * static_cast<double>(b[c]); }, n,
                        out);
}
