// Exact sign of a sum of products of float32 values (bf16 values are float32
// values), for host and device code.
//
// The hashing steps set a bit when a projection is >= 0 (SOCKET overview
// page, "Core mechanism: soft LSH", item 1; binary codes alike).  Each
// product of two float32 values is exact in float64 (two 24-bit
// significands give at most 48 bits), and every such product is an integer
// multiple of 2^-298 (subnormal float32 values included) below 2^256 in
// magnitude.  So the sum is accumulated exactly in a fixed-point number:
// kExactLimbs 64-bit words of two's complement, lowest bit 2^kExactLsb
// (640 bits: from 2^-320 up to the sign at 2^319).  Adding a product shifts
// its integer significand into place and propagates the carry (or borrow)
// up the words; nothing is rounded and the length never grows, so the sign
// of the total is the sign of the top word, for any number of terms up to
// 2^31.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define HST_EXACT_HD __host__ __device__
#else
#define HST_EXACT_HD
#endif

namespace hst {

constexpr int kExactLimbs = 10;
constexpr int kExactLsb = -320;

// w += p.  p must be zero or an integer multiple of 2^kExactLsb below 2^287
// in magnitude (every product of two float32 values, summed up to 2^31
// times, is).
HST_EXACT_HD inline void exact_acc_add(uint64_t* w, double p) {
  const uint64_t u = __builtin_bit_cast(uint64_t, p);
  const uint64_t mant = u & 0xFFFFFFFFFFFFFull;
  const int ex = static_cast<int>((u >> 52) & 0x7ffu);
  if (ex == 0 && mant == 0) return;  // +-0
  uint64_t m = ex != 0 ? (mant | (1ull << 52)) : mant;
  int e = (ex != 0 ? ex : 1) - 1075;  // |p| = m * 2^e
  const int tz = __builtin_ctzll(m);
  m >>= tz;
  e += tz;
  const int sh = e - kExactLsb;  // bit offset of m's lowest bit; >= 0 by the precondition
  if (sh < 0 || sh + 53 > 64 * kExactLimbs - 1) return;  // outside the precondition
  const int i0 = sh >> 6, b = sh & 63;
  const uint64_t lo = m << b, hi = b != 0 ? (m >> (64 - b)) : 0ull;
  const bool neg = (u >> 63) != 0;
  uint64_t c = 0;  // carry, or borrow
  for (int i = i0; i < kExactLimbs; ++i) {
    const uint64_t v = i == i0 ? lo : (i == i0 + 1 ? hi : 0ull);
    const uint64_t x = w[i];
    if (!neg) {
      const uint64_t s = x + v, s2 = s + c;
      c = static_cast<uint64_t>(s < v) | static_cast<uint64_t>(s2 < c);
      w[i] = s2;
    } else {
      const uint64_t d = x - v, d2 = d - c;
      c = static_cast<uint64_t>(x < v) | static_cast<uint64_t>(d < c);
      w[i] = d2;
    }
    if (i > i0 && c == 0) break;
  }
}

HST_EXACT_HD inline bool exact_acc_nonneg(const uint64_t* w) {
  return static_cast<int64_t>(w[kExactLimbs - 1]) >= 0;
}

// [ sum_{c < n} prod(c) >= 0 ], exactly; prod(c) returns the c-th product in
// float64 (exact).  w: kExactLimbs words of scratch (registers, LDS or
// memory).
template <class Prod>
HST_EXACT_HD inline bool exact_sum_nonneg(const Prod& prod, int n, uint64_t* w) {
  for (int i = 0; i < kExactLimbs; ++i) w[i] = 0ull;
  for (int c = 0; c < n; ++c) exact_acc_add(w, prod(c));
  return exact_acc_nonneg(w);
}

}  // namespace hst
