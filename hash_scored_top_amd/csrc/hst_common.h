// Internal device helpers shared by the HIP kernels of libhst (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hst.h"

namespace hst {

constexpr int kWave = 64;

// Native 128-bit vector (stays in registers where HIP's struct vector types
// can end up in scratch memory when held in arrays).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// bf16 element stored as its 16 bit pattern.
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}
__device__ __forceinline__ double to_f64(float x) { return static_cast<double>(x); }
__device__ __forceinline__ double to_f64(bf16 x) { return static_cast<double>(to_f32(x)); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sum over each aligned group of W = 16 or 8 lanes, left in every lane
// of the group: DPP quad permutes and row mirrors, no LDS traffic.
template <int W>
__device__ __forceinline__ float dpp_group_sum(float v) {
  static_assert(W == 8 || W == 16, "group of 8 or 16 lanes");
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1,
                                                             0xf, 0xf, false));  // quad [1,0,3,2]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E,
                                                             0xf, 0xf, false));  // quad [2,3,0,1]
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141,
                                                             0xf, 0xf, false));  // row half mirror
  if (W == 16)
    v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x140,
                                                               0xf, 0xf, false));  // row mirror
  return v;
}

// Context length of sequence b.
__device__ __forceinline__ int seq_len(const int32_t* seq_lens, int b, int nmax) {
  if (seq_lens == nullptr) return nmax;
  int n = seq_lens[b];
  return n < 0 ? 0 : (n > nmax ? nmax : n);
}

// Sign of a sum of float64 values, exactly: Shewchuk's growing expansion
// ("Adaptive precision floating-point arithmetic", 1997) keeps the running
// sum as non-overlapping partials, so the sign of the total is the sign of
// the largest non-zero partial.  Returns true when the sum is >= 0.  h holds
// up to hcap partials (products of stored bf16 / float32 values span at most
// about 600 bits, i.e. a dozen non-overlapping float64 partials).
template <typename T>
__device__ __forceinline__ bool expansion_dot_nonneg_in(const T* __restrict__ a,
                                                     const T* __restrict__ b, int n,
                                                     double* h, int hcap) {
  int nh = 0;
  for (int c = 0; c < n; ++c) {
    double x = to_f64(a[c]) * to_f64(b[c]);  // exact: at most 48 significant bits
    int k = 0;
    for (int i = 0; i < nh; ++i) {
      double y = h[i];
      double hi = x + y;
      double bv = hi - x;
      double lo = (x - (hi - bv)) + (y - bv);
      if (lo != 0.0) h[k++] = lo;
      x = hi;
    }
    if (k < hcap) h[k++] = x;
    nh = k;
  }
  for (int i = nh - 1; i >= 0; --i)
    if (h[i] != 0.0) return h[i] > 0.0;
  return true;
}

template <typename T>
__device__ __noinline__ bool expansion_dot_nonneg(const T* __restrict__ a,
                                                  const T* __restrict__ b, int n) {
  double h[48];
  return expansion_dot_nonneg_in(a, b, n, h, 48);
}

// [ a . b >= 0 ] for the exact real dot product of stored float32/bf16
// vectors.  The float64 sum has error below n * 2^-53 * sum|a_c b_c| for any
// order; only inside twice that band is the exact expansion needed.
template <typename T>
__device__ __forceinline__ bool dot_nonneg_exact(const T* __restrict__ a,
                                                 const T* __restrict__ b, int n) {
  double s = 0.0, sa = 0.0;
  for (int c = 0; c < n; ++c) {
    double p = to_f64(a[c]) * to_f64(b[c]);
    s += p;
    sa += fabs(p);
  }
  if (fabs(s) > 2.0 * n * 0x1p-53 * sa) return s >= 0.0;
  return expansion_dot_nonneg(a, b, n);
}

// float64 -> IEEE binary16 bits, round to nearest, ties to even, in one
// rounding step (no intermediate float32).
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
  uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  uint16_t sign = static_cast<uint16_t>((u >> 48) & 0x8000u);
  uint64_t a = u & 0x7fffffffffffffffull;
  if (a >= 0x7ff0000000000000ull)  // inf / nan
    return sign | 0x7c00u | (a > 0x7ff0000000000000ull ? 0x200u : 0u);
  if (a == 0) return sign;
  int e = static_cast<int>(a >> 52) - 1023;
  if (e >= 16) return sign | 0x7c00u;
  if (e < -26) return sign;  // below half of the smallest subnormal
  uint64_t mant = (a & 0x000fffffffffffffull) | 0x0010000000000000ull;
  int emin = e < -14 ? -14 : e;       // exponent of the target ulp + 10
  int shift = 42 + (emin - e);         // 52 - e + (emin - 10)
  uint64_t q = mant >> shift;
  uint64_t rem = mant & ((1ull << shift) - 1);
  uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  uint32_t bits = (e >= -14) ? (static_cast<uint32_t>(e + 14) << 10) + static_cast<uint32_t>(q)
                             : static_cast<uint32_t>(q);
  if (bits >= 0x7c00u) bits = 0x7c00u;
  return sign | static_cast<uint16_t>(bits);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

}  // namespace hst
