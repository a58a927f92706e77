// Internal device helpers shared by the HIP kernels of libhst (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exact_dot.h"
#include "hst.h"

namespace hst {

constexpr int kWave = 64;

// Checks of the debug build (compiled with HST_DEBUG into libhst_debug.so,
// as relocatable device code so that one word serves every kernel).  A
// failed check records its code in hst_debug_word (the first failure wins)
// and execution goes on with the value clamped into range, so the kernel
// completes normally; hst_debug_status() reads and clears the word.  In the
// release build the checks compile to nothing and the value passes through.
#ifdef HST_DEBUG
extern __device__ uint32_t hst_debug_word;
__device__ __forceinline__ void hst_dfail(uint32_t code) { atomicCAS(&hst_debug_word, 0u, code); }
__device__ __forceinline__ int hst_dclamp(int v, int lo, int hi, uint32_t code) {
  if (v < lo || v > hi) {
    hst_dfail(code);
    return v < lo ? lo : hi;
  }
  return v;
}
#define HST_DCHECK(cond, code) \
  do {                         \
    if (!(cond)) hst_dfail(code); \
  } while (0)
#define HST_DCLAMP(v, lo, hi, code) hst_dclamp((v), (lo), (hi), (code))
#else
#define HST_DCHECK(cond, code) \
  do {                         \
  } while (0)
#define HST_DCLAMP(v, lo, hi, code) (v)
#endif

// Codes of the debug checks.
enum : uint32_t {
  kDbgChunkCount = 1,   // a scan chunk's candidate count above its slot capacity
  kDbgCandLds = 2,      // a candidate copied past the LDS candidate region
  kDbgRankSlot = 3,     // a rank entry past its LDS slots
  kDbgRowLds = 4,       // a selected row written past the split's LDS rows
  kDbgGatherRow = 5,    // a gathered row outside [0, n)
  kDbgMergeLds = 6,     // the split merge's weights past its LDS region
  kDbgSelectCount = 7,  // a selection that does not take exactly k_eff rows
  kDbgSampleRow = 8,    // a sampled key outside [0, n)
  kDbgCardRow = 9,      // an index card outside the head's card rows
};

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

// A float64 moved across lanes by one DPP control (both halves; a lane
// whose source lane is outside its row reads 0, by bound_ctrl).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(u), CTRL, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(u >> 32), CTRL, 0xf, 0xf, true);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                                     static_cast<uint32_t>(lo)));
}

// dpp_f64 with row_shr:s (1 <= s <= 15): lane i of a 16-lane row takes lane
// i - s of the row (lanes i < s read 0).  s must fold to a constant.
__device__ __forceinline__ double dpp_f64_row_shr(double v, int s) {
  switch (s) {
    case 1: return dpp_f64<0x111>(v);
    case 2: return dpp_f64<0x112>(v);
    case 3: return dpp_f64<0x113>(v);
    case 4: return dpp_f64<0x114>(v);
    case 5: return dpp_f64<0x115>(v);
    case 6: return dpp_f64<0x116>(v);
    case 7: return dpp_f64<0x117>(v);
    case 8: return dpp_f64<0x118>(v);
    case 9: return dpp_f64<0x119>(v);
    case 10: return dpp_f64<0x11a>(v);
    case 11: return dpp_f64<0x11b>(v);
    case 12: return dpp_f64<0x11c>(v);
    case 13: return dpp_f64<0x11d>(v);
    case 14: return dpp_f64<0x11e>(v);
    default: return dpp_f64<0x11f>(v);
  }
}

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

// [ a . b >= 0 ] exactly for stored float32/bf16 vectors: the products
// (exact in float64) summed in the fixed-point accumulator of exact_dot.h.
// w: kExactLimbs words of scratch (registers, LDS or memory).
template <typename T>
__device__ __forceinline__ bool exact_dot_nonneg_in(const T* __restrict__ a, const T* __restrict__ b, int n,
                                                    uint64_t* w) {
  return exact_sum_nonneg([&](int c) { return to_f64(a[c]) * to_f64(b[c]); }, n, w);
}

template <typename T>
__device__ __noinline__ bool exact_dot_nonneg(const T* __restrict__ a, const T* __restrict__ b, int n) {
  uint64_t w[kExactLimbs];
  return exact_dot_nonneg_in(a, b, n, w);
}

// [ a . b >= 0 ] for the exact real dot product of stored float32/bf16
// vectors.  The float64 sum has error below n * 2^-53 * sum|a_c b_c| for any
// order; only inside twice that band is the exact sum needed.
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
  return exact_dot_nonneg(a, b, n);
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
