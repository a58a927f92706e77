// Decode-time append of one token per sequence with incremental hashing.
// SOCKET overview page, "Core mechanism: soft LSH", item 1: a key's bucket
// ids and its value norm are computed once, when the key enters the cache;
// HATA explainer page, section 3: likewise a key's binary code.  During
// decode one key enters per sequence and step, so its metadata is produced
// right there, with the same exact sign rule as the prefill hashing.
//
// Two launches: append_rows_kernel writes row N_b of K, V and the metadata
// of every (sequence, kv head) (reading N_b), then advance_lens_kernel
// increments N_b.  Splitting them keeps every workgroup of a sequence reading
// the same N_b, and a decode step enqueued after them sees the new token.
// The work is latency bound (one key per head against its planes); the
// planes are spread over workgroups so that one memory round trip covers
// them.
#include "hst_common.h"
#include "hst_launch.h"

namespace hst {

constexpr int kAppendNT = 256;
constexpr int kAppendLanes = 4;                         // lanes per plane
constexpr int kAppendPlanes = kAppendNT / kAppendLanes;  // planes per workgroup
constexpr int kAppendExp = kExactLimbs;  // words of an exact fixed-point sum (LDS, per plane)

__device__ __forceinline__ void load8(const float* __restrict__ p, float (&x)[8]) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  const u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
  for (int e = 0; e < 4; ++e) {
    x[e] = __uint_as_float(a[e]);
    x[4 + e] = __uint_as_float(b[e]);
  }
}

__device__ __forceinline__ void load8(const bf16* __restrict__ p, float (&x)[8]) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(a[e]);
    x[2 * e + 1] = bf16_hi(a[e]);
  }
}

// Grid (B * Hkv, groups).  Workgroup (bh, y) takes a group of at most 64
// planes: MODE 0, the tables [y * tpg, (y + 1) * tpg) with tpg = 64 / P, whose
// ids it writes; MODE 1, code words 2y and 2y + 1.  Four lanes share a plane,
// each holding D/4 products, so all loads of the group are in flight at once.
// Workgroup y == 0 also copies the K and V rows and writes the value norm.
template <typename T, int D, int MODE>
__global__ void __launch_bounds__(kAppendNT)
append_rows_kernel(const T* __restrict__ k_new, const T* __restrict__ v_new,
                   const T* __restrict__ Wp, const int32_t* __restrict__ lens, int Hkv, int Nmax,
                   int L, int P, int norm_f16, T* __restrict__ K, T* __restrict__ V,
                   uint8_t* __restrict__ ids, void* __restrict__ vnorm,
                   uint32_t* __restrict__ codes) {
  constexpr int kPer = D / kAppendLanes;  // elements per lane
  __shared__ uint32_t bits[kAppendPlanes / 32];
  __shared__ double nsum[kAppendNT / 64];
  __shared__ uint64_t hx[kAppendPlanes * kAppendExp];
  const int bh = blockIdx.x, b = bh / Hkv, h = bh % Hkv, y = blockIdx.y;
  const int n = lens[b] < 0 ? 0 : lens[b];
  if (n >= Nmax) return;  // full cache: nothing written, the length stays
  const int t = threadIdx.x;
  const T* kn = k_new + static_cast<long long>(bh) * D;
  const T* vn = v_new + static_cast<long long>(bh) * D;
  const long long row = static_cast<long long>(bh) * Nmax + n;
  const int nplanes = MODE == 0 ? L * P : 128;
  const int tpg = MODE == 0 ? kAppendPlanes / P : 0;  // tables per group
  const int p0 = MODE == 0 ? y * tpg * P : y * kAppendPlanes;
  const int gplanes = MODE == 0 ? min(tpg, L - y * tpg) * P : kAppendPlanes;
  if (t < kAppendPlanes / 32) bits[t] = 0u;
  __syncthreads();

  // this lane's slice of the key and of its plane, all loads issued up front
  const int pl = t / kAppendLanes, part = t % kAppendLanes;
  const bool live = pl < gplanes;
  const T* wr = Wp + (static_cast<long long>(h) * nplanes + p0 + (live ? pl : 0)) * D;
  float kv[kPer], wv[kPer];
#pragma unroll
  for (int c = 0; c < kPer; c += 8) {
    float k8[8], w8[8];
    load8(kn + part * kPer + c, k8);
    load8(wr + part * kPer + c, w8);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      kv[c + e] = k8[e];
      wv[c + e] = w8[e];
    }
  }
  double s = 0.0, sa = 0.0;
#pragma unroll
  for (int c = 0; c < kPer; ++c) {
    const double q = static_cast<double>(wv[c]) * static_cast<double>(kv[c]);  // exact
    s += q;
    sa += fabs(q);
  }
  // group of four lanes: any summation order stays within the bound below
  s += __shfl_xor(s, 1);
  sa += __shfl_xor(sa, 1);
  s += __shfl_xor(s, 2);
  sa += __shfl_xor(sa, 2);
  if (live && part == 0) {
    const bool bit = fabs(s) > 2.0 * D * 0x1p-53 * sa
                         ? s >= 0.0
                         : exact_dot_nonneg_in(wr, kn, D, hx + pl * kAppendExp);
    if (bit) atomicOr(&bits[pl >> 5], 1u << (pl & 31));
  }

  // rows and value norm (float64 sum of squares, one rounding)
  if (y == 0) {
    double sq = 0.0;
    for (int c = t; c < D; c += kAppendNT) {
      K[row * D + c] = kn[c];
      V[row * D + c] = vn[c];
      const double x = to_f64(vn[c]);
      sq += x * x;
    }
    if (MODE == 0) {
      for (int m = 32; m >= 1; m >>= 1) sq += __shfl_xor(sq, m);
      if ((t & 63) == 0) nsum[t >> 6] = sq;
    }
  }
  __syncthreads();
  if (MODE == 0) {
    // id of table l: plane p of the table is bit p
    for (int j = t; j < gplanes / P; j += kAppendNT) {
      uint32_t id = 0;
      for (int p = 0; p < P; ++p) {
        const int r = j * P + p;
        id |= ((bits[r >> 5] >> (r & 31)) & 1u) << p;
      }
      ids[row * L + y * tpg + j] = static_cast<uint8_t>(id);
    }
    if (y == 0 && t == 0) {
      double a = 0.0;
      for (int w = 0; w < kAppendNT / 64; ++w) a += nsum[w];
      const double r = sqrt(a);
      if (norm_f16)
        static_cast<uint16_t*>(vnorm)[row] = f64_to_f16_bits(r);
      else
        static_cast<float*>(vnorm)[row] = static_cast<float>(r);
    }
  } else {
    if (t < 2) codes[row * 4 + 2 * y + t] = bits[t];
  }
}

__global__ void advance_lens_kernel(int32_t* __restrict__ lens, int B, int Nmax) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) {
    const int n = lens[b] < 0 ? 0 : lens[b];
    if (n < Nmax) lens[b] = n + 1;
  }
}

template <typename T, int MODE>
static void launch_rows(const hst_shape& s, dim3 grid, const void* k_new, const void* v_new,
                        const void* Wp, int L, int P, int norm_f16, void* K, void* V,
                        uint8_t* ids, void* vnorm, uint32_t* codes, hipStream_t st) {
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, dim3(kAppendNT), 0, st, static_cast<const T*>(k_new),
                       static_cast<const T*>(v_new), static_cast<const T*>(Wp), s.seq_lens,
                       s.Hkv, s.Nmax, L, P, norm_f16, static_cast<T*>(K), static_cast<T*>(V), ids,
                       vnorm, codes);
  };
  if (s.d == 64)
    go(append_rows_kernel<T, 64, MODE>);
  else
    go(append_rows_kernel<T, 128, MODE>);
}

template <int MODE>
static hipError_t launch_append(const hst_shape& s, const void* k_new, const void* v_new,
                                const void* Wp, int L, int P, int norm_f16, void* K, void* V,
                                uint8_t* ids, void* vnorm, uint32_t* codes, hipStream_t st) {
  const int tpg = MODE == 0 ? kAppendPlanes / P : 0;
  const int groups = MODE == 0 ? (L + tpg - 1) / tpg : 128 / kAppendPlanes;
  const dim3 grid(static_cast<unsigned>(s.B * s.Hkv), static_cast<unsigned>(groups));
  if (s.kv_dtype == HST_F32)
    launch_rows<float, MODE>(s, grid, k_new, v_new, Wp, L, P, norm_f16, K, V, ids, vnorm, codes,
                             st);
  else
    launch_rows<bf16, MODE>(s, grid, k_new, v_new, Wp, L, P, norm_f16, K, V, ids, vnorm, codes,
                            st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(advance_lens_kernel, dim3((s.B + 255) / 256), dim3(256), 0, st,
                     const_cast<int32_t*>(s.seq_lens), s.B, s.Nmax);
  return hipGetLastError();
}

hipError_t launch_append_softlsh(const hst_shape& s, const void* k_new, const void* v_new,
                                 const void* W, int L, int P, int norm_dtype, void* K, void* V,
                                 uint8_t* ids, void* vnorm, hipStream_t st) {
  return launch_append<0>(s, k_new, v_new, W, L, P, norm_dtype == HST_F16 ? 1 : 0, K, V, ids,
                          vnorm, nullptr, st);
}

hipError_t launch_append_binary(const hst_shape& s, const void* k_new, const void* v_new,
                                const void* R, void* K, void* V, uint32_t* codes, hipStream_t st) {
  return launch_append<1>(s, k_new, v_new, R, 0, 0, 0, K, V, nullptr, nullptr, codes, st);
}

}  // namespace hst
