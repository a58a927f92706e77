// Prefill hashing of keys: soft-LSH bucket ids + value norms, and binary
// codes.  SOCKET overview page, "Core mechanism: soft LSH", item 1 (one
// bucket id per table from random projections, value norm cached); HATA
// explainer page, section 3 (binary codes of keys).
//
// The sign decisions are exact: each projection is summed in float64 and,
// only when that sum lies inside its rounding band, re-summed exactly.
#include "hst_common.h"
#include "hst_launch.h"

namespace hst {

// One thread per (key, table): P projections, P sign bits -> one id byte.
template <typename T>
__global__ void __launch_bounds__(256)
hash_softlsh_generic_kernel(const T* __restrict__ K, const T* __restrict__ W,
                            const int32_t* __restrict__ seq_lens, int Hkv, int Nmax,
                            int d, int L, int P, uint8_t* __restrict__ ids) {
  const int bh = blockIdx.y;
  const int b = bh / Hkv, h = bh % Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const long long t = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long long j = t / L;
  const int l = static_cast<int>(t % L);
  if (j >= n) return;
  const T* key = K + (static_cast<long long>(bh) * Nmax + j) * d;
  const T* wt = W + (static_cast<long long>(h) * L * P + static_cast<long long>(l) * P) * d;
  uint32_t id = 0;
  for (int p = 0; p < P; ++p)
    if (dot_nonneg_exact(wt + static_cast<long long>(p) * d, key, d)) id |= 1u << p;
  ids[(static_cast<long long>(bh) * Nmax + j) * L + l] = static_cast<uint8_t>(id);
}

// Value norms: 16 lanes per key, float64 sum of squares (each square is
// exact), square root, one rounding to the storage type.
template <typename T, bool F16OUT>
__global__ void __launch_bounds__(256)
value_norm_kernel(const T* __restrict__ V, const int32_t* __restrict__ seq_lens,
                  int Hkv, int Nmax, int d, void* __restrict__ vnorm) {
  const int bh = blockIdx.y;
  const int b = bh / Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int sub = threadIdx.x & 15;
  const long long j = static_cast<long long>(blockIdx.x) * (blockDim.x / 16) + (threadIdx.x >> 4);
  double acc = 0.0;
  if (j < n) {
    const T* row = V + (static_cast<long long>(bh) * Nmax + j) * d;
    for (int c = sub; c < d; c += 16) {
      double v = to_f64(row[c]);
      acc += v * v;
    }
  }
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (j < n && sub == 0) {
    double r = sqrt(acc);
    long long o = static_cast<long long>(bh) * Nmax + j;
    if (F16OUT)
      static_cast<uint16_t*>(vnorm)[o] = f64_to_f16_bits(r);
    else
      static_cast<float*>(vnorm)[o] = static_cast<float>(r);
  }
}

// Binary codes: a block of 2*64 threads handles keys one at a time; thread i
// decides bit i, a wave ballot packs 64 bits into two words.
template <typename T>
__global__ void __launch_bounds__(128)
binary_codes_generic_kernel(const T* __restrict__ X, const T* __restrict__ R,
                            const int32_t* __restrict__ seq_lens, int Hkv, int Nmax,
                            int d, int keys_per_block, uint32_t* __restrict__ codes) {
  const int bh = blockIdx.y;
  const int b = bh / Hkv, h = bh % Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int i = threadIdx.x;  // bit index 0..127
  const T* rrow = R + (static_cast<long long>(h) * 128 + i) * d;
  const long long j0 = static_cast<long long>(blockIdx.x) * keys_per_block;
  for (int u = 0; u < keys_per_block; ++u) {
    const long long j = j0 + u;
    if (j >= n) break;
    const T* x = X + (static_cast<long long>(bh) * Nmax + j) * d;
    bool bit = dot_nonneg_exact(rrow, x, d);
    unsigned long long m = __ballot(bit);
    if ((i & 63) == 0) {
      uint32_t* dst = codes + (static_cast<long long>(bh) * Nmax + j) * 4 + (i >> 6) * 2;
      dst[0] = static_cast<uint32_t>(m);
      dst[1] = static_cast<uint32_t>(m >> 32);
    }
  }
}

hipError_t launch_hash_softlsh(const hst_shape& s, const void* K, const void* V,
                               const void* W, int L, int P, int norm_dtype,
                               uint8_t* ids, void* vnorm, hipStream_t st) {
  const int BH = s.B * s.Hkv;
  {
    long long work = static_cast<long long>(s.Nmax) * L;
    dim3 grid(static_cast<unsigned>((work + 255) / 256), BH);
    if (s.kv_dtype == HST_F32)
      hipLaunchKernelGGL(hash_softlsh_generic_kernel<float>, grid, dim3(256), 0, st,
                         static_cast<const float*>(K), static_cast<const float*>(W),
                         s.seq_lens, s.Hkv, s.Nmax, s.d, L, P, ids);
    else
      hipLaunchKernelGGL(hash_softlsh_generic_kernel<bf16>, grid, dim3(256), 0, st,
                         static_cast<const bf16*>(K), static_cast<const bf16*>(W),
                         s.seq_lens, s.Hkv, s.Nmax, s.d, L, P, ids);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    dim3 grid(static_cast<unsigned>((s.Nmax + 15) / 16), BH);
    const bool f16 = norm_dtype == HST_F16;
    if (s.kv_dtype == HST_F32) {
      if (f16)
        hipLaunchKernelGGL((value_norm_kernel<float, true>), grid, dim3(256), 0, st,
                           static_cast<const float*>(V), s.seq_lens, s.Hkv, s.Nmax, s.d, vnorm);
      else
        hipLaunchKernelGGL((value_norm_kernel<float, false>), grid, dim3(256), 0, st,
                           static_cast<const float*>(V), s.seq_lens, s.Hkv, s.Nmax, s.d, vnorm);
    } else {
      if (f16)
        hipLaunchKernelGGL((value_norm_kernel<bf16, true>), grid, dim3(256), 0, st,
                           static_cast<const bf16*>(V), s.seq_lens, s.Hkv, s.Nmax, s.d, vnorm);
      else
        hipLaunchKernelGGL((value_norm_kernel<bf16, false>), grid, dim3(256), 0, st,
                           static_cast<const bf16*>(V), s.seq_lens, s.Hkv, s.Nmax, s.d, vnorm);
    }
  }
  return hipGetLastError();
}

hipError_t launch_hash_binary(const hst_shape& s, const void* K, const void* R,
                              uint32_t* codes, hipStream_t st) {
  const int kpb = 16;
  dim3 grid(static_cast<unsigned>((s.Nmax + kpb - 1) / kpb), s.B * s.Hkv);
  if (s.kv_dtype == HST_F32)
    hipLaunchKernelGGL(binary_codes_generic_kernel<float>, grid, dim3(128), 0, st,
                       static_cast<const float*>(K), static_cast<const float*>(R),
                       s.seq_lens, s.Hkv, s.Nmax, s.d, kpb, codes);
  else
    hipLaunchKernelGGL(binary_codes_generic_kernel<bf16>, grid, dim3(128), 0, st,
                       static_cast<const bf16*>(K), static_cast<const bf16*>(R),
                       s.seq_lens, s.Hkv, s.Nmax, s.d, kpb, codes);
  return hipGetLastError();
}

}  // namespace hst
