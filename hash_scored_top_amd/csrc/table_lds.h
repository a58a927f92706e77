// LDS copies of a kv head's soft-LSH table and key scoring from them
// (internal to libhst).  The table is bucket-major [2^P][L] in the
// workspace; in LDS it is table-major with rows of pitch 2^P + 1, so that
// the lookups of a wave (random buckets) spread over the banks and the
// transposing stores (consecutive tables of one bucket) do not collide.
#pragma once

#include "hst_common.h"

namespace hst {

// Vector loads, four per thread in flight before any store.
template <int NT>
__device__ __forceinline__ void load_table_t(const float* __restrict__ Tg, float* tl, int L, int nb) {
  const int n4 = (nb * L) / 4;  // nb * L is a multiple of 16
  const u32x4* src = reinterpret_cast<const u32x4*>(Tg);
  for (int base = 0; base < n4; base += 4 * NT) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + u * NT + static_cast<int>(threadIdx.x);
      if (i < n4) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = base + u * NT + static_cast<int>(threadIdx.x);
      if (i < n4) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int e = 4 * i + q, bk = e / L, l = e % L;
          tl[l * (nb + 1) + bk] = __uint_as_float(v[u][q]);
        }
      }
    }
  }
}

// sum_l T[l][id_l] over a key's L bucket ids (L / 16 vectors of 16 bytes),
// in table order, float32.
template <int L>
__device__ __forceinline__ float table_sum(const u32x4 (&idv)[L / 16], const float* tl, int nb) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < L / 16; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t word = idv[i][q];
#pragma unroll
      for (int by = 0; by < 4; ++by) {
        const int l = i * 16 + q * 4 + by;
        s += tl[l * (nb + 1) + ((word >> (8 * by)) & 0xffu)];
      }
    }
  }
  return s;
}

}  // namespace hst
