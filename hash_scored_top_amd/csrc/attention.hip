// Exact softmax attention over the selected keys (SOCKET overview page,
// "Core mechanism: soft LSH", item 4: exact attention on the chosen subset).
//
// Split-K flash decode over gathered rows: the idx row of a kv head is cut
// into splits; one workgroup gathers each selected K/V row of its split once
// and reuses it for all G query heads of the group (grouped-query
// attention), keeping an online-softmax state (m, l, o) per head in the
// base-2 exponent domain.  A second kernel merges the split states through
// their log-sum-exp.
#include "hst_common.h"
#include "hst_launch.h"

namespace hst {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename T, int EPL>
struct RowLoad;

template <>
struct RowLoad<bf16, 8> {  // 16 bytes
  static __device__ __forceinline__ void ld(const bf16* p, float (&x)[8]) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
};
template <>
struct RowLoad<bf16, 4> {  // 8 bytes
  static __device__ __forceinline__ void ld(const bf16* p, float (&x)[4]) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  }
};
template <>
struct RowLoad<float, 8> {  // 32 bytes
  static __device__ __forceinline__ void ld(const float* p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};
template <>
struct RowLoad<float, 4> {  // 16 bytes
  static __device__ __forceinline__ void ld(const float* p, float (&x)[4]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  }
};

// Merge online-softmax state (m2, l2, o2) into (m, l, o); m in log2 units.
template <int EPL>
__device__ __forceinline__ void merge_state(float& m, float& l, float (&o)[EPL], float m2, float l2,
                                            const float (&o2)[EPL]) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  const float a = exp2f(m - mn), c = exp2f(m2 - mn);
  l = l * a + l2 * c;
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = o[e] * a + o2[e] * c;
  m = mn;
}

template <typename T, int D, int GMAX>
__global__ void __launch_bounds__(256)
sparse_attn_split_kernel(const T* __restrict__ q, const T* __restrict__ K,
                         const T* __restrict__ Vv, const int32_t* __restrict__ idx,
                         const int32_t* __restrict__ seq_lens, int Hq, int Hkv, int Nmax,
                         int kcap, int rps, int nsplit, float scale_log2,
                         float* __restrict__ part_o, float* __restrict__ part_ml) {
  constexpr int EPL = D / 16;
  constexpr int U = 2;
  __shared__ float red_ml[4][GMAX][2];
  __shared__ float red_o[4][GMAX][D];
  const int G = Hq / Hkv;
  const int bh = blockIdx.y;
  const int b = bh / Hkv, h = bh % Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int split = blockIdx.x;
  const int r0 = split * rps;
  const int r1 = min(r0 + rps, kcap);
  const int sub = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;  // 0..15
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  float qv[GMAX][EPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g < G) {
      RowLoad<T, EPL>::ld(q + (static_cast<long long>(b) * Hq + h * G + g) * D + sub * EPL, qv[g]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[g][e] *= scale_log2;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qv[g][e] = 0.f;
    }
  }
  float m[GMAX], l[GMAX], o[GMAX][EPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
  }
  const long long kvbase = static_cast<long long>(bh) * Nmax;
  const int32_t* irow = idx + static_cast<long long>(bh) * kcap;

  for (int rb = r0 + grp; rb < r1; rb += 16 * U) {
    float kx[U][EPL], vx[U][EPL];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + u * 16;
      const int j = r < r1 ? irow[r] : -1;
      ok[u] = j >= 0 && j < n;
      if (ok[u]) {
        RowLoad<T, EPL>::ld(K + (kvbase + j) * D + sub * EPL, kx[u]);
        RowLoad<T, EPL>::ld(Vv + (kvbase + j) * D + sub * EPL, vx[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!ok[u]) continue;  // uniform across the 16 lanes of the group
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        if (g >= G) break;
        float sdot = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) sdot += qv[g][e] * kx[u][e];
#pragma unroll
        for (int mm = 8; mm >= 1; mm >>= 1) sdot += __shfl_xor(sdot, mm, 16);
        const float mn = fmaxf(m[g], sdot);
        const float a = exp2f(m[g] - mn);
        const float p = exp2f(sdot - mn);
        l[g] = l[g] * a + p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] = o[g][e] * a + p * vx[u][e];
        m[g] = mn;
      }
    }
  }

  // merge the four 16-lane groups of each wave
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= G) break;
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
      const float m2 = __shfl_xor(m[g], x, 64);
      const float l2 = __shfl_xor(l[g], x, 64);
      float o2[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) o2[e] = __shfl_xor(o[g][e], x, 64);
      merge_state<EPL>(m[g], l[g], o[g], m2, l2, o2);
    }
  }
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) break;
      if (lane == 0) {
        red_ml[wave][g][0] = m[g];
        red_ml[wave][g][1] = l[g];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_o[wave][g][lane * EPL + e] = o[g][e];
    }
  }
  __syncthreads();
  // merge the four waves: thread t handles (g, element) pairs
  for (int t = threadIdx.x; t < G * D; t += blockDim.x) {
    const int g = t / D, c = t % D;
    float mm = -INFINITY;
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, red_ml[w][g][0]);
    float ll = 0.f, oo = 0.f;
    if (mm != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        const float wgt = exp2f(red_ml[w][g][0] - mm);
        ll += red_ml[w][g][1] * wgt;
        oo += red_o[w][g][c] * wgt;
      }
    }
    const long long pi = (static_cast<long long>(b) * Hq + h * G + g) * nsplit + split;
    part_o[pi * D + c] = oo;
    if (c == 0) {
      part_ml[pi * 2] = mm;
      part_ml[pi * 2 + 1] = ll;
    }
  }
}

__global__ void __launch_bounds__(256)
attn_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml, int D,
                    int nsplit, float* __restrict__ out, float* __restrict__ lse) {
  const int bq = blockIdx.x;  // b * Hq + hq
  const float* ml = part_ml + static_cast<long long>(bq) * nsplit * 2;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, ml[2 * s]);
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float Lsum = 0.f, O = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        const float ms = ml[2 * s];
        if (ms == -INFINITY) continue;
        const float w = exp2f(ms - M);
        Lsum += ml[2 * s + 1] * w;
        O += part_o[(static_cast<long long>(bq) * nsplit + s) * D + c] * w;
      }
    }
    out[static_cast<long long>(bq) * D + c] = Lsum > 0.f ? O / Lsum : 0.f;
    if (c == 0 && lse != nullptr)
      lse[bq] = Lsum > 0.f ? (M + log2f(Lsum)) * kLn2 : -INFINITY;
  }
}

void attention_plan(const hst_shape& s, int kcap, int* rps, int* nsplit) {
  const long long rows = static_cast<long long>(kcap) * s.B * s.Hkv;
  long long r = (rows + 2047) / 2048;
  r = ((r + 31) / 32) * 32;
  if (r < 32) r = 32;
  if (r > 512) r = 512;
  *rps = static_cast<int>(r);
  *nsplit = static_cast<int>((kcap + r - 1) / r);
}

size_t attention_ws_bytes(const hst_shape& s, int kcap) {
  int rps, nsplit;
  attention_plan(s, kcap, &rps, &nsplit);
  const size_t parts = static_cast<size_t>(s.B) * s.Hq * nsplit;
  return parts * (static_cast<size_t>(s.d) + 2) * sizeof(float) + 256;
}

template <typename T, int D, int GMAX>
static void launch_attn_t(const hst_shape& s, const void* q, const void* K, const void* V,
                          const int32_t* idx, int kcap, int rps, int nsplit, float scale_log2,
                          float* po, float* pml, hipStream_t st) {
  dim3 grid(nsplit, s.B * s.Hkv);
  hipLaunchKernelGGL((sparse_attn_split_kernel<T, D, GMAX>), grid, dim3(256), 0, st,
                     static_cast<const T*>(q), static_cast<const T*>(K), static_cast<const T*>(V),
                     idx, s.seq_lens, s.Hq, s.Hkv, s.Nmax, kcap, rps, nsplit, scale_log2, po, pml);
}

template <typename T, int D>
static void launch_attn_g(const hst_shape& s, const void* q, const void* K, const void* V,
                          const int32_t* idx, int kcap, int rps, int nsplit, float scale_log2,
                          float* po, float* pml, hipStream_t st) {
  const int G = s.Hq / s.Hkv;
  if (G <= 1) launch_attn_t<T, D, 1>(s, q, K, V, idx, kcap, rps, nsplit, scale_log2, po, pml, st);
  else if (G <= 2) launch_attn_t<T, D, 2>(s, q, K, V, idx, kcap, rps, nsplit, scale_log2, po, pml, st);
  else if (G <= 4) launch_attn_t<T, D, 4>(s, q, K, V, idx, kcap, rps, nsplit, scale_log2, po, pml, st);
  else launch_attn_t<T, D, 8>(s, q, K, V, idx, kcap, rps, nsplit, scale_log2, po, pml, st);
}

hipError_t launch_attention(const hst_shape& s, const void* q, const void* K, const void* V,
                            const int32_t* idx, int kcap, float scale, float* out, float* lse,
                            void* ws, hipStream_t st) {
  int rps, nsplit;
  attention_plan(s, kcap, &rps, &nsplit);
  const size_t parts = static_cast<size_t>(s.B) * s.Hq * nsplit;
  float* po = static_cast<float*>(ws);
  float* pml = po + parts * s.d;
  const float sl2 = scale * kLog2e;
  if (s.kv_dtype == HST_F32) {
    if (s.d == 64) launch_attn_g<float, 64>(s, q, K, V, idx, kcap, rps, nsplit, sl2, po, pml, st);
    else launch_attn_g<float, 128>(s, q, K, V, idx, kcap, rps, nsplit, sl2, po, pml, st);
  } else {
    if (s.d == 64) launch_attn_g<bf16, 64>(s, q, K, V, idx, kcap, rps, nsplit, sl2, po, pml, st);
    else launch_attn_g<bf16, 128>(s, q, K, V, idx, kcap, rps, nsplit, sl2, po, pml, st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(s.B * s.Hq), dim3(s.d), 0, st, po, pml, s.d,
                     nsplit, out, lse);
  return hipGetLastError();
}

}  // namespace hst
