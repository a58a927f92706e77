// Key scoring scans, the bandwidth-dominant stage of a decode step.
//  * Soft-collision score (SOCKET overview page, "Core mechanism: soft LSH",
//    item 3): score_j = ||v_j|| * sum_l T[l][id_{j,l}], with the kv head's
//    bucket-probability table T resident in LDS and each key's L one-byte
//    bucket ids streamed from HBM exactly once.
//  * Code-similarity score (HATA explainer page, section 3): XOR + popcount
//    of 128-bit codes against the G query-head codes.
#include "hst_common.h"
#include "hst_launch.h"

namespace hst {

template <int LPL>
struct IdVec;
template <>
struct IdVec<16> {
  using type = uint4;
  static __device__ __forceinline__ uint32_t word(const uint4& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
  }
};
template <>
struct IdVec<8> {
  using type = uint2;
  static __device__ __forceinline__ uint32_t word(const uint2& v, int i) { return i == 0 ? v.x : v.y; }
};
template <>
struct IdVec<4> {
  using type = uint32_t;
  static __device__ __forceinline__ uint32_t word(const uint32_t& v, int) { return v; }
};

template <bool F16N>
__device__ __forceinline__ float load_norm(const void* vnorm, long long o) {
  if (F16N) return f16_bits_to_f32(static_cast<const uint16_t*>(vnorm)[o]);
  return static_cast<const float*>(vnorm)[o];
}

__device__ __forceinline__ void load_table_lds(float* tbl, const float* __restrict__ src, int n) {
  const int n4 = n >> 2;
  const float4* s4 = reinterpret_cast<const float4*>(src);
  float4* d4 = reinterpret_cast<float4*>(tbl);
  for (int i = threadIdx.x; i < n4; i += blockDim.x) d4[i] = s4[i];
  for (int i = (n4 << 2) + threadIdx.x; i < n; i += blockDim.x) tbl[i] = src[i];
}

// LANES lanes cooperate on one key; each holds LPL consecutive table ids.
template <int LPL, int LANES, bool F16N>
__global__ void __launch_bounds__(256)
score_softlsh_kernel(const float* __restrict__ tables, const uint8_t* __restrict__ ids,
                     const void* __restrict__ vnorm, const int32_t* __restrict__ seq_lens,
                     int Hkv, int Nmax, int P, int kpb, float* __restrict__ scores) {
  extern __shared__ float tbl[];
  constexpr int L = LPL * LANES;
  constexpr int KPI = 256 / LANES;  // keys per block iteration
  constexpr int U = 4;              // keys in flight per lane group
  using V = typename IdVec<LPL>::type;
  const int bh = blockIdx.y;
  const int b = bh / Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int j0 = blockIdx.x * kpb;
  if (j0 >= n) return;
  const int P_ = P;
  load_table_lds(tbl, tables + static_cast<long long>(bh) * (L << P_), L << P_);
  __syncthreads();
  const int jend = min(j0 + kpb, n);
  const int sub = threadIdx.x % LANES;
  const int grp = threadIdx.x / LANES;
  const long long base = static_cast<long long>(bh) * Nmax;
  const V* idv = reinterpret_cast<const V*>(ids);
  const float* tsub = tbl + ((sub * LPL) << P_);
  const uint32_t idmask = (1u << P_) - 1u;  // ids >= 2^P cannot leave the table

  for (int jb = j0 + grp; jb < jend; jb += KPI * U) {
    V w[U];
    float nr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * KPI;
      if (j < jend) {
        w[u] = idv[(base + j) * LANES + sub];
        nr[u] = load_norm<F16N>(vnorm, base + j);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * KPI;
      if (j < jend) {  // uniform across the LANES lanes of a key
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < LPL; ++i) {
          const uint32_t wd = IdVec<LPL>::word(w[u], i >> 2);
          const uint32_t id = (wd >> ((i & 3) * 8)) & idmask;
          acc += tsub[(i << P_) + id];
        }
#pragma unroll
        for (int m = LANES / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LANES);
        if (sub == 0) scores[base + j] = acc * nr[u];
      }
    }
  }
}

// Any L: one thread per key, byte loads.
template <bool F16N>
__global__ void __launch_bounds__(256)
score_softlsh_anyL_kernel(const float* __restrict__ tables, const uint8_t* __restrict__ ids,
                          const void* __restrict__ vnorm, const int32_t* __restrict__ seq_lens,
                          int Hkv, int Nmax, int L, int P, int kpb, float* __restrict__ scores) {
  extern __shared__ float tbl[];
  const int bh = blockIdx.y;
  const int b = bh / Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int j0 = blockIdx.x * kpb;
  if (j0 >= n) return;
  load_table_lds(tbl, tables + static_cast<long long>(bh) * (L << P), L << P);
  __syncthreads();
  const int jend = min(j0 + kpb, n);
  const long long base = static_cast<long long>(bh) * Nmax;
  for (int j = j0 + threadIdx.x; j < jend; j += blockDim.x) {
    const uint8_t* r = ids + (base + j) * L;
    float acc = 0.f;
    for (int l = 0; l < L; ++l) acc += tbl[(l << P) + (r[l] & ((1 << P) - 1))];
    scores[base + j] = acc * load_norm<F16N>(vnorm, base + j);
  }
}

__global__ void __launch_bounds__(256)
score_hamming_kernel(const uint32_t* __restrict__ qcodes, const uint4* __restrict__ codes,
                     const int32_t* __restrict__ seq_lens, int Hq, int Hkv, int Nmax, int kpb,
                     int32_t* __restrict__ scores) {
  __shared__ uint32_t qc[4 * 64];
  const int G = Hq / Hkv;
  const int bh = blockIdx.y;
  const int b = bh / Hkv, h = bh % Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int j0 = blockIdx.x * kpb;
  if (j0 >= n) return;
  for (int i = threadIdx.x; i < 4 * G; i += blockDim.x)
    qc[i] = qcodes[(static_cast<long long>(b) * Hq + h * G) * 4 + i];
  __syncthreads();
  const int jend = min(j0 + kpb, n);
  const long long base = static_cast<long long>(bh) * Nmax;
  for (int j = j0 + threadIdx.x; j < jend; j += blockDim.x) {
    const uint4 c = codes[base + j];
    int ham = 0;
    for (int g = 0; g < G; ++g)
      ham += __popc(c.x ^ qc[4 * g]) + __popc(c.y ^ qc[4 * g + 1]) +
             __popc(c.z ^ qc[4 * g + 2]) + __popc(c.w ^ qc[4 * g + 3]);
    scores[base + j] = 128 * G - ham;
  }
}

template <int LPL, int LANES>
static void launch_soft_t(dim3 grid, size_t smem, hipStream_t st, bool f16, const float* tables,
                          const uint8_t* ids, const void* vnorm, const hst_shape& s, int P,
                          int kpb, float* scores) {
  if (f16)
    hipLaunchKernelGGL((score_softlsh_kernel<LPL, LANES, true>), grid, dim3(256), smem, st,
                       tables, ids, vnorm, s.seq_lens, s.Hkv, s.Nmax, P, kpb, scores);
  else
    hipLaunchKernelGGL((score_softlsh_kernel<LPL, LANES, false>), grid, dim3(256), smem, st,
                       tables, ids, vnorm, s.seq_lens, s.Hkv, s.Nmax, P, kpb, scores);
}

hipError_t launch_score_softlsh(const hst_shape& s, const float* tables, int L, int P,
                                const uint8_t* ids, const void* vnorm, int norm_dtype,
                                float* scores, hipStream_t st) {
  const int kpb = 2048;
  dim3 grid((s.Nmax + kpb - 1) / kpb, s.B * s.Hkv);
  const size_t smem = sizeof(float) * (static_cast<size_t>(L) << P);
  const bool f16 = norm_dtype == HST_F16;
  switch (L) {
    case 4: launch_soft_t<4, 1>(grid, smem, st, f16, tables, ids, vnorm, s, P, kpb, scores); break;
    case 8: launch_soft_t<8, 1>(grid, smem, st, f16, tables, ids, vnorm, s, P, kpb, scores); break;
    case 16: launch_soft_t<16, 1>(grid, smem, st, f16, tables, ids, vnorm, s, P, kpb, scores); break;
    case 32: launch_soft_t<16, 2>(grid, smem, st, f16, tables, ids, vnorm, s, P, kpb, scores); break;
    case 64: launch_soft_t<16, 4>(grid, smem, st, f16, tables, ids, vnorm, s, P, kpb, scores); break;
    case 128: launch_soft_t<16, 8>(grid, smem, st, f16, tables, ids, vnorm, s, P, kpb, scores); break;
    default:
      if (f16)
        hipLaunchKernelGGL((score_softlsh_anyL_kernel<true>), grid, dim3(256), smem, st, tables,
                           ids, vnorm, s.seq_lens, s.Hkv, s.Nmax, L, P, kpb, scores);
      else
        hipLaunchKernelGGL((score_softlsh_anyL_kernel<false>), grid, dim3(256), smem, st, tables,
                           ids, vnorm, s.seq_lens, s.Hkv, s.Nmax, L, P, kpb, scores);
  }
  return hipGetLastError();
}

hipError_t launch_score_hamming(const hst_shape& s, const uint32_t* qcodes,
                                const uint32_t* codes, int32_t* scores, hipStream_t st) {
  const int kpb = 4096;
  dim3 grid((s.Nmax + kpb - 1) / kpb, s.B * s.Hkv);
  hipLaunchKernelGGL(score_hamming_kernel, grid, dim3(256), 0, st, qcodes,
                     reinterpret_cast<const uint4*>(codes), s.seq_lens, s.Hq, s.Hkv, s.Nmax, kpb,
                     scores);
  return hipGetLastError();
}

}  // namespace hst
