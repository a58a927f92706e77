// Binary-code scoring for code lengths other than 128 bits (64, 256).
// HATA explainer page, section 3: queries and keys become binary codes and
// keys are ranked by comparing codes.  The 128-bit codes run through the
// fused decode path; other lengths (the code-length trade-off of the same
// page, section 1) are scored here: the query codes come from the key
// hashing applied to the queries (so their signs are exact in the same
// way), and hamming_scan_kernel scores every key against the G query codes
// of its kv head, one key per thread, W 32-bit words per code.
#include "hst_common.h"
#include "hst_fused.h"
#include "hst_launch.h"

namespace hst {

constexpr int kHamNT = 1024;

// scores[bh][j] = sum_g (32 W - popcount(qc[b][h][g] ^ kc[bh][j])) for j < N_b.
template <int W>
__global__ void __launch_bounds__(kHamNT)
hamming_scan_kernel(const uint32_t* __restrict__ qcodes, const uint32_t* __restrict__ kcodes,
                    const int32_t* __restrict__ seq_lens, int Hkv, int G, int Nmax,
                    int32_t* __restrict__ scores) {
  __shared__ uint32_t qc[8 * W];
  const int bh = blockIdx.y, b = bh / Hkv, t = threadIdx.x;
  const int n = seq_len(seq_lens, b, Nmax);
  if (t < G * W) qc[t] = qcodes[static_cast<long long>(bh) * G * W + t];
  const int j = blockIdx.x * kHamNT + t;
  uint32_t kc[W];
  if (j < n) {
    const uint32_t* kp = kcodes + (static_cast<long long>(bh) * Nmax + j) * W;
#pragma unroll
    for (int w = 0; w < W; ++w) kc[w] = kp[w];
  }
  __syncthreads();
  if (j >= n) return;
  int s = 0;
  for (int g = 0; g < G; ++g) {
    int ham = 0;
#pragma unroll
    for (int w = 0; w < W; ++w) ham += __popc(qc[g * W + w] ^ kc[w]);
    s += 32 * W - ham;
  }
  scores[static_cast<long long>(bh) * Nmax + j] = s;
}

hipError_t launch_hamming_scan(const hst_shape& s, int code_bits, const uint32_t* qcodes,
                               const uint32_t* kcodes, int32_t* scores, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((s.Nmax + kHamNT - 1) / kHamNT),
                  static_cast<unsigned>(s.B * s.Hkv));
  const int G = s.Hq / s.Hkv;
  switch (code_bits) {
    case 64:
      hipLaunchKernelGGL(hamming_scan_kernel<2>, grid, dim3(kHamNT), 0, st, qcodes, kcodes,
                         s.seq_lens, s.Hkv, G, s.Nmax, scores);
      break;
    case 128:
      hipLaunchKernelGGL(hamming_scan_kernel<4>, grid, dim3(kHamNT), 0, st, qcodes, kcodes,
                         s.seq_lens, s.Hkv, G, s.Nmax, scores);
      break;
    default:
      hipLaunchKernelGGL(hamming_scan_kernel<8>, grid, dim3(kHamNT), 0, st, qcodes, kcodes,
                         s.seq_lens, s.Hkv, G, s.Nmax, scores);
      break;
  }
  return hipGetLastError();
}

// Query codes [B][Hkv][G][W]: the queries [B][Hq][d] viewed as a cache of
// G keys per kv head, hashed with the keys' projection.
hipError_t launch_query_codes(const hst_shape& s, const void* q, const void* R, int code_bits,
                              uint32_t* qcodes, hipStream_t st) {
  hst_shape qs = s;
  qs.Nmax = s.Hq / s.Hkv;
  qs.seq_lens = nullptr;
  return launch_hash_binary(qs, q, R, code_bits, qcodes, st);
}

}  // namespace hst
