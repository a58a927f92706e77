// Per-step query preprocessing.
//  * Soft bucket assignment tables (SOCKET overview page, "Core mechanism:
//    soft LSH", item 2): the normalised query is projected on every
//    hyperplane and each table gets a temperature softmax over all of its
//    2^P buckets; the G query heads of a kv head are summed into one table.
//    The softmax of a logit linear in the bucket's sign pattern factorises
//    into a product of P logistic terms, sigma(2 s_p z_p / tau), which is how
//    it is evaluated here (in float64, rounded once to float32).
//  * Binary query codes (HATA explainer page, section 3).
#include "hst_common.h"
#include "hst_launch.h"

namespace hst {

constexpr int kTablesPerBlockMaxDots = 256;

template <typename T>
__global__ void __launch_bounds__(256)
query_tables_kernel(const T* __restrict__ q, const T* __restrict__ W, int Hq, int Hkv,
                    int d, int L, int P, int TL, double inv_tau,
                    float* __restrict__ tables) {
  extern __shared__ double smem[];
  const int G = Hq / Hkv;
  const int bh = blockIdx.y;
  const int b = bh / Hkv, h = bh % Hkv;
  const int l0 = blockIdx.x * TL;
  const int tl = min(TL, L - l0);
  const int nb = 1 << P;
  double* qn = smem;                 // [G][d]
  double* sp1 = qn + G * d;          // [G][TL][P] probability that bit p is set
  double* sp0 = sp1 + G * TL * P;    // [G][TL][P] probability that bit p is clear
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwave = blockDim.x >> 6;

  for (int g = wave; g < G; g += nwave) {
    const T* qr = q + (static_cast<long long>(b) * Hq + h * G + g) * d;
    double ss = 0.0;
    for (int c = lane; c < d; c += 64) {
      double v = to_f64(qr[c]);
      qn[g * d + c] = v;
      ss += v * v;
    }
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const double nrm = sqrt(ss);
    for (int c = lane; c < d; c += 64) qn[g * d + c] = nrm > 0.0 ? qn[g * d + c] / nrm : 0.0;
  }
  __syncthreads();

  const int ndot = G * tl * P;
  for (int t = threadIdx.x; t < ndot; t += blockDim.x) {
    const int g = t / (tl * P);
    const int r = t % (tl * P);  // = lt * P + p
    const T* wr = W + (static_cast<long long>(h) * L * P + static_cast<long long>(l0) * P + r) * d;
    const double* qq = qn + g * d;
    double z = 0.0;
    for (int c = 0; c < d; ++c) z += to_f64(wr[c]) * qq[c];
    const double x = 2.0 * z * inv_tau;
    sp1[g * TL * P + r] = 1.0 / (1.0 + exp(-x));
    sp0[g * TL * P + r] = 1.0 / (1.0 + exp(x));
  }
  __syncthreads();

  const int nent = tl * nb;
  for (int t = threadIdx.x; t < nent; t += blockDim.x) {
    const int lt = t >> P;
    const int c = t & (nb - 1);
    double acc = 0.0;
    for (int g = 0; g < G; ++g) {
      const double* s1 = sp1 + (g * TL + lt) * P;
      const double* s0 = sp0 + (g * TL + lt) * P;
      double pr = 1.0;
      for (int p = 0; p < P; ++p) pr *= ((c >> p) & 1) ? s1[p] : s0[p];
      acc += pr;
    }
    tables[(static_cast<long long>(bh) * L + l0 + lt) * nb + c] = static_cast<float>(acc);
  }
}

template <typename T>
__global__ void __launch_bounds__(128)
query_codes_kernel(const T* __restrict__ q, const T* __restrict__ R, int Hq, int Hkv, int d,
                   uint32_t* __restrict__ qcodes) {
  const int bq = blockIdx.x;  // b * Hq + hq
  const int hq = bq % Hq;
  const int G = Hq / Hkv;
  const int h = hq / G;
  const int i = threadIdx.x;
  const bool bit = dot_nonneg_exact(R + (static_cast<long long>(h) * 128 + i) * d,
                                    q + static_cast<long long>(bq) * d, d);
  const unsigned long long m = __ballot(bit);
  if ((i & 63) == 0) {
    qcodes[static_cast<long long>(bq) * 4 + (i >> 6) * 2] = static_cast<uint32_t>(m);
    qcodes[static_cast<long long>(bq) * 4 + (i >> 6) * 2 + 1] = static_cast<uint32_t>(m >> 32);
  }
}

size_t query_tables_smem(const hst_shape& s, int P, int TL) {
  const int G = s.Hq / s.Hkv;
  return sizeof(double) * (static_cast<size_t>(G) * s.d + 2ull * G * TL * P);
}

int query_tables_tl(const hst_shape& s, int L, int P) {
  const int G = s.Hq / s.Hkv;
  int tl = kTablesPerBlockMaxDots / (G * P);
  if (tl < 1) tl = 1;
  if (tl > L) tl = L;
  return tl;
}

hipError_t launch_query_tables(const hst_shape& s, const void* q, const void* W, int L, int P,
                               float tau, float* tables, hipStream_t st) {
  const int TL = query_tables_tl(s, L, P);
  dim3 grid((L + TL - 1) / TL, s.B * s.Hkv);
  const size_t smem = query_tables_smem(s, P, TL);
  const double inv_tau = 1.0 / static_cast<double>(tau);
  if (s.kv_dtype == HST_F32)
    hipLaunchKernelGGL(query_tables_kernel<float>, grid, dim3(256), smem, st,
                       static_cast<const float*>(q), static_cast<const float*>(W), s.Hq, s.Hkv,
                       s.d, L, P, TL, inv_tau, tables);
  else
    hipLaunchKernelGGL(query_tables_kernel<bf16>, grid, dim3(256), smem, st,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(W), s.Hq, s.Hkv,
                       s.d, L, P, TL, inv_tau, tables);
  return hipGetLastError();
}

hipError_t launch_query_codes(const hst_shape& s, const void* q, const void* R,
                              uint32_t* qcodes, hipStream_t st) {
  dim3 grid(s.B * s.Hq);
  if (s.kv_dtype == HST_F32)
    hipLaunchKernelGGL(query_codes_kernel<float>, grid, dim3(128), 0, st,
                       static_cast<const float*>(q), static_cast<const float*>(R), s.Hq, s.Hkv,
                       s.d, qcodes);
  else
    hipLaunchKernelGGL(query_codes_kernel<bf16>, grid, dim3(128), 0, st,
                       static_cast<const bf16*>(q), static_cast<const bf16*>(R), s.Hq, s.Hkv,
                       s.d, qcodes);
  return hipGetLastError();
}

}  // namespace hst
