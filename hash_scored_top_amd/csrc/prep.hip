// Per-step query preprocessing, one workgroup per (sequence, kv head).
//
// Soft-LSH (SOCKET overview page, "Core mechanism: soft LSH", item 2): the
// normalised query of each of the G query heads is projected on every
// hyperplane (float64: z = W q_hat), and each table's bucket probabilities
// are the temperature softmax over all 2^P buckets of sum_p s_p z_p / tau.
// That softmax of a logit linear in the bucket's sign pattern factorises into
// a product of logistic terms sigma(2 s_p z_p / tau); the product over the P
// planes is formed as (low half of the bits) x (high half), so a 256-bucket
// table costs 16 + 16 partial products instead of 256 x 8 multiplies.  The G
// heads are summed into one float32 table per kv head, stored bucket-major.
//
// Binary codes (HATA explainer page, section 3): the G query codes, each bit
// the exact sign of a projection.
//
// When a top-k follows, the same workgroup scores a stratified sample of the
// keys and derives the candidate threshold theta the scan filters with.
#include "fused_device.h"
#include "hst_launch.h"

namespace hst {

constexpr int kPrepNT = 1024;

// LDS map of the soft-LSH prep (bytes):
//   [0, 128K)       W row chunk (rows padded by 16 bytes); later T (fp32, <= 64 KB)
//                   and then the sample keys (16 KB) + histogram (8 KB) at 64K
//   [64K, 96K)      z [G][L*P] fp64 (written once W^T is dead)
//   [96K, 112K)     logistic pairs of the current query head [L*P][2] fp64
//   [112K, 144K)    low/high half products of the current head [L][2^plo + 2^phi]
//   [144K, 144K + 8*G*d)  q_hat [G][d] fp64 (G*d <= 1024)
constexpr int kPrepW = 0, kPrepZ = 65536, kPrepSig = 98304, kPrepHalf = 114688, kPrepQ = 147456;
static int prep_soft_smem(int G, int d) { return kPrepQ + 8 * G * d; }

template <typename T>
__global__ void __launch_bounds__(kPrepNT)
prep_softlsh_kernel(const T* __restrict__ q, const T* __restrict__ W,
                    const uint8_t* __restrict__ ids, const void* __restrict__ vnorm, int norm_f16,
                    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_seq,
                    FusedArgs a) {
  constexpr int NT = kPrepNT;
  extern __shared__ __align__(16) unsigned char sm[];
  __shared__ BlockScratch<NT> sc;
  const int G = a.Hq / a.Hkv, d = a.d, L = a.L, P = a.P, LP = L * P, nb = 1 << P;
  const int plo = P < 4 ? P : 4, phi = P - plo;
  const int nlo = 1 << plo, nhi = 1 << phi;
  const int bh = blockIdx.x, b = bh / a.Hkv, h = bh % a.Hkv;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  double* qn = reinterpret_cast<double*>(sm + kPrepQ);
  double* z = reinterpret_cast<double*>(sm + kPrepZ);
  double* sg = reinterpret_cast<double*>(sm + kPrepSig);
  double* half = reinterpret_cast<double*>(sm + kPrepHalf);
  T* wt = reinterpret_cast<T*>(sm + kPrepW);
  float* tl = reinterpret_cast<float*>(sm + kPrepW);

  // 1. normalised queries
  for (int g = wave; g < G; g += NT / 64) {
    const T* qr = q + (static_cast<long long>(b) * a.Hq + h * G + g) * d;
    double ss = 0.0;
    for (int c = lane; c < d; c += 64) {
      const double v = to_f64(qr[c]);
      qn[g * d + c] = v;
      ss += v * v;
    }
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const double nrm = sqrt(ss);
    for (int c = lane; c < d; c += 64) qn[g * d + c] = nrm > 0.0 ? qn[g * d + c] / nrm : 0.0;
  }

  // 2. projections z[g][r] = W[h][r] . q_hat[g].  W rows are staged in LDS
  //    row-major with a 16-byte pad per row (16-byte reads of 64 lanes then
  //    spread over all banks), a chunk of rows at a time; each thread owns the
  //    pairs (g, r) = (t / TPG, r0 + t % TPG + k * TPG) and keeps z in registers
  constexpr int kMaxPairs = 4;  // G * L * P <= 4 * NT
  constexpr int E = 16 / static_cast<int>(sizeof(T));
  const int rowb = d * static_cast<int>(sizeof(T)) + 16;      // padded row bytes
  const int rc = 131072 / rowb;                                // rows per chunk
  const int tpg = NT / G;                                      // threads per query head
  const int myg = t / tpg, myr = t % tpg;
  double zr[kMaxPairs];
#pragma unroll
  for (int u = 0; u < kMaxPairs; ++u) zr[u] = 0.0;
  const T* wh = W + static_cast<long long>(h) * LP * d;
  for (int r0 = 0; r0 < LP; r0 += rc) {
    const int rn = min(rc, LP - r0);
    __syncthreads();
    const int nblk = rn * (d / E);
    for (int i0 = 0; i0 < nblk; i0 += NT * 4) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = i0 + u * NT + t;
        if (e < nblk) v[u] = reinterpret_cast<const u32x4*>(wh + static_cast<long long>(r0) * d)[e];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = i0 + u * NT + t;
        if (e < nblk) {
          const int r = e / (d / E), cb = e % (d / E);
          *reinterpret_cast<u32x4*>(sm + kPrepW + r * rowb + cb * 16) = v[u];
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kMaxPairs; ++u) {
      const int r = myr + u * tpg;  // row of this pair
      if (myg < G && r >= r0 && r < r0 + rn && r < LP) {
        const unsigned char* wr = sm + kPrepW + (r - r0) * rowb;
        const double* qq = qn + myg * d;
        double acc = 0.0;
        for (int cb = 0; cb < d / E; ++cb) {
          const u32x4 wv = *reinterpret_cast<const u32x4*>(wr + cb * 16);
          const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
          for (int x = 0; x < E; ++x) {
            float f;
            if (sizeof(T) == 2) f = (x & 1) ? bf16_hi(ww[x >> 1]) : bf16_lo(ww[x >> 1]);
            else f = __uint_as_float(ww[x]);
            acc += static_cast<double>(f) * qq[cb * E + x];
          }
        }
        zr[u] = acc;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kMaxPairs; ++u) {
    const int r = myr + u * tpg;
    if (myg < G && r < LP) z[myg * LP + r] = zr[u];
  }
  __syncthreads();

  // 3. tables: for each query head, logistic pairs -> half products -> sum.
  //    sg[(bit*P + p)*L + l] and half[c*L + l] keep consecutive threads on
  //    consecutive tables l (conflict-free LDS).
  constexpr int kMaxEnt = 16;  // nb * L <= 16 * NT
  const int nent = nb * L;
  const int hw = nlo + nhi;
  double acc[kMaxEnt];
#pragma unroll
  for (int u = 0; u < kMaxEnt; ++u) acc[u] = 0.0;
  for (int g = 0; g < G; ++g) {
    for (int e = t; e < LP; e += NT) {
      const int p = e / L, l = e % L;
      const double x = 2.0 * z[g * LP + l * P + p] * a.inv_tau;
      sg[(0 * P + p) * L + l] = 1.0 / (1.0 + exp(x));   // bit clear
      sg[(1 * P + p) * L + l] = 1.0 / (1.0 + exp(-x));  // bit set
    }
    __syncthreads();
    for (int e = t; e < hw * L; e += NT) {
      const int c = e / L, l = e % L;
      double pr = 1.0;
      if (c < nlo) {
        for (int p = 0; p < plo; ++p) pr *= sg[(((c >> p) & 1) * P + p) * L + l];
      } else {
        const int ch = c - nlo;
        for (int p = 0; p < phi; ++p) pr *= sg[(((ch >> p) & 1) * P + plo + p) * L + l];
      }
      half[e] = pr;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kMaxEnt; ++u) {
      const int e = t + u * NT;
      if (e < nent) {
        const int c = e / L, l = e % L;
        acc[u] += half[(c & (nlo - 1)) * L + l] * half[(nlo + (c >> plo)) * L + l];
      }
    }
    __syncthreads();
  }
  // bucket-major float32 table, to HBM and (for the sample) to LDS
  float* Tg = a.tables + static_cast<long long>(bh) * nent;
#pragma unroll
  for (int u = 0; u < kMaxEnt; ++u) {
    const int e = t + u * NT;
    if (e < nent) {
      const float v = static_cast<float>(acc[u]);
      Tg[e] = v;
      tl[e] = v;
    }
  }
  if (a.sample == 0) return;  // tables only

  // 4. sample scores -> candidate threshold
  __syncthreads();
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int S_eff = a.sample > n ? n : a.sample;
  const int k_eff = keff_of(a.kcap, k_per_seq, b, n);
  uint2* sk = reinterpret_cast<uint2*>(sm + 65536);
  uint32_t* hist = reinterpret_cast<uint32_t*>(sm + 65536 + 16384);
  uint32_t theta = 0u;
  if (S_eff > 0 && k_eff > 0) {
    const long long base = static_cast<long long>(bh) * a.Nmax;
    const uint32_t idm = static_cast<uint32_t>(nb - 1);
    for (int i0 = 0; i0 < S_eff; i0 += NT * 2) {
      int jj[2];
      float vn[2];
      uint4 w4[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * NT + t;
        jj[u] = i < S_eff ? sample_pos(i, S_eff, n) : 0;
        if (i < S_eff) {
          const long long o = base + jj[u];
          vn[u] = norm_f16 ? f16_bits_to_f32(static_cast<const uint16_t*>(vnorm)[o])
                           : static_cast<const float*>(vnorm)[o];
          if (L == 64) {
#pragma unroll
            for (int x = 0; x < 4; ++x) w4[u][x] = reinterpret_cast<const uint4*>(ids + o * 64)[x];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * NT + t;
        if (i >= S_eff) continue;
        float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
        if (L == 64) {
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const uint32_t wd[4] = {w4[u][x].x, w4[u][x].y, w4[u][x].z, w4[u][x].w};
#pragma unroll
            for (int y = 0; y < 16; y += 4) {
              const int l = x * 16 + y;
              const uint32_t wv = wd[y >> 2];
              s0 += tl[((wv) & idm) * 64 + l];
              s1 += tl[((wv >> 8) & idm) * 64 + l + 1];
              s2 += tl[((wv >> 16) & idm) * 64 + l + 2];
              s3 += tl[((wv >> 24) & idm) * 64 + l + 3];
            }
          }
        } else {
          const uint8_t* row = ids + (base + jj[u]) * L;
          for (int l = 0; l < L; ++l) s0 += tl[(row[l] & idm) * L + l];
        }
        sk[i] = make_uint2(order_key_f32(((s0 + s1) + (s2 + s3)) * vn[u]), static_cast<uint32_t>(jj[u]));
      }
    }
    __syncthreads();
    const int r = sample_rank(k_eff, n, S_eff);
    theta = r >= S_eff ? 0u : block_rank_lower_bound<NT>(PairSrc{sk}, S_eff, r, hist, sc);
  }
  if (t == 0) {
    HeadState* hs = a.heads + bh;
    hs->theta = theta;
    hs->k_eff = k_eff;
    hs->n = n;
  }
}

// Exact sign of sum_c R^T[c][i] * x[c] for LDS-resident float data (values
// exact in float64; see dot_nonneg_exact).
__device__ __forceinline__ bool col_dot_nonneg(const float* rt, int stride, int i, const float* x,
                                               int d) {
  double s = 0.0, sa = 0.0;
  for (int c = 0; c < d; ++c) {
    const double p = static_cast<double>(rt[c * stride + i]) * static_cast<double>(x[c]);
    s += p;
    sa += fabs(p);
  }
  if (fabs(s) > 2.0 * d * 0x1p-53 * sa) return s >= 0.0;
  // rare: gather the column and decide exactly
  float col[256];
  for (int c = 0; c < d; ++c) col[c] = rt[c * stride + i];
  return expansion_dot_nonneg(col, x, d);
}

// Binary-code prep: query codes for the G heads (+ the key sample).
// LDS: R^T [d][128] float (64 KB at d = 128), q [G][d] float, sample keys.
template <typename T>
__global__ void __launch_bounds__(kPrepNT)
prep_hamming_kernel(const T* __restrict__ q, const T* __restrict__ R,
                    const uint4* __restrict__ codes, const int32_t* __restrict__ seq_lens,
                    const int32_t* __restrict__ k_per_seq, FusedArgs a) {
  constexpr int NT = kPrepNT;
  extern __shared__ __align__(16) unsigned char sm[];
  __shared__ BlockScratch<NT> sc;
  __shared__ uint32_t qc[64 * 4];
  const int G = a.Hq / a.Hkv, d = a.d;
  const int bh = blockIdx.x, b = bh / a.Hkv, h = bh % a.Hkv;
  const int t = threadIdx.x, lane = t & 63;
  float* rt = reinterpret_cast<float*>(sm);      // [d][128]
  float* ql = rt + d * 128;                       // [G][d]
  uint2* sk = reinterpret_cast<uint2*>(sm + hst_align16(static_cast<size_t>(d * 128 + G * d) * 4));
  uint32_t* hist = reinterpret_cast<uint32_t*>(sk + kSample);
  const T* rs = R + static_cast<long long>(h) * 128 * d;
  {
    // 16-byte loads, consecutive threads on consecutive rows i (conflict-free
    // transposed LDS writes), all loads of a thread issued together
    constexpr int E = 16 / static_cast<int>(sizeof(T));
    const int nblk = 128 * (d / E);
    for (int i0 = 0; i0 < nblk; i0 += NT * 4) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = i0 + u * NT + t;
        if (e < nblk) v[u] = *reinterpret_cast<const uint4*>(rs + static_cast<long long>(e % 128) * d + (e / 128) * E);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = i0 + u * NT + t;
        if (e < nblk) {
          const T* pv = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
          for (int x = 0; x < E; ++x) rt[((e / 128) * E + x) * 128 + (e % 128)] = to_f32(pv[x]);
        }
      }
    }
  }
  const T* qs = q + (static_cast<long long>(b) * a.Hq + h * G) * d;
  for (int e = t; e < G * d; e += NT) ql[e] = to_f32(qs[e]);
  __syncthreads();
  for (int e = t; e < G * 128; e += NT) {  // trip count uniform per wave
    const int g = e >> 7, i = e & 127;
    const bool bit = col_dot_nonneg(rt, 128, i, ql + g * d, d);
    const unsigned long long m = __ballot(bit);
    if (lane == 0) {
      qc[g * 4 + (i >> 6) * 2] = static_cast<uint32_t>(m);
      qc[g * 4 + (i >> 6) * 2 + 1] = static_cast<uint32_t>(m >> 32);
    }
  }
  __syncthreads();
  for (int e = t; e < G * 4; e += NT) a.qcodes[static_cast<long long>(bh) * G * 4 + e] = qc[e];
  if (a.sample == 0) return;
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int S_eff = a.sample > n ? n : a.sample;
  const int k_eff = keff_of(a.kcap, k_per_seq, b, n);
  uint32_t theta = 0u;
  if (S_eff > 0 && k_eff > 0) {
    for (int i0 = 0; i0 < S_eff; i0 += NT * 2) {
      uint4 cv[2];
      int jj[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * NT + t;
        jj[u] = i < S_eff ? sample_pos(i, S_eff, n) : 0;
        if (i < S_eff) cv[u] = codes[static_cast<long long>(bh) * a.Nmax + jj[u]];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * NT + t;
        if (i >= S_eff) continue;
        int ham = 0;
        for (int g = 0; g < G; ++g)
          ham += __popc(cv[u].x ^ qc[4 * g]) + __popc(cv[u].y ^ qc[4 * g + 1]) +
                 __popc(cv[u].z ^ qc[4 * g + 2]) + __popc(cv[u].w ^ qc[4 * g + 3]);
        sk[i] = make_uint2(order_key_i32(128 * G - ham), static_cast<uint32_t>(jj[u]));
      }
    }
    __syncthreads();
    const int r = sample_rank(k_eff, n, S_eff);
    theta = r >= S_eff ? 0u : block_rank_lower_bound<NT>(PairSrc{sk}, S_eff, r, hist, sc);
  }
  if (t == 0) {
    HeadState* hs = a.heads + bh;
    hs->theta = theta;
    hs->k_eff = k_eff;
    hs->n = n;
  }
}

size_t prep_hamming_smem(int G, int d) {
  return hst_align16(static_cast<size_t>(d * 128 + G * d) * 4) + kSample * 8 + 2048 * 4;
}

__device__ __forceinline__ uint32_t order_key_of(float v) { return order_key_f32(v); }
__device__ __forceinline__ uint32_t order_key_of(int32_t v) { return order_key_i32(v); }

// Threshold for a top-k over given scores.
template <typename KT>
__global__ void __launch_bounds__(kPrepNT)
prep_given_kernel(const KT* __restrict__ scores, const int32_t* __restrict__ seq_lens,
                  const int32_t* __restrict__ k_per_seq, FusedArgs a) {
  constexpr int NT = kPrepNT;
  __shared__ uint2 sk[kSample];
  __shared__ uint32_t hist[2048];
  __shared__ BlockScratch<NT> sc;
  const int bh = blockIdx.x, b = bh / a.Hkv;
  const int t = threadIdx.x;
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int S_eff = a.sample > n ? n : a.sample;
  const int k_eff = keff_of(a.kcap, k_per_seq, b, n);
  uint32_t theta = 0u;
  if (S_eff > 0 && k_eff > 0) {
    for (int i0 = 0; i0 < S_eff; i0 += NT * 2) {
      KT v[2];
      int jj[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * NT + t;
        jj[u] = i < S_eff ? sample_pos(i, S_eff, n) : 0;
        if (i < S_eff) v[u] = scores[static_cast<long long>(bh) * a.Nmax + jj[u]];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * NT + t;
        if (i < S_eff) sk[i] = make_uint2(order_key_of(v[u]), static_cast<uint32_t>(jj[u]));
      }
    }
    __syncthreads();
    const int r = sample_rank(k_eff, n, S_eff);
    theta = r >= S_eff ? 0u : block_rank_lower_bound<NT>(PairSrc{sk}, S_eff, r, hist, sc);
  }
  if (t == 0) {
    HeadState* hs = a.heads + bh;
    hs->theta = theta;
    hs->k_eff = k_eff;
    hs->n = n;
  }
}

hipError_t launch_prep_soft(const hst_shape& s, const FusedArgs& a, const void* q, const void* W,
                            const uint8_t* ids, const void* vnorm, int norm_f16,
                            const int32_t* kps, hipStream_t st) {
  dim3 grid(s.B * s.Hkv);
  const int kPrepSmem = prep_soft_smem(s.Hq / s.Hkv, s.d);
  if (s.kv_dtype == HST_F32) {
    auto kern = prep_softlsh_kernel<float>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kPrepSmem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kPrepNT), kPrepSmem, st, static_cast<const float*>(q),
                       static_cast<const float*>(W), ids, vnorm, norm_f16, s.seq_lens, kps, a);
  } else {
    auto kern = prep_softlsh_kernel<bf16>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kPrepSmem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kPrepNT), kPrepSmem, st, static_cast<const bf16*>(q),
                       static_cast<const bf16*>(W), ids, vnorm, norm_f16, s.seq_lens, kps, a);
  }
  return hipGetLastError();
}

hipError_t launch_prep_hamming(const hst_shape& s, const FusedArgs& a, const void* q, const void* R,
                               const uint32_t* codes, const int32_t* kps, hipStream_t st) {
  dim3 grid(s.B * s.Hkv);
  const int smem = static_cast<int>(prep_hamming_smem(s.Hq / s.Hkv, s.d));
  if (s.kv_dtype == HST_F32) {
    auto kern = prep_hamming_kernel<float>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kPrepNT), smem, st, static_cast<const float*>(q),
                       static_cast<const float*>(R), reinterpret_cast<const uint4*>(codes),
                       s.seq_lens, kps, a);
  } else {
    auto kern = prep_hamming_kernel<bf16>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kPrepNT), smem, st, static_cast<const bf16*>(q),
                       static_cast<const bf16*>(R), reinterpret_cast<const uint4*>(codes),
                       s.seq_lens, kps, a);
  }
  return hipGetLastError();
}

hipError_t launch_prep_given(const hst_shape& s, const FusedArgs& a, int score_dtype,
                             const void* scores, const int32_t* kps, hipStream_t st) {
  dim3 grid(s.B * s.Hkv);
  if (score_dtype == HST_F32)
    hipLaunchKernelGGL(prep_given_kernel<float>, grid, dim3(kPrepNT), 0, st,
                       static_cast<const float*>(scores), s.seq_lens, kps, a);
  else
    hipLaunchKernelGGL(prep_given_kernel<int32_t>, grid, dim3(kPrepNT), 0, st,
                       static_cast<const int32_t*>(scores), s.seq_lens, kps, a);
  return hipGetLastError();
}

}  // namespace hst
