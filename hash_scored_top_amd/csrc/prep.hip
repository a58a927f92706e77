// Per-step query preprocessing and the candidate threshold of the top-k.
//
// prep: X >= 8 workgroups per (sequence, kv head).
//  * Soft-LSH (SOCKET overview page, "Core mechanism: soft LSH", item 2):
//    workgroup j builds the query tables of hash tables [8j, 8j + 8).  The
//    normalised query of each of the G query heads is projected on the
//    hyperplanes of those tables (float64: z = W q_hat), and a table's bucket
//    probabilities are the temperature softmax over all 2^P buckets of
//    sum_p s_p z_p / tau.  That softmax of a logit linear in the bucket's sign
//    pattern factorises into a product of logistic terms sigma(2 s_p z_p / tau);
//    the product over the P planes is formed as (low half of the bits) x (high
//    half), so a 256-bucket table costs 16 + 16 partial products instead of
//    256 x 8 multiplies.  The G heads are summed into one float32 table per kv
//    head, stored bucket-major.
//  * Binary codes (HATA explainer page, section 3): workgroup j computes bits
//    [16j, 16j + 16) of the G query codes, each the exact sign of a projection.
//  * When a top-k follows, every workgroup also copies its share of a
//    stratified key sample (kSample keys per head) into a compact buffer, so
//    the scattered reads are spread over many compute units.
//
// A small kernel ahead of the scan derives the candidate threshold from that
// sample (scan.hip); the scan keeps the keys scoring >= theta.  theta only bounds the work of the
// selection: the selected set never depends on it.
#include "fused_device.h"
#include "hst_launch.h"

namespace hst {

constexpr int kPrepNT = 256;
constexpr int kThrNT = 1024;
constexpr int kTabGroup = 8;  // hash tables per prep workgroup

static int prep_blocks_soft(int L) {
  const int g = (L + kTabGroup - 1) / kTabGroup;
  return g > kPrepBlocks ? g : kPrepBlocks;
}

// ---------------------------------------------------------------------------
// sample gather

struct SampleShare {
  int n, S, i0, i1;  // context length, sample size, this workgroup's entries
};

__device__ __forceinline__ SampleShare sample_share(const FusedArgs& a, const int32_t* seq_lens,
                                                    const int32_t* k_per_seq, int b) {
  SampleShare s{};
  s.n = seq_len(seq_lens, b, a.Nmax);
  s.S = a.sample > s.n ? s.n : a.sample;
  if (a.sample == 0 || keff_of(a.kcap, k_per_seq, b, s.n) == 0) s.S = 0;
  const int X = gridDim.x, j = blockIdx.x;
  s.i0 = static_cast<int>(static_cast<long long>(j) * s.S / X);
  s.i1 = static_cast<int>(static_cast<long long>(j + 1) * s.S / X);
  return s;  // i1 - i0 <= kSample / kPrepBlocks <= blockDim.x
}

// Rows of `rb` bytes (rb a multiple of 16, at most 128): one sampled key per
// thread; the loads are issued here and the stores done by store().
struct RowGather {
  u32x4 v[8];
  int nv;
  bool on;
  long long dst;
  __device__ __forceinline__ void load(const uint8_t* src_rows, long long row, int rb, bool active,
                                       long long dst_row) {
    nv = rb >> 4;
    on = active;
    dst = dst_row;
    if (!on) return;
    const u32x4* p = reinterpret_cast<const u32x4*>(src_rows + row * rb);
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (x < nv) v[x] = p[x];
  }
  __device__ __forceinline__ void store(uint8_t* dst_rows, int rb) const {
    if (!on) return;
    u32x4* p = reinterpret_cast<u32x4*>(dst_rows + dst * rb);
#pragma unroll
    for (int x = 0; x < 8; ++x)
      if (x < nv) p[x] = v[x];
  }
};

// ---------------------------------------------------------------------------
// soft-LSH tables (+ sample)

struct TabSmem {
  int wrows, qn, z, sg, half, bytes;
};

// LDS map of one table group: W rows (padded by 16 bytes), q_hat [G][d],
// z [G][8P], logistic pairs [G][2][P][8], half products [G][hw][8] (float64).
__host__ __device__ inline TabSmem tab_smem(int G, int d, int esize, int P) {
  const int plo = P < 4 ? P : 4;
  const int hw = (1 << plo) + (1 << (P - plo));
  TabSmem m{};
  m.wrows = 0;
  m.qn = m.wrows + kTabGroup * P * (d * esize + 16);
  m.z = m.qn + G * d * 8;
  m.sg = m.z + G * kTabGroup * P * 8;
  m.half = m.sg + G * 2 * P * kTabGroup * 8;
  m.bytes = m.half + G * hw * kTabGroup * 8;
  return m;
}

template <typename T>
__global__ void __launch_bounds__(kPrepNT)
prep_tables_kernel(const T* __restrict__ q, const T* __restrict__ W, const uint8_t* __restrict__ ids,
                   const void* __restrict__ vnorm, int norm_f16, const int32_t* __restrict__ seq_lens,
                   const int32_t* __restrict__ k_per_seq, FusedArgs a) {
  constexpr int NT = kPrepNT;
  constexpr int E = 16 / static_cast<int>(sizeof(T));
  extern __shared__ __align__(16) unsigned char sm[];
  const int G = a.Hq / a.Hkv, d = a.d, L = a.L, P = a.P, nb = 1 << P;
  const int bh = blockIdx.y, b = bh / a.Hkv, h = bh % a.Hkv, j = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;

  // sample share: loads issued now, stored after the table work
  const SampleShare ss = sample_share(a, seq_lens, k_per_seq, b);
  const int si = ss.i0 + t;
  const bool son = si < ss.i1;
  const long long krow = static_cast<long long>(bh) * a.Nmax + (son ? sample_pos(si, ss.S, ss.n) : 0);
  const long long drow = static_cast<long long>(bh) * kSample + si;
  RowGather rg;
  const bool vec = (L & 15) == 0;
  rg.load(ids, krow, L, son && vec, drow);
  float vn = 0.f;
  if (son) vn = norm_f16 ? f16_bits_to_f32(static_cast<const uint16_t*>(vnorm)[krow])
                         : static_cast<const float*>(vnorm)[krow];

  const int l0 = j * kTabGroup;
  if (l0 < L) {
    const int lg = min(kTabGroup, L - l0), R = lg * P;
    const int plo = P < 4 ? P : 4, phi = P - plo, nlo = 1 << plo, hw = nlo + (1 << phi);
    const TabSmem mp = tab_smem(G, d, static_cast<int>(sizeof(T)), P);
    const int rowb = d * static_cast<int>(sizeof(T)) + 16;
    double* qn = reinterpret_cast<double*>(sm + mp.qn);
    double* zl = reinterpret_cast<double*>(sm + mp.z);
    double* sg = reinterpret_cast<double*>(sm + mp.sg);
    double* half = reinterpret_cast<double*>(sm + mp.half);

    // W rows of the group (contiguous in HBM), 16-byte loads all in flight
    const T* wsrc = W + (static_cast<long long>(h) * L * P + static_cast<long long>(l0) * P) * d;
    const int nblk = R * (d / E);
    for (int i0 = 0; i0 < nblk; i0 += NT * 8) {
      u32x4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = i0 + u * NT + t;
        if (e < nblk) v[u] = reinterpret_cast<const u32x4*>(wsrc)[e];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = i0 + u * NT + t;
        if (e < nblk) {
          const int r = e / (d / E), cb = e % (d / E);
          *reinterpret_cast<u32x4*>(sm + mp.wrows + r * rowb + cb * 16) = v[u];
        }
      }
    }
    // normalised queries
    for (int g = wave; g < G; g += NT / 64) {
      const T* qr = q + (static_cast<long long>(b) * a.Hq + h * G + g) * d;
      double s2 = 0.0;
      for (int c = lane; c < d; c += 64) {
        const double v = to_f64(qr[c]);
        qn[g * d + c] = v;
        s2 += v * v;
      }
      for (int m = 32; m >= 1; m >>= 1) s2 += __shfl_xor(s2, m, 64);
      const double nrm = sqrt(s2);
      for (int c = lane; c < d; c += 64) qn[g * d + c] = nrm > 0.0 ? qn[g * d + c] / nrm : 0.0;
    }
    __syncthreads();

    // projections z[g][r], r = ll * P + p (four partial sums per dot)
    for (int pr = t; pr < G * R; pr += NT) {
      const int g = pr / R, r = pr % R;
      const unsigned char* wr = sm + mp.wrows + r * rowb;
      const double* qq = qn + g * d;
      double acc[4] = {0.0, 0.0, 0.0, 0.0};
      for (int cb = 0; cb < d / E; ++cb) {
        const u32x4 wv = *reinterpret_cast<const u32x4*>(wr + cb * 16);
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int x = 0; x < E; ++x) {
          float f;
          if (sizeof(T) == 2) f = (x & 1) ? bf16_hi(ww[x >> 1]) : bf16_lo(ww[x >> 1]);
          else f = __uint_as_float(ww[x]);
          acc[x & 3] += static_cast<double>(f) * qq[cb * E + x];
        }
      }
      zl[g * R + r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    __syncthreads();
    // logistic pairs: sg[((g*2 + bit)*P + p)*8 + ll]
    for (int e = t; e < G * P * lg; e += NT) {
      const int g = e / (P * lg), rem = e % (P * lg), p = rem / lg, ll = rem % lg;
      const double x = 2.0 * zl[g * R + ll * P + p] * a.inv_tau;
      sg[((g * 2 + 0) * P + p) * kTabGroup + ll] = 1.0 / (1.0 + exp(x));   // bit clear
      sg[((g * 2 + 1) * P + p) * kTabGroup + ll] = 1.0 / (1.0 + exp(-x));  // bit set
    }
    __syncthreads();
    // half products: half[(g*hw + c)*8 + ll], c < nlo: low bits, else high bits
    for (int e = t; e < G * hw * lg; e += NT) {
      const int g = e / (hw * lg), rem = e % (hw * lg), c = rem / lg, ll = rem % lg;
      double pr = 1.0;
      if (c < nlo) {
        for (int p = 0; p < plo; ++p) pr *= sg[((g * 2 + ((c >> p) & 1)) * P + p) * kTabGroup + ll];
      } else {
        const int ch = c - nlo;
        for (int p = 0; p < phi; ++p)
          pr *= sg[((g * 2 + ((ch >> p) & 1)) * P + plo + p) * kTabGroup + ll];
      }
      half[(g * hw + c) * kTabGroup + ll] = pr;
    }
    __syncthreads();
    // entries (bucket c, table l0 + ll), summed over the query heads in order
    float* Tg = a.tables + static_cast<long long>(bh) * nb * L;
    for (int e = t; e < nb * lg; e += NT) {
      const int c = e / lg, ll = e % lg;
      double acc = 0.0;
      for (int g = 0; g < G; ++g)
        acc += half[(g * hw + (c & (nlo - 1))) * kTabGroup + ll] *
               half[(g * hw + nlo + (c >> plo)) * kTabGroup + ll];
      Tg[c * L + l0 + ll] = static_cast<float>(acc);
    }
  }

  if (son) {
    if (vec) {
      rg.store(a.samp, L);
    } else {
      const uint8_t* src = ids + krow * L;
      uint8_t* dst = a.samp + drow * L;
      for (int x = 0; x < L; ++x) dst[x] = src[x];
    }
    a.samp_vn[drow] = vn;
  }
}

// ---------------------------------------------------------------------------
// binary-code query codes (+ sample)

// [ sum_c r[c] x[c] >= 0 ] exactly for float data in LDS (see dot_nonneg_exact)
__device__ __forceinline__ bool lds_dot_nonneg(const float* r, const float* x, int d) {
  double s = 0.0, sa = 0.0;
  for (int c = 0; c < d; ++c) {
    const double p = static_cast<double>(r[c]) * static_cast<double>(x[c]);
    s += p;
    sa += fabs(p);
  }
  if (fabs(s) > 2.0 * d * 0x1p-53 * sa) return s >= 0.0;
  return expansion_dot_nonneg(r, x, d);
}

// LDS: 16 rows of R [16][d + 1] float, q [G][d + 1] float (rows padded by one
// word so that lanes on different rows use different banks)
static size_t qcodes_smem(int G, int d) { return static_cast<size_t>(16 + G) * (d + 1) * 4; }

template <typename T>
__global__ void __launch_bounds__(kPrepNT)
prep_qcodes_kernel(const T* __restrict__ q, const T* __restrict__ R, const uint32_t* __restrict__ codes,
                   const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_seq,
                   FusedArgs a) {
  constexpr int NT = kPrepNT;
  extern __shared__ __align__(16) unsigned char sm[];
  const int G = a.Hq / a.Hkv, d = a.d, ds = d + 1;
  const int bh = blockIdx.y, b = bh / a.Hkv, h = bh % a.Hkv, j = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63;
  float* rl = reinterpret_cast<float*>(sm);
  float* ql = rl + 16 * ds;

  const SampleShare ss = sample_share(a, seq_lens, k_per_seq, b);
  const int si = ss.i0 + t;
  const bool son = si < ss.i1;
  const long long krow = static_cast<long long>(bh) * a.Nmax + (son ? sample_pos(si, ss.S, ss.n) : 0);
  RowGather rg;
  rg.load(reinterpret_cast<const uint8_t*>(codes), krow, 16, son, static_cast<long long>(bh) * kSample + si);

  if (j < 8) {  // bits [16j, 16j + 16)
    const T* rs = R + (static_cast<long long>(h) * 128 + j * 16) * d;
    for (int e = t; e < 16 * d; e += NT) rl[(e / d) * ds + e % d] = to_f32(rs[e]);
    const T* qs = q + (static_cast<long long>(b) * a.Hq + h * G) * d;
    for (int e = t; e < G * d; e += NT) ql[(e / d) * ds + e % d] = to_f32(qs[e]);
    __syncthreads();
    uint16_t* qc16 = reinterpret_cast<uint16_t*>(a.qcodes) + static_cast<long long>(bh) * G * 8;
    for (int p0 = 0; p0 < G * 16; p0 += NT) {  // uniform trip count: ballots see whole waves
      const int p = p0 + t, g = p >> 4, i = p & 15;
      const bool bit = p < G * 16 && lds_dot_nonneg(rl + i * ds, ql + g * ds, d);
      const unsigned long long m = __ballot(bit);
      if (p < G * 16 && i == 0) qc16[g * 8 + j] = static_cast<uint16_t>(m >> (lane & 48));
    }
  }
  rg.store(a.samp, 16);
}

// ---------------------------------------------------------------------------
// given scores: the sample as order keys

__device__ __forceinline__ uint32_t order_key_of(float v) { return order_key_f32(v); }
__device__ __forceinline__ uint32_t order_key_of(int32_t v) { return order_key_i32(v); }

template <typename KT>
__global__ void __launch_bounds__(kPrepNT)
prep_given_kernel(const KT* __restrict__ scores, const int32_t* __restrict__ seq_lens,
                  const int32_t* __restrict__ k_per_seq, FusedArgs a) {
  const int bh = blockIdx.y, b = bh / a.Hkv;
  const SampleShare ss = sample_share(a, seq_lens, k_per_seq, b);
  const int si = ss.i0 + static_cast<int>(threadIdx.x);
  if (si < ss.i1) {
    const KT v = scores[static_cast<long long>(bh) * a.Nmax + sample_pos(si, ss.S, ss.n)];
    reinterpret_cast<uint32_t*>(a.samp)[static_cast<long long>(bh) * kSample + si] = order_key_of(v);
  }
}

// ---------------------------------------------------------------------------
// launchers

// Raises a kernel's dynamic LDS limit once per device (the largest size
// requested so far).
template <typename K>
static hipError_t set_smem(K kern, size_t bytes) {
  static size_t done[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && done[dev] >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(bytes));
  if (e == hipSuccess && dev >= 0 && dev < 64) done[dev] = bytes;
  return e;
}

hipError_t launch_prep_soft(const hst_shape& s, const FusedArgs& a, const void* q, const void* W,
                            const uint8_t* ids, const void* vnorm, int norm_f16,
                            const int32_t* kps, hipStream_t st) {
  const int G = s.Hq / s.Hkv;
  dim3 grid(a.sample ? prep_blocks_soft(a.L) : (a.L + kTabGroup - 1) / kTabGroup, s.B * s.Hkv);
  if (s.kv_dtype == HST_F32) {
    auto kern = prep_tables_kernel<float>;
    const size_t smem = tab_smem(G, s.d, 4, a.P).bytes;
    hipError_t e = set_smem(kern, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kPrepNT), smem, st, static_cast<const float*>(q),
                       static_cast<const float*>(W), ids, vnorm, norm_f16, s.seq_lens, kps, a);
  } else {
    auto kern = prep_tables_kernel<bf16>;
    const size_t smem = tab_smem(G, s.d, 2, a.P).bytes;
    hipError_t e = set_smem(kern, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kPrepNT), smem, st, static_cast<const bf16*>(q),
                       static_cast<const bf16*>(W), ids, vnorm, norm_f16, s.seq_lens, kps, a);
  }
  return hipGetLastError();
}

hipError_t launch_prep_hamming(const hst_shape& s, const FusedArgs& a, const void* q, const void* R,
                               const uint32_t* codes, const int32_t* kps, hipStream_t st) {
  dim3 grid(kPrepBlocks, s.B * s.Hkv);
  const size_t smem = qcodes_smem(s.Hq / s.Hkv, s.d);
  if (s.kv_dtype == HST_F32) {
    auto kern = prep_qcodes_kernel<float>;
    hipError_t e = set_smem(kern, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kPrepNT), smem, st, static_cast<const float*>(q),
                       static_cast<const float*>(R), codes, s.seq_lens, kps, a);
  } else {
    auto kern = prep_qcodes_kernel<bf16>;
    hipError_t e = set_smem(kern, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(kPrepNT), smem, st, static_cast<const bf16*>(q),
                       static_cast<const bf16*>(R), codes, s.seq_lens, kps, a);
  }
  return hipGetLastError();
}

hipError_t launch_prep_given(const hst_shape& s, const FusedArgs& a, int score_dtype,
                             const void* scores, const int32_t* kps, hipStream_t st) {
  dim3 grid(kPrepBlocks, s.B * s.Hkv);
  if (score_dtype == HST_F32)
    hipLaunchKernelGGL(prep_given_kernel<float>, grid, dim3(kPrepNT), 0, st,
                       static_cast<const float*>(scores), s.seq_lens, kps, a);
  else
    hipLaunchKernelGGL(prep_given_kernel<int32_t>, grid, dim3(kPrepNT), 0, st,
                       static_cast<const int32_t*>(scores), s.seq_lens, kps, a);
  return hipGetLastError();
}

}  // namespace hst
