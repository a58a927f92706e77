// Per-step query preprocessing, X workgroups per (sequence, kv head).
//
//  * Soft-LSH (SOCKET overview page, "Core mechanism: soft LSH", item 2):
//    workgroup j builds the query tables of hash tables [TG*j, TG*j + TG)
//    (TG = 4, or 8 from 128 tables on; see tab_group).  The
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
//
// When a top-k follows, each workgroup also scores the key sample on its own
// part of the hash (its TG tables, its 16 code bits), reading only that slice
// of each sampled key's metadata; the scan adds the parts up and derives the
// candidate threshold theta from them (scan.hip).  theta only bounds the work
// of the selection: the selected set never depends on it.  For the routed
// step the soft-LSH workgroups score the head's index cards the same way,
// and the card cut adds the parts up (route.hip).
#include "fused_device.h"
#include "hst_launch.h"

namespace hst {

constexpr int kPrepNT = 512;
// hash tables per prep workgroup: 4 (8 from L = 128 on, so that a head has
// at most 16 parts of its sample scores)
__host__ __device__ constexpr int tab_group(int L) { return L > 64 ? 8 : 4; }
constexpr int kSPer = kSample / kPrepNT;  // sampled keys per thread

// Raises a kernel's dynamic LDS limit (kept per kernel and device).
template <typename K>
static hipError_t set_smem(K kern, size_t bytes) {
  return raise_lds_limit(reinterpret_cast<const void*>(kern), bytes);
}

// A workgroup barrier that orders LDS accesses only: unlike __syncthreads()
// it does not wait for this thread's global loads (the sample loads stay in
// flight across it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sample size of head b (0 when no top-k follows or nothing is selected).
__device__ __forceinline__ int sample_size(const FusedArgs& a, const int32_t* seq_lens,
                                           const int32_t* k_per_seq, int b, int& n) {
  n = seq_len(seq_lens, b, a.Nmax);
  if (a.sample == 0 || keff_of(a.kcap, k_per_seq, b, n) == 0) return 0;
  return a.sample > n ? n : a.sample;
}

// Zeroes the head's threshold word, which the filtering scan publishes.
__device__ __forceinline__ void reset_scan_state(const FusedArgs& a, int bh) {
  if (a.sample != 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    a.heads[bh].thr_word = 0ull;
    a.heads[bh].arrive = 0u;
  }
}

// ---------------------------------------------------------------------------
// soft-LSH tables (+ partial sample scores)

struct TabSmem {
  int wrows, qn, lpair, half, tl, bytes;
};

// LDS map of one group of TG tables: W rows (padded by 64 bytes), q [G][d]
// (float64), the logistic pairs [G][TG*P] (float64 x 2), half products
// [G][TG][hw] (float64), the group's float32 table [TG][2^P + 1]
// (table-major, rows padded by one word).
__host__ __device__ inline TabSmem tab_smem(int G, int d, int esize, int P, int TG) {
  const int plo = P < 4 ? P : 4;
  const int hw = (1 << plo) + (1 << (P - plo));
  TabSmem m{};
  m.wrows = 0;
  m.qn = m.wrows + TG * P * (d * esize + 64);
  m.lpair = m.qn + G * d * 8;
  m.half = m.lpair + G * TG * P * 16;
  m.tl = m.half + G * hw * TG * 8;
  m.bytes = m.tl + TG * ((1 << P) + 1) * 4;
  return m;
}

// CARDS: the routed step's variant, which scores the index cards (a.cpart
// set) instead of the key sample.
template <typename T, int TG, bool CARDS>
__global__ void __launch_bounds__(kPrepNT)
__attribute__((amdgpu_waves_per_eu(TG == 4 ? 8 : 1)))  // four groups of 4 tables per CU (64 VGPRs)
prep_tables_kernel(const T* __restrict__ q, const T* __restrict__ W, const uint8_t* __restrict__ ids,
                   const int32_t* __restrict__ seq_lens,
                   const int32_t* __restrict__ k_per_seq, FusedArgs a) {
  constexpr int NT = kPrepNT;
  constexpr int E = 16 / static_cast<int>(sizeof(T));
  extern __shared__ __align__(16) unsigned char sm[];
  const int G = a.Hq / a.Hkv, d = a.d, L = a.L, P = a.P, nb = 1 << P;
  const int bh = blockIdx.x, b = bh / a.Hkv, h = bh % a.Hkv, j = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  reset_scan_state(a, bh);
  const int l0 = j * TG, lg = min(TG, L - l0), R = lg * P;
  const bool fullg = lg == TG && L % TG == 0;  // the group's ids are one aligned word (pair)

  const int plo = P < 4 ? P : 4, phi = P - plo, nlo = 1 << plo, hw = nlo + (1 << phi);
  const TabSmem mp = tab_smem(G, d, static_cast<int>(sizeof(T)), P, TG);
  // W rows padded by 64 bytes: the four lanes of a dot product read blocks
  // cb, cb + 4, ... of four consecutive rows at once, and a row stride of 16
  // words (mod the 64 banks) keeps those sixteen 16-byte reads apart
  const int rowb = d * static_cast<int>(sizeof(T)) + 64;
  double* qn = reinterpret_cast<double*>(sm + mp.qn);
  double* half = reinterpret_cast<double*>(sm + mp.half);
  float* tl = reinterpret_cast<float*>(sm + mp.tl);

  // W rows of the group (contiguous in HBM) and the G query rows:
  // unconditional (clamped) loads, all in flight together.  They are issued
  // before the scattered sample loads below, so waiting for them does not
  // wait for those (loads complete in issue order for the wait counter).
  const T* wsrc = W + (static_cast<long long>(h) * L * P + static_cast<long long>(l0) * P) * d;
  // >= 1 and <= 4 * NT: at most 8 tables x 8 planes x 128 dims x 4 bytes / 16
  const int nblk = R * (d / E);
  u32x4 wv4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = u * NT + t;
    wv4[u] = reinterpret_cast<const u32x4*>(wsrc)[e < nblk ? e : nblk - 1];
  }
  const T* qsrc = q + (static_cast<long long>(b) * a.Hq + h * G) * d;
  constexpr int kQPer = 2;  // G * d <= 1024 = kQPer * NT
  float qv[kQPer];
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int e = u * NT + t;
    qv[u] = to_f32(qsrc[e < G * d ? e : G * d - 1]);
  }

  // The items this group scores on its tables, their ids (TG bytes each)
  // loaded now: the key sample, or for the routed step the head's index cards
  // (the first ceil(n / kCardKeys) rows of a.cids; the card cut applies the
  // card weights).
  int n;
  const int S0 = sample_size(a, seq_lens, k_per_seq, b, n);
  constexpr bool cards = CARDS;
  const int S = cards ? (n + kCardKeys - 1) / kCardKeys : S0;  // items
  const long long base = static_cast<long long>(bh) * a.Nmax;
  const uint8_t* isrc = cards ? a.cids : ids;
  const auto item_row = [&](int i) -> long long {
    if (cards) {
      HST_DCHECK(i >= 0 && i < a.ncards, kDbgCardRow);
      return static_cast<long long>(bh) * a.ncards + i;
    }
    const int sp = sample_pos(i, S, n);
    HST_DCHECK(sp >= 0 && sp < n, kDbgSampleRow);
    return base + sp;
  };
  // The loads are unconditional (an item this group does not read from its
  // row reads the first W word instead), so that the memory counter knows how
  // many are in flight: the LDS stores of W and q below wait for W and q
  // alone, and the sample loads stay in flight until the scoring.
  uint32_t sid[kSPer][TG / 4];
  {
    const bool rd_id = S > 0 && fullg;
    const unsigned char* dflt = reinterpret_cast<const unsigned char*>(wsrc);
#pragma unroll
    for (int u = 0; u < kSPer; ++u) {
      const int i = t + u * NT;
      const long long row = S > 0 ? item_row(i < S ? i : S - 1) : 0;
      const unsigned char* ip = rd_id ? isrc + row * L + l0 : dflt;
      if constexpr (TG == 8) {
        const uint2 v = *reinterpret_cast<const uint2*>(ip);
        sid[u][0] = v.x;
        sid[u][1] = v.y;
      } else {
        sid[u][0] = *reinterpret_cast<const uint32_t*>(ip);
      }
    }
  }

#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = u * NT + t;
    if (e < nblk) {
      const int r = e / (d / E), cb = e % (d / E);
      *reinterpret_cast<u32x4*>(sm + mp.wrows + r * rowb + cb * 16) = wv4[u];
    }
  }
#pragma unroll
  for (int u = 0; u < kQPer; ++u) {
    const int e = u * NT + t;
    if (e < G * d) qn[e] = static_cast<double>(qv[u]);
  }
  lds_barrier();

  // projections of the raw queries z[g][r] = W_r . q_g, r = ll * P + p: four
  // lanes per dot (interleaved 16-byte blocks of the row), each with its own
  // partial sums of the dot and of q_g's squares (the same four lanes read
  // all of q_g), added over the four lanes by DPP quad permutations; then
  // lane 0 of the four forms the logistic pair of the plane from
  // z / ||q|| (the projection of the normalised query): one exp, with
  // e = exp(-|x|), sigma(|x|) = 1 / (1 + e) and sigma(-|x|) = e / (1 + e),
  // kept as (bit set, bit clear)
  double2* lp = reinterpret_cast<double2*>(sm + mp.lpair);
  for (int pr0 = 0; pr0 < G * R * 4; pr0 += NT) {  // uniform trip count (lane moves below)
    const int pq = pr0 + t, pr = pq >> 2, part = pq & 3;
    double acc = 0.0, qsq = 0.0;
    if (pr < G * R) {
      const int g = pr / R, r = pr % R;
      const unsigned char* wr = sm + mp.wrows + r * rowb;
      const double* qq = qn + g * d;
      double ac[4] = {0.0, 0.0, 0.0, 0.0};  // four independent chains
      double q2[4] = {0.0, 0.0, 0.0, 0.0};
      for (int cb = part; cb < d / E; cb += 4) {
        const u32x4 wv = *reinterpret_cast<const u32x4*>(wr + cb * 16);
        const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int x = 0; x < E; ++x) {
          float f;
          if (sizeof(T) == 2) f = (x & 1) ? bf16_hi(ww[x >> 1]) : bf16_lo(ww[x >> 1]);
          else f = __uint_as_float(ww[x]);
          const double qv = qq[cb * E + x];
          ac[x & 3] += static_cast<double>(f) * qv;
          q2[x & 3] += qv * qv;
        }
      }
      acc = (ac[0] + ac[1]) + (ac[2] + ac[3]);
      qsq = (q2[0] + q2[1]) + (q2[2] + q2[3]);
    }
    const double a1 = acc + dpp_f64<0xB1>(acc);  // quad [1,0,3,2]: the xor-1 lane
    const double z = a1 + dpp_f64<0x4E>(a1);     // quad [2,3,0,1]: the xor-2 lane
    const double s1 = qsq + dpp_f64<0xB1>(qsq);
    const double n2 = s1 + dpp_f64<0x4E>(s1);
    if (pr < G * R && part == 0) {
      const double nq = sqrt(n2);
      const double x = nq > 0.0 ? 2.0 * (z / nq) * a.inv_tau : 0.0;
      const double e = exp(-fabs(x));
      const double big = 1.0 / (1.0 + e), small = e * big;
      lp[pr] = x >= 0.0 ? make_double2(big, small) : make_double2(small, big);
    }
  }
  lds_barrier();
  // one thread per (query head g, table ll, half of the planes, bit pattern
  // b of the half): the product over the half's planes in plane order,
  // half[(g*TG + ll)*hw + c] (the table phase reads consecutive buckets'
  // halves of one table from consecutive lanes)
  for (int e = t; e < G * lg * hw; e += NT) {
    const int g = e / (lg * hw), rem = e % (lg * hw), ll = rem / hw, c = rem % hw;
    const bool hi = c >= nlo;
    const int p0 = hi ? plo : 0, m = hi ? phi : plo, b = hi ? c - nlo : c;
    const double2* pp = lp + g * R + ll * P + p0;
    double v = 1.0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k < m) v *= ((b >> k) & 1) ? pp[k].x : pp[k].y;
    half[(g * TG + ll) * hw + c] = v;
  }
  lds_barrier();
  // entries (bucket c, table l0 + ll), summed over the query heads in order,
  // to LDS table-major as tl[ll*(2^P + 1) + c]: a lookup's bank follows its
  // bucket over all 64 banks (bucket-major rows of TG words used 16), and
  // the pad puts the TG entries of one bucket in different banks
  const int tls = nb + 1;  // LDS row of one table
  for (int e = t; e < nb * lg; e += NT) {  // consecutive lanes, consecutive buckets
    const int ll = e / nb, c = e % nb;
    double acc = 0.0;
    for (int g = 0; g < G; ++g)
      acc += half[(g * TG + ll) * hw + (c & (nlo - 1))] * half[(g * TG + ll) * hw + nlo + (c >> plo)];
    tl[ll * tls + c] = static_cast<float>(acc);
  }
  lds_barrier();
  // the group's table to HBM, bucket-major (after the scoring below, which
  // waits for the sample loads: stores issued before it would be waited for
  // too)
  float* Tg = a.tables + static_cast<long long>(bh) * nb * L;
  const auto table_out = [&]() {
    for (int e = t; e < nb * lg; e += NT) {
      const int c = e / lg, ll = e % lg;
      Tg[c * L + l0 + ll] = tl[ll * tls + c];
    }
  };
  if (S == 0) {
    table_out();
    return;
  }

  // partial item scores on this group's tables
  const uint32_t idm = static_cast<uint32_t>(nb - 1);
  float* part = cards ? a.cpart + (static_cast<long long>(bh) * a.xparts + j) * a.ncards
                      : a.spart + (static_cast<long long>(bh) * a.xparts + j) * kSample;
  const auto score_row = [&](int i) {
    const uint8_t* row = isrc + item_row(i) * L + l0;
    float s2[2] = {0.f, 0.f};
    for (int ll = 0; ll < lg; ++ll) {
      const int c = static_cast<int>(row[ll] & idm);
      s2[ll & 1] += tl[ll * tls + c];
    }
    return s2[0] + s2[1];
  };
#pragma unroll
  for (int u = 0; u < kSPer; ++u) {
    const int i = t + u * NT;
    if (i >= S) continue;
    float s2[2] = {0.f, 0.f};
    if (fullg) {
#pragma unroll
      for (int ll = 0; ll < TG; ++ll) {
        const int c = static_cast<int>((sid[u][ll >> 2] >> (8 * (ll & 3))) & idm);
        s2[ll & 1] += tl[ll * tls + c];
      }
      part[i] = s2[0] + s2[1];
    } else {
      part[i] = score_row(i);
    }
  }
  if constexpr (CARDS)  // cards past the first kSPer * NT (the sample has at most kSample keys)
    for (int i = kSPer * NT + t; i < S; i += NT) part[i] = score_row(i);
  table_out();
}

// ---------------------------------------------------------------------------
// binary-code query codes (+ partial sample scores)

// [ sum_c r[c] x[c] >= 0 ] exactly for float data in LDS (see dot_nonneg_exact)
__device__ __forceinline__ bool lds_dot_nonneg(const float* r, const float* x, int d) {
  double s = 0.0, sa = 0.0;
  for (int c = 0; c < d; ++c) {
    const double p = static_cast<double>(r[c]) * static_cast<double>(x[c]);
    s += p;
    sa += fabs(p);
  }
  if (fabs(s) > 2.0 * d * 0x1p-53 * sa) return s >= 0.0;
  return exact_dot_nonneg(r, x, d);
}

// LDS: 16 rows of R [16][d + 1] float, q [G][d + 1] float (rows padded by one
// word so that lanes on different rows use different banks), G 16-bit code
// slices
static size_t qcodes_smem(int G, int d) { return static_cast<size_t>(16 + G) * (d + 1) * 4 + G * 4; }

template <typename T>
__global__ void __launch_bounds__(kPrepNT)
prep_qcodes_kernel(const T* __restrict__ q, const T* __restrict__ R, const uint32_t* __restrict__ codes,
                   const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_seq,
                   FusedArgs a) {
  constexpr int NT = kPrepNT;
  extern __shared__ __align__(16) unsigned char sm[];
  const int G = a.Hq / a.Hkv, d = a.d, ds = d + 1;
  const int bh = blockIdx.x, b = bh / a.Hkv, h = bh % a.Hkv, j = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63;
  float* rl = reinterpret_cast<float*>(sm);
  float* ql = rl + 16 * ds;
  uint32_t* q16 = reinterpret_cast<uint32_t*>(ql + G * ds);
  reset_scan_state(a, bh);

  // sampled keys' code bits [16j, 16j + 16), loads issued now
  int n;
  const int S = sample_size(a, seq_lens, k_per_seq, b, n);
  const long long base = static_cast<long long>(bh) * a.Nmax;
  uint32_t sc16[kSPer];
  if (S > 0) {
#pragma unroll
    for (int u = 0; u < kSPer; ++u) {
      const int i = t + u * NT;
      const int sp = sample_pos(i < S ? i : S - 1, S, n);
      HST_DCHECK(sp >= 0 && sp < n, kDbgSampleRow);
      const long long row = base + sp;
      sc16[u] = reinterpret_cast<const uint16_t*>(codes)[row * 8 + j];
    }
  }

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
    if (p < G * 16 && i == 0) {
      const uint16_t v = static_cast<uint16_t>(m >> (lane & 48));
      qc16[g * 8 + j] = v;
      q16[g] = v;
    }
  }
  if (S == 0) return;
  __syncthreads();
  float* part = a.spart + (static_cast<long long>(bh) * a.xparts + j) * kSample;
#pragma unroll
  for (int u = 0; u < kSPer; ++u) {
    const int i = t + u * NT;
    if (i >= S) continue;
    int ham = 0;
    for (int g = 0; g < G; ++g) ham += __popc((sc16[u] ^ q16[g]) & 0xffffu);
    part[i] = static_cast<float>(ham);  // exact: at most 16 * G
  }
}

// ---------------------------------------------------------------------------
// given scores: the sample's order keys (part 0)

__device__ __forceinline__ uint32_t order_key_of(float v) { return order_key_f32(v); }
__device__ __forceinline__ uint32_t order_key_of(int32_t v) { return order_key_i32(v); }

template <typename KT>
__global__ void __launch_bounds__(kPrepNT)
prep_given_kernel(const KT* __restrict__ scores, const int32_t* __restrict__ seq_lens,
                  const int32_t* __restrict__ k_per_seq, FusedArgs a) {
  const int bh = blockIdx.x, b = bh / a.Hkv;
  reset_scan_state(a, bh);
  int n;
  const int S = sample_size(a, seq_lens, k_per_seq, b, n);
  for (int i = threadIdx.x; i < S; i += kPrepNT) {
    const KT v = scores[static_cast<long long>(bh) * a.Nmax + sample_pos(i, S, n)];
    reinterpret_cast<uint32_t*>(a.spart)[static_cast<long long>(bh) * a.xparts * kSample + i] = order_key_of(v);
  }
}

// ---------------------------------------------------------------------------
// launchers

int prep_parts(int kind, int L) {
  if (kind == kScanSoftFast || kind == kScanSoftAny) return (L + tab_group(L) - 1) / tab_group(L);
  return kind == kScanHamming ? 8 : 1;
}

hipError_t launch_prep_soft(const hst_shape& s, const FusedArgs& a, const void* q, const void* W,
                            const uint8_t* ids, const int32_t* kps, hipStream_t st) {
  const int G = s.Hq / s.Hkv;
  // x = (sequence, kv head): workgroups are handed to the XCDs round robin in
  // linear order, so the parts of one head (B*Hkv apart) share an XCD and its
  // L2 whenever B*Hkv is a multiple of 8, and the sampled id rows are fetched
  // from HBM once per head
  const int TG = tab_group(a.L);
  dim3 grid(s.B * s.Hkv, (a.L + TG - 1) / TG);
#define HST_PREP(TT, TGV)                                                                      \
  do {                                                                                         \
    auto kern = a.cpart != nullptr ? prep_tables_kernel<TT, TGV, true> : prep_tables_kernel<TT, TGV, false>; \
    const size_t smem = tab_smem(G, s.d, static_cast<int>(sizeof(TT)), a.P, TGV).bytes;        \
    hipError_t e = set_smem(kern, smem);                                                       \
    if (e != hipSuccess) return e;                                                             \
    hipLaunchKernelGGL(kern, grid, dim3(kPrepNT), smem, st, static_cast<const TT*>(q),         \
                       static_cast<const TT*>(W), ids, s.seq_lens, kps, a);                  \
  } while (0)
  if (s.kv_dtype == HST_F32) {
    if (TG == 8) HST_PREP(float, 8);
    else HST_PREP(float, 4);
  } else {
    if (TG == 8) HST_PREP(bf16, 8);
    else HST_PREP(bf16, 4);
  }
#undef HST_PREP
  return hipGetLastError();
}

hipError_t launch_prep_hamming(const hst_shape& s, const FusedArgs& a, const void* q, const void* R,
                               const uint32_t* codes, const int32_t* kps, hipStream_t st) {
  dim3 grid(s.B * s.Hkv, 8);
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
  dim3 grid(s.B * s.Hkv, 1);
  if (score_dtype == HST_F32)
    hipLaunchKernelGGL(prep_given_kernel<float>, grid, dim3(kPrepNT), 0, st,
                       static_cast<const float*>(scores), s.seq_lens, kps, a);
  else
    hipLaunchKernelGGL(prep_given_kernel<int32_t>, grid, dim3(kPrepNT), 0, st,
                       static_cast<const int32_t*>(scores), s.seq_lens, kps, a);
  return hipGetLastError();
}

}  // namespace hst
