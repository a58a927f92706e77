// Cumulative-mass selection over a candidate set.
// Tactic page ("Tactic: Adaptive Sparse Attention with Clustering and
// Distribution Fitting for Long-Context LLMs"), sections 1 and 3: instead of
// a fixed token budget, tokens are added until the summed softmax-normalised
// attention score of the chosen set reaches a target, so the count adapts
// per head and query.  Here the candidates are the keys of highest hash
// score (the soft-LSH selection), their exact logits give the mass, and the
// kept set is the shortest prefix of the order (mass descending, index
// ascending) whose mass reaches p of the total.
//
//   mass_logits_kernel  grid (ceil(k / 64), B*Hkv): float64 logits of the
//                       G query heads against 64 candidate rows (16 lanes per
//                       row, all row loads of a workgroup issued up front),
//                       and per head their max, exp(a - max) and its sum.
//   mass_pick_kernel    one 1024-thread workgroup per (sequence, kv head):
//                       the log-sum-exp merge of the workgroups, the masses, a radix
//                       select of the cut on the mass bits with exact
//                       fixed-point running sums, and the compaction in
//                       candidate order.
//
// The masses are float64; the running sums are exact integers (the masses
// in units of 2^-62), so the result does not depend on any reduction order
// and does not change from run to run.  Equal masses go to the earlier
// candidate (the lower index when the candidates are ascending).
#include "hst_common.h"
#include "hst_fused.h"
#include "hst_launch.h"

namespace hst {

constexpr int kMassRows = 64;    // candidate rows per logits workgroup
constexpr int kMassNT = 1024;    // threads of the pick workgroup
constexpr int kMassGmax = 8;     // query heads per kv head

template <typename T, int E>
__device__ __forceinline__ void load_f64(const T* __restrict__ p, double (&x)[E]);

template <>
__device__ __forceinline__ void load_f64<bf16, 8>(const bf16* __restrict__ p, double (&x)[8]) {
  const u32x4 v = *reinterpret_cast<const u32x4*>(p);
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(v[e]);
    x[2 * e + 1] = bf16_hi(v[e]);
  }
}
template <>
__device__ __forceinline__ void load_f64<bf16, 4>(const bf16* __restrict__ p, double (&x)[4]) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  x[0] = bf16_lo(v.x);
  x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y);
  x[3] = bf16_hi(v.y);
}
template <>
__device__ __forceinline__ void load_f64<float, 8>(const float* __restrict__ p, double (&x)[8]) {
  const u32x4 a = reinterpret_cast<const u32x4*>(p)[0];
  const u32x4 b = reinterpret_cast<const u32x4*>(p)[1];
  for (int e = 0; e < 4; ++e) {
    x[e] = __uint_as_float(a[e]);
    x[4 + e] = __uint_as_float(b[e]);
  }
}
template <>
__device__ __forceinline__ void load_f64<float, 4>(const float* __restrict__ p, double (&x)[4]) {
  const u32x4 a = *reinterpret_cast<const u32x4*>(p);
  for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(a[e]);
}

// Sum over each aligned group of 16 lanes, left in every lane of the group
// (DPP butterflies on both halves of the double, in a fixed order).
__device__ __forceinline__ double dpp16_sum_d(double v) {
  auto step = [](double x, int ctrl) {
    const long long b = __double_as_longlong(x);
    int lo = static_cast<int>(b), hi = static_cast<int>(b >> 32);
    switch (ctrl) {
      case 0xB1:
        lo = __builtin_amdgcn_update_dpp(0, lo, 0xB1, 0xf, 0xf, false);
        hi = __builtin_amdgcn_update_dpp(0, hi, 0xB1, 0xf, 0xf, false);
        break;
      case 0x4E:
        lo = __builtin_amdgcn_update_dpp(0, lo, 0x4E, 0xf, 0xf, false);
        hi = __builtin_amdgcn_update_dpp(0, hi, 0x4E, 0xf, 0xf, false);
        break;
      case 0x141:
        lo = __builtin_amdgcn_update_dpp(0, lo, 0x141, 0xf, 0xf, false);
        hi = __builtin_amdgcn_update_dpp(0, hi, 0x141, 0xf, 0xf, false);
        break;
      default:
        lo = __builtin_amdgcn_update_dpp(0, lo, 0x140, 0xf, 0xf, false);
        hi = __builtin_amdgcn_update_dpp(0, hi, 0x140, 0xf, 0xf, false);
        break;
    }
    return __longlong_as_double((static_cast<long long>(hi) << 32) |
                                static_cast<long long>(static_cast<uint32_t>(lo)));
  };
  v += step(v, 0xB1);   // quad [1,0,3,2]
  v += step(v, 0x4E);   // quad [2,3,0,1]
  v += step(v, 0x141);  // row half mirror
  v += step(v, 0x140);  // row mirror
  return v;
}

// Per workgroup of 64 candidate rows and per query head g: the logits
// a = scale * q[b][h*G+g] . K[b][h][cand] in float64 (bf16 and float32
// products are exact in float64), their max m_w over the rows, and
// e = exp(a - m_w) with its sum z_w.  e goes to ework[bh][r][g] (0 for
// padding), (m_w, z_w) to wstat[bh][g][w].  The pick kernel merges the
// workgroups' (m_w, z_w) as a log-sum-exp.
template <typename T, int D>
__global__ void __launch_bounds__(256)
mass_logits_kernel(const T* __restrict__ q, const T* __restrict__ K,
                   const int32_t* __restrict__ cand, const int32_t* __restrict__ seq_lens, int Hq,
                   int Hkv, int Nmax, int kcap, double scale, double* __restrict__ ework,
                   double2* __restrict__ wstat) {
  constexpr int EPL = D / 16;
  constexpr int U = kMassRows / 16;  // rows per lane group
  __shared__ double qs[kMassGmax][D];
  __shared__ double at[kMassGmax][kMassRows];
  const int bh = blockIdx.y, b = bh / Hkv, h = bh % Hkv, G = Hq / Hkv;
  const int nw = gridDim.x, w = blockIdx.x;
  const int n = seq_len(seq_lens, b, Nmax);
  const int t = threadIdx.x, sub = t & 15, grp = t >> 4, lane = t & 63, wave = t >> 6;
  const int r0 = w * kMassRows;
  const int32_t* crow = cand + static_cast<long long>(bh) * kcap;
  int j[U];
  bool ok[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = r0 + grp + 16 * u;
    j[u] = r < kcap ? crow[r] : -1;
    ok[u] = j[u] >= 0 && j[u] < n;
  }
  // every load first; absent rows read row 0 of the head, which exists
  double kx[U][EPL];
#pragma unroll
  for (int u = 0; u < U; ++u)
    load_f64<T, EPL>(K + (static_cast<long long>(bh) * Nmax + (ok[u] ? j[u] : 0)) * D + sub * EPL,
                     kx[u]);
  for (int i = t; i < G * D; i += 256)
    qs[i / D][i % D] = to_f64(q[(static_cast<long long>(b) * Hq + h * G) * D + i]);
  __syncthreads();
#pragma unroll
  for (int u = 0; u < U; ++u) {
    for (int g = 0; g < G; ++g) {
      double s = 0.0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) s += qs[g][sub * EPL + e] * kx[u][e];
      s = dpp16_sum_d(s);
      if (sub == 0) at[g][grp + 16 * u] = ok[u] ? scale * s : -INFINITY;
    }
  }
  __syncthreads();
  // one wave per query head: max, exp and sum over the 64 rows (lane = row)
  for (int g = wave; g < G; g += 4) {
    const double a = at[g][lane];
    double m = a;
    for (int x = 32; x >= 1; x >>= 1) m = fmax(m, __shfl_xor(m, x));
    const double e = (a == -INFINITY) ? 0.0 : exp(a - m);
    double z = e;
    for (int x = 32; x >= 1; x >>= 1) z += __shfl_xor(z, x);
    const int r = r0 + lane;
    if (r < kcap) ework[(static_cast<long long>(bh) * kcap + r) * G + g] = e;
    if (lane == 0) wstat[(static_cast<long long>(bh) * G + g) * nw + w] = make_double2(m, z);
  }
}

// Exclusive prefix over the threads of the block (fixed order).
template <typename V>
__device__ __forceinline__ V block_excl_scan(V v, V* red) {
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  V incl = v;
  for (int m = 1; m < 64; m <<= 1) {
    const V o = __shfl_up(incl, m);
    if (lane >= m) incl += o;
  }
  __syncthreads();
  if (lane == 63) red[w] = incl;
  __syncthreads();
  V base = V(0);
  for (int i = 0; i < w; ++i) base += red[i];
  return base + incl - v;
}

// Order key of a candidate: the bits of its (non-negative) mass plus one, so
// that larger keys are larger masses and 0 marks padding.
__device__ __forceinline__ uint64_t mass_key(double m) {
  return static_cast<uint64_t>(__double_as_longlong(m)) + 1ull;
}

// floor(m * 2^62) for 0 <= m <= 1, from the bits of m (exact).
__device__ __forceinline__ uint64_t mass_fixed(double m) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(m));
  const int e = static_cast<int>(u >> 52) & 0x7ff;
  if (e == 0) return 0;  // below 2^-1022: nothing at 2^-62 resolution
  const uint64_t mant = (u & ((1ull << 52) - 1)) | (1ull << 52);
  const int sh = e - 1023 + 10;  // value = mant * 2^(e - 1075); times 2^62
  if (sh >= 0) return mant << sh;
  return sh <= -64 ? 0ull : (mant >> -sh);
}

// Wave-wide sum of a 64-bit unsigned value (every lane active).
__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
  return v;
}

// (key descending, position ascending)
__device__ __forceinline__ bool key_before(uint64_t ka, uint32_t pa, uint64_t kb, uint32_t pb) {
  return ka > kb || (ka == kb && pa < pb);
}

constexpr int kMassSmall = 64;  // a radix bucket this small is finished by one wave

// One workgroup per (sequence, kv head).
//   1. Per query head the max logit, exp(a - max) (written over the logits)
//      and its sum; then per candidate the mass m, an order key (the mass
//      bits) and the mass in fixed point, fm = floor(m * 2^62), in LDS.
//   2. Radix select from the top byte of the order key.  Each level builds
//      a histogram (counts and fixed-point masses) of the candidates sharing
//      the prefix; the bucket where the running mass from the top reaches
//      the target ceil(p * T) extends the prefix.  Fixed-point sums are
//      exact, so no reduction order can change a decision.  A bucket of at
//      most 64 candidates is sorted by one wave and cut there; after eight
//      levels the bucket holds equal keys and is cut by position.
//   3. Kept: every candidate above the threshold key and the first need_eq
//      at it (by position), compacted in candidate order.
__global__ void __launch_bounds__(kMassNT)
mass_pick_kernel(const double* __restrict__ logits, const double2* __restrict__ wstat,
                 const int32_t* __restrict__ cand,
                 const int32_t* __restrict__ seq_lens, int Hq, int Hkv, int Nmax, int kcap,
                 double p, int32_t* __restrict__ idx, int32_t* __restrict__ counts) {
  extern __shared__ __align__(16) unsigned char sm[];
  uint64_t* okey = reinterpret_cast<uint64_t*>(sm);            // [kcap]
  uint64_t* fmv = reinterpret_cast<uint64_t*>(sm + kcap * 8);  // [kcap]
  __shared__ uint32_t hcnt[256];
  __shared__ unsigned long long hsum[256];
  __shared__ uint64_t small_key[kMassSmall], small_fm[kMassSmall];
  __shared__ uint32_t small_pos[kMassSmall];
  __shared__ uint64_t redu[kMassNT / 64];
  __shared__ double fac[kMassCap / kMassRows][kMassGmax];
  __shared__ uint64_t s_prefix, s_mhi, s_thr, s_need, s_fmeq;
  __shared__ int s_state, s_level, s_nsmall, s_total;
  const int bh = blockIdx.x, G = Hq / Hkv;
  const int n = seq_len(seq_lens, bh / Hkv, Nmax);
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const double* lg = logits + static_cast<long long>(bh) * G * kcap;
  const int32_t* crow = cand + static_cast<long long>(bh) * kcap;
  int32_t* orow = idx + static_cast<long long>(bh) * kcap;

  // 1. masses: merge the workgroups' (max, sum) per query head as a
  // log-sum-exp (one wave per head, fixed order), then per candidate
  // m = (1/G) sum_g e_g * exp(m_w - M_g) / Z_g
  const int nw = (kcap + kMassRows - 1) / kMassRows;  // at most 128
  for (int g = wv; g < G; g += kMassNT / 64) {
    const double2* st = wstat + (static_cast<long long>(bh) * G + g) * nw;
    const double2 none = make_double2(-INFINITY, 0.0);
    const double2 s0 = lane < nw ? st[lane] : none;
    const double2 s1 = lane + 64 < nw ? st[lane + 64] : none;
    double M = fmax(s0.x, s1.x);
    for (int x = 32; x >= 1; x >>= 1) M = fmax(M, __shfl_xor(M, x));
    const double f0 = s0.x == -INFINITY ? 0.0 : exp(s0.x - M);
    const double f1 = s1.x == -INFINITY ? 0.0 : exp(s1.x - M);
    double Z = s0.y * f0 + s1.y * f1;
    for (int x = 32; x >= 1; x >>= 1) Z += __shfl_xor(Z, x);
    if (lane < nw) fac[lane][g] = f0 / Z / G;
    if (lane + 64 < nw) fac[lane + 64][g] = f1 / Z / G;
  }
  // this thread's candidates r = t + 1024 i: each row's G exponentials are
  // contiguous ([r][g]), every load independent of the others
  constexpr int kPer = kMassCap / kMassNT;
  bool live[kPer];
  double mr[kPer];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = t + i * kMassNT;
    const int j = r < kcap ? crow[r] : -1;
    live[i] = j >= 0 && j < n;
    double m = 0.0;
    if (r < kcap) {
      const double* er = lg + static_cast<long long>(r) * G;
#pragma unroll
      for (int g = 0; g < kMassGmax; ++g)
        if (g < G) m += er[g] * fac[r / kMassRows][g];
    }
    mr[i] = m;
  }
  uint64_t tloc = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int r = t + i * kMassNT;
    if (r >= kcap) break;
    uint64_t k = 0, f = 0;
    if (live[i]) {
      k = mass_key(mr[i]);
      f = mass_fixed(mr[i]);
    }
    okey[r] = k;
    fmv[r] = f;
    tloc += f;
  }
  tloc = wave_sum_u64(tloc);
  if (lane == 0) redu[wv] = tloc;
  if (t == 0) {
    s_prefix = 0;
    s_mhi = 0;
    s_state = 0;
    s_level = 0;
    s_nsmall = 0;
  }
  __syncthreads();
  uint64_t T = 0;
  for (int w = 0; w < kMassNT / 64; ++w) T += redu[w];
  uint64_t tgt = static_cast<uint64_t>(ceil(p * static_cast<double>(T)));
  if (tgt < 1) tgt = 1;
  if (tgt > T) tgt = T;

  uint64_t thr = ~0ull, need = 0;  // nothing kept unless set below
  if (T > 0) {
    // 2. radix select, one byte of the order key per level
    for (int level = 0; level < 8; ++level) {
      const int shift = 56 - 8 * level;
      const uint64_t prefix = s_prefix;
      if (t < 256) {
        hcnt[t] = 0;
        hsum[t] = 0;
      }
      __syncthreads();
      for (int base = wv * 64; base < kcap; base += kMassNT) {
        const int r = base + lane;  // every lane of the wave takes part
        const uint64_t k = r < kcap ? okey[r] : 0ull;
        const bool in = k != 0 && (level == 0 || (k >> (shift + 8)) == prefix);
        const uint32_t dgt = static_cast<uint32_t>(k >> shift) & 255u;
        const uint64_t f = in ? fmv[r] : 0ull;
        // lanes that share a digit add once: up to four digits per wave
        // this way (contended buckets), any others one lane at a time
        bool left = in;
        for (int it = 0; it < 4; ++it) {
          const unsigned long long act = __ballot(left);
          if (act == 0) break;
          const int lead = __ffsll(static_cast<long long>(act)) - 1;
          const uint32_t d0 = __shfl(dgt, lead);
          const bool mine = left && dgt == d0;
          const unsigned long long grp = __ballot(mine);
          const uint64_t fs = wave_sum_u64(mine ? f : 0ull);
          if (lane == lead) {
            atomicAdd(&hcnt[d0], static_cast<uint32_t>(__popcll(grp)));
            atomicAdd(&hsum[d0], static_cast<unsigned long long>(fs));
          }
          left = left && !mine;
        }
        if (left) {
          atomicAdd(&hcnt[dgt], 1u);
          atomicAdd(&hsum[dgt], static_cast<unsigned long long>(f));
        }
      }
      __syncthreads();
      if (wv == 0) {
        // lane i holds buckets 255 - 4i .. 252 - 4i, in descending order
        uint64_t part = 0;
        for (int u = 0; u < 4; ++u) part += hsum[255 - 4 * lane - u];
        uint64_t incl = part;
        for (int m = 1; m < 64; m <<= 1) {
          const uint64_t o = __shfl_up(incl, m);
          if (lane >= m) incl += o;
        }
        const uint64_t mhi = s_mhi;
        const unsigned long long rm = __ballot(mhi + incl >= tgt);
        const int first = rm ? __ffsll(static_cast<long long>(rm)) - 1 : 63;
        if (lane == first) {
          uint64_t acc = mhi + incl - part;
          int bstar = 252 - 4 * lane;
          for (int u = 0; u < 4; ++u) {
            const int bk = 255 - 4 * lane - u;
            if (acc + hsum[bk] >= tgt) {
              bstar = bk;
              break;
            }
            acc += hsum[bk];
          }
          s_mhi = acc;
          s_prefix = (prefix << 8) | static_cast<uint64_t>(bstar);
          s_level = level + 1;
          const uint32_t c = hcnt[bstar];
          s_state = c <= kMassSmall ? 1 : (level == 7 ? 2 : 0);
          if (c > 0) s_fmeq = hsum[bstar] / c;  // equal keys share one mass (level 7)
        }
      }
      __syncthreads();
      if (s_state != 0) break;
    }
    const int bits = 8 * s_level;
    const uint64_t P = s_prefix, mhi = s_mhi;
    if (s_state == 2) {
      // equal keys: take as many, by position, as the target still needs
      thr = P;
      const uint64_t fe = s_fmeq;
      need = fe == 0 ? 1 : (tgt - mhi + fe - 1) / fe;
    } else {
      // at most 64 candidates share the prefix: one wave sorts and cuts them
      for (int r = t; r < kcap; r += kMassNT) {
        const uint64_t k = okey[r];
        if (k != 0 && (bits == 64 ? k == P : (k >> (64 - bits)) == P)) {
          const int slot = atomicAdd(&s_nsmall, 1);
          small_key[slot] = k;
          small_fm[slot] = fmv[r];
          small_pos[slot] = static_cast<uint32_t>(r);
        }
      }
      __syncthreads();
      if (wv == 0) {
        const int ns = s_nsmall;
        uint64_t k = lane < ns ? small_key[lane] : 0ull;
        uint64_t f = lane < ns ? small_fm[lane] : 0ull;
        uint32_t ps = lane < ns ? small_pos[lane] : 0xffffffffu;
        for (int kk = 2; kk <= 64; kk <<= 1) {
          for (int jj = kk >> 1; jj > 0; jj >>= 1) {
            const uint64_t k2 = __shfl_xor(k, jj);
            const uint64_t f2 = __shfl_xor(f, jj);
            const uint32_t p2 = __shfl_xor(ps, jj);
            const bool mine_first = key_before(k, ps, k2, p2);
            const bool lower = (lane & jj) == 0, up = (lane & kk) == 0;
            if ((lower == up) != mine_first) {
              k = k2;
              f = f2;
              ps = p2;
            }
          }
        }
        uint64_t incl = f;
        for (int m = 1; m < 64; m <<= 1) {
          const uint64_t o = __shfl_up(incl, m);
          if (lane >= m) incl += o;
        }
        const unsigned long long rm = __ballot(lane < ns && mhi + incl >= tgt);
        const int cut = rm ? __ffsll(static_cast<long long>(rm)) - 1 : ns - 1;
        const uint64_t tk = __shfl(k, cut);
        const unsigned long long eq = __ballot(lane <= cut && k == tk);
        if (lane == 0) {
          s_thr = tk;
          s_need = static_cast<uint64_t>(__popcll(eq));
        }
      }
      __syncthreads();
      thr = s_thr;
      need = s_need;
    }
  }

  // 3. compaction in candidate order: contiguous positions per thread; one
  // scan of (candidates above the threshold, candidates at it) gives every
  // output position (those at it are kept up to need, by position)
  const int per = (kcap + kMassNT - 1) / kMassNT;
  const int q0 = min(t * per, kcap), q1 = min(q0 + per, kcap);
  uint32_t gtl = 0, eql = 0;
  for (int r = q0; r < q1; ++r) {
    const uint64_t k = okey[r];
    gtl += k != 0 && k > thr;
    eql += k != 0 && k == thr;
  }
  const uint64_t packed = block_excl_scan<uint64_t>((static_cast<uint64_t>(eql) << 32) | gtl, redu);
  uint64_t eqb = packed >> 32;
  int pos = static_cast<int>((packed & 0xffffffffu) + (eqb < need ? eqb : need));
  if (t == kMassNT - 1) {
    const uint64_t eqt = eqb + eql;
    s_total = static_cast<int>((packed & 0xffffffffu) + gtl + (eqt < need ? eqt : need));
  }
  for (int r = q0; r < q1; ++r) {
    const uint64_t k = okey[r];
    bool kp = k != 0 && k > thr;
    if (k != 0 && k == thr) kp = eqb++ < need;
    if (kp) orow[pos++] = crow[r];
  }
  __syncthreads();
  const int total = s_total;
  for (int r = total + t; r < kcap; r += kMassNT) orow[r] = -1;
  if (t == 0) counts[bh] = total;
}

// [B*Hq][kcap] doubles (exp of the logits), then [B*Hq][ceil(kcap/64)]
// (max, sum) pairs
static size_t mass_e_bytes(const hst_shape& s, int kcap) {
  return (static_cast<size_t>(s.B) * s.Hq * static_cast<size_t>(kcap) * 8 + 255) / 256 * 256;
}

size_t mass_logits_bytes(const hst_shape& s, int kcap) {
  const size_t nw = (static_cast<size_t>(kcap) + kMassRows - 1) / kMassRows;
  return mass_e_bytes(s, kcap) + static_cast<size_t>(s.B) * s.Hq * nw * 16;
}

template <typename K>
static hipError_t mass_lds_limit(K kern, size_t bytes) {
  return raise_lds_limit(reinterpret_cast<const void*>(kern), bytes);
}

hipError_t launch_select_mass(const hst_shape& s, const void* q, const void* K,
                              const int32_t* cand, int kcap, double p, float scale, int32_t* idx,
                              int32_t* counts, double* logits, hipStream_t st) {
  const dim3 lgrid(static_cast<unsigned>((kcap + kMassRows - 1) / kMassRows),
                   static_cast<unsigned>(s.B * s.Hkv));
  const double sc = static_cast<double>(scale);
  double2* wstat = reinterpret_cast<double2*>(reinterpret_cast<char*>(logits) +
                                              mass_e_bytes(s, kcap));
  if (s.kv_dtype == HST_F32) {
    if (s.d == 64)
      hipLaunchKernelGGL((mass_logits_kernel<float, 64>), lgrid, dim3(256), 0, st,
                         static_cast<const float*>(q), static_cast<const float*>(K), cand,
                         s.seq_lens, s.Hq, s.Hkv, s.Nmax, kcap, sc, logits, wstat);
    else
      hipLaunchKernelGGL((mass_logits_kernel<float, 128>), lgrid, dim3(256), 0, st,
                         static_cast<const float*>(q), static_cast<const float*>(K), cand,
                         s.seq_lens, s.Hq, s.Hkv, s.Nmax, kcap, sc, logits, wstat);
  } else {
    if (s.d == 64)
      hipLaunchKernelGGL((mass_logits_kernel<bf16, 64>), lgrid, dim3(256), 0, st,
                         static_cast<const bf16*>(q), static_cast<const bf16*>(K), cand,
                         s.seq_lens, s.Hq, s.Hkv, s.Nmax, kcap, sc, logits, wstat);
    else
      hipLaunchKernelGGL((mass_logits_kernel<bf16, 128>), lgrid, dim3(256), 0, st,
                         static_cast<const bf16*>(q), static_cast<const bf16*>(K), cand,
                         s.seq_lens, s.Hq, s.Hkv, s.Nmax, kcap, sc, logits, wstat);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t smem = static_cast<size_t>(kcap) * 16;
  e = mass_lds_limit(mass_pick_kernel, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mass_pick_kernel, dim3(s.B * s.Hkv), dim3(kMassNT), smem, st, logits, wstat,
                     cand, s.seq_lens, s.Hq, s.Hkv, s.Nmax, kcap, p, idx, counts);
  return hipGetLastError();
}

}  // namespace hst
