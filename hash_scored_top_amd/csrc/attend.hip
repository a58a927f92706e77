// Selection and exact attention over the selected keys.
//  * Top-k (SOCKET overview page, "Core mechanism: soft LSH", item 4: the
//    top-k keys by soft score, chosen deterministically; ties go to the lower
//    index): each workgroup derives the head's selection from the candidate
//    slots itself and keeps the part of the ascending index row that falls in
//    its split, so no workgroup waits for another.
//  * Attention (same item: exact attention on that subset): a split-K flash
//    decode; each gathered K/V row is read once per kv head and used for all G
//    query heads of the group (grouped-query attention), with an online
//    softmax in the base-2 exponent domain.  A second kernel merges the split
//    states through their log-sum-exp.
#include "fused_device.h"
#include "hst_launch.h"

namespace hst {

constexpr int kAttNT = 512;
constexpr int kSelNT = 1024;

// A lane's EPL elements of a K/V/q row: raw load (issued first, so that all
// loads of a batch are in flight together) and conversion to float.
template <typename T, int EPL>
struct RowLd;
template <>
struct RowLd<bf16, 8> {
  typedef u32x4 raw;
  static __device__ __forceinline__ raw load(const bf16* p) { return *reinterpret_cast<const u32x4*>(p); }
  static __device__ __forceinline__ uint32_t word(const raw& v, int i) { return v[i]; }
  static __device__ __forceinline__ void cvt(const raw& v, float (&x)[8]) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
};
template <>
struct RowLd<bf16, 4> {
  typedef uint2 raw;
  static __device__ __forceinline__ raw load(const bf16* p) { return *reinterpret_cast<const uint2*>(p); }
  static __device__ __forceinline__ uint32_t word(const raw& v, int i) { return i == 0 ? v.x : v.y; }
  static __device__ __forceinline__ void cvt(const raw& v, float (&x)[4]) {
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  }
};
struct U32x8 {
  u32x4 a, b;
};
template <>
struct RowLd<float, 8> {
  typedef U32x8 raw;
  static __device__ __forceinline__ raw load(const float* p) {
    return U32x8{reinterpret_cast<const u32x4*>(p)[0], reinterpret_cast<const u32x4*>(p)[1]};
  }
  static __device__ __forceinline__ void cvt(const raw& v, float (&x)[8]) {
    x[0] = __uint_as_float(v.a.x); x[1] = __uint_as_float(v.a.y);
    x[2] = __uint_as_float(v.a.z); x[3] = __uint_as_float(v.a.w);
    x[4] = __uint_as_float(v.b.x); x[5] = __uint_as_float(v.b.y);
    x[6] = __uint_as_float(v.b.z); x[7] = __uint_as_float(v.b.w);
  }
};
template <>
struct RowLd<float, 4> {
  typedef u32x4 raw;
  static __device__ __forceinline__ raw load(const float* p) { return *reinterpret_cast<const u32x4*>(p); }
  static __device__ __forceinline__ void cvt(const raw& v, float (&x)[4]) {
    x[0] = __uint_as_float(v.x); x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z); x[3] = __uint_as_float(v.w);
  }
};

// Dot product of two packed bf16 pairs added to c: both products are exact in
// fp32, the sum is taken in fp32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float dot2_bf16(uint32_t x, uint32_t y, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), __builtin_bit_cast(bf16x2, y), c,
                                         false);
}

// LDS of the attend kernel: [64 KB: candidate keys and indices, later the
// wave partials][hist 8 KB][chunk offsets][rows of this split]
static_assert(8 * kSelCap <= 65536, "candidate region");
size_t attend_smem(int nchunks, int rps) {
  return 65536 + 8192 + static_cast<size_t>(nchunks + 1) * 4 + static_cast<size_t>(rps) * 4;
}

// grid (nsplit, B*Hkv).  SELECT: rows come from the head's selection (and
// the split's part of the index row is written to idx); otherwise rows are
// read from idx.  Rows outside [0, N_b) are skipped.
// bf16 rows with up to four query heads per kv head fit 128 VGPRs, so that two
// workgroups share a CU.
template <typename T, int D, int GMAX, bool SELECT>
__global__ void __launch_bounds__(kAttNT)
__attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 && GMAX <= 4 ? 4 : 1)))
attend_kernel(const T* __restrict__ q, const T* __restrict__ K, const T* __restrict__ V,
              int32_t* __restrict__ idx, const void* __restrict__ scores, int scores_int, int chunk,
              const int32_t* __restrict__ seq_lens, float scale_log2, FusedArgs a) {
  constexpr int NT = kAttNT;
  constexpr int EPL = D / 16;
  constexpr int NW = NT / 64;
  constexpr int NG = NT / 16;
  constexpr int U = 4;
  // bf16 rows: q stays in packed bf16 pairs and each lane's part of a score is
  // a chain of pair dot products, scaled once after the row-group sum
  constexpr bool PK = sizeof(T) == 2;
  extern __shared__ __align__(16) unsigned char sm[];
  __shared__ BlockScratch<NT> sc;
  __shared__ float red_ml[NW][GMAX][2];
  float* red_o = reinterpret_cast<float*>(sm);  // [NW][GMAX][D], after the selection
  const int nchunks = a.nchunks;
  int* offs = reinterpret_cast<int*>(sm + 65536 + 8192);
  int32_t* rows = reinterpret_cast<int32_t*>(sm + 65536 + 8192 + (nchunks + 1) * 4);
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const int bh = blockIdx.y, b = bh / Hkv, h = bh % Hkv;
  const int n = seq_len(seq_lens, b, a.Nmax) + (SELECT ? 0 : a.np);
  const int split = blockIdx.x, nsplit = gridDim.x;
  const int r0 = split * a.rps, r1 = min(r0 + a.rps, a.kcap);
  const int t = threadIdx.x, sub = t & 15, grp = t >> 4, lane = t & 63, wave = t >> 6;
  int32_t* irow = idx + static_cast<long long>(bh) * a.kcap;
  int nrows;
  if (SELECT) {
    const int k_eff = a.heads[bh].k_eff;
    SelectScratch ws{reinterpret_cast<uint32_t*>(sm), reinterpret_cast<int32_t*>(sm + 4 * kSelCap),
                     reinterpret_cast<uint32_t*>(sm + 65536), offs};
    int M = 0;
    const void* srow =
        scores != nullptr ? static_cast<const char*>(scores) + static_cast<long long>(bh) * a.Nmax * 4 : nullptr;
    const int path = select_range<NT>(a, bh, n, k_eff, chunk, srow, scores_int != 0, ws, r0, r1, irow,
                                      rows, sc, &M);
    nrows = max(0, min(k_eff, r1) - r0);
    if (split == 0 && t == 0) {
      a.heads[bh].path = static_cast<uint32_t>(path);
      a.heads[bh].cand_total = static_cast<uint32_t>(M);
    }
  } else {
    nrows = max(0, r1 - r0);
    for (int i = t; i < nrows; i += NT) rows[i] = irow[r0 + i];
  }
  __syncthreads();

  float qv[GMAX][EPL];
  uint32_t qp[GMAX][EPL / 2];
  {
    typename RowLd<T, EPL>::raw qr[GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
      if (g < G) qr[g] = RowLd<T, EPL>::load(q + (static_cast<long long>(b) * Hq + h * G + g) * D + sub * EPL);
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if constexpr (PK) {
#pragma unroll
        for (int w = 0; w < EPL / 2; ++w) qp[g][w] = g < G ? RowLd<T, EPL>::word(qr[g], w) : 0u;
      } else if (g < G) {
        RowLd<T, EPL>::cvt(qr[g], qv[g]);
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[g][e] *= scale_log2;
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) qv[g][e] = 0.f;
      }
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
  const long long kvb = static_cast<long long>(bh) * a.Nmax;
  for (int rb = grp; rb < nrows; rb += NG * U) {
    // all row loads of the batch issued back to back, without branches: a
    // row that is absent or out of range reads row 0 of the head (allocated
    // whenever the head exists) and is skipped below
    typename RowLd<T, EPL>::raw kr[U], vr[U];
    bool ok[U];
    const T* kp[U];
    const T* vp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + u * NG;
      const int j = r < nrows ? rows[r] : -1;
      ok[u] = j >= 0 && j < n;
      const int jj = ok[u] ? j : 0;
      // a shared prefix row, or a row of the sequence's own cache
      const bool pre = !SELECT && jj < a.np;
      const long long off = pre ? (static_cast<long long>(h) * a.np + jj) * D + sub * EPL
                                : (kvb + (jj - (SELECT ? 0 : (ok[u] ? a.np : 0)))) * D + sub * EPL;
      kp[u] = (pre ? static_cast<const T*>(a.pk) : K) + off;
      vp[u] = (pre ? static_cast<const T*>(a.pv) : V) + off;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kr[u] = RowLd<T, EPL>::load(kp[u]);
      vr[u] = RowLd<T, EPL>::load(vp[u]);
    }
    // scores of the batch's rows for every query head slot (slots past G
    // hold a zero query and are never written out); an absent row scores -inf
    float sc[U][GMAX];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kx[EPL];
      if constexpr (!PK) RowLd<T, EPL>::cvt(kr[u], kx);
#pragma unroll
      for (int g = 0; g < GMAX; ++g) {
        float s = 0.f;
        if constexpr (PK) {
#pragma unroll
          for (int w = 0; w < EPL / 2; ++w) s = dot2_bf16(qp[g][w], RowLd<T, EPL>::word(kr[u], w), s);
        } else {
#pragma unroll
          for (int e = 0; e < EPL; ++e) s += qv[g][e] * kx[e];
        }
        // sum over the 16 lanes of the row group, all in-row DPP (no LDS
        // crossbar): rotations by 8 and 4, then the quad exchanges; every
        // lane ends with the same sum.  Every lane of a row rotation reads a
        // lane of its own row, so bound_ctrl changes nothing there; set, it
        // lets the move fold into the add.
        s += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), 0x128, 0xF, 0xF, true));
        s += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), 0x124, 0xF, 0xF, true));
        s += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), 0x4E, 0xF, 0xF, true));
        s += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(s), 0xB1, 0xF, 0xF, true));
        if constexpr (PK) s *= scale_log2;
        sc[u][g] = ok[u] ? s : -INFINITY;
      }
    }
    // one online-softmax step per batch: the running state of each head is
    // rescaled once to the batch's new maximum, then the rows are added.
    // While a head has seen no row its maximum stays -inf and the exponents
    // are taken against 0, so that every weight is exactly 0 (never NaN).
    float pw[U][GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc[u][g]);
      const float ms = mx == -INFINITY ? 0.f : mx;
      const float c = __builtin_amdgcn_exp2f(m[g] - ms);
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pw[u][g] = __builtin_amdgcn_exp2f(sc[u][g] - ms);
        ps += pw[u][g];
      }
      l[g] = l[g] * c + ps;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[g][e] *= c;
      m[g] = mx;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vx[EPL];
      RowLd<T, EPL>::cvt(vr[u], vx);
#pragma unroll
      for (int g = 0; g < GMAX; ++g)
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[g][e] += pw[u][g] * vx[e];
    }
  }
  // merge the row groups of a wave (lanes 16 apart, then 32 apart), then the
  // waves.  A lane swap (v_permlane16/32_swap of a value with itself) gives
  // every lane the pair's two states in the same order, so both lanes of a
  // pair compute the same merge, without the LDS crossbar.
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    if (g >= G) break;
#pragma unroll
    for (int x = 16; x <= 32; x <<= 1) {
      const auto pair = [x](float v) {
        const uint32_t u = __float_as_uint(v);
        if (x == 16) {
          const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
          return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
        }
        const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        return make_float2(__uint_as_float(r[0]), __uint_as_float(r[1]));
      };
      const float2 mp = pair(m[g]), lp = pair(l[g]);
      const float mn = fmaxf(mp.x, mp.y);
      const float c1 = mn == -INFINITY ? 0.f : exp2f(mp.x - mn);
      const float c2 = mn == -INFINITY ? 0.f : exp2f(mp.y - mn);
      l[g] = lp.x * c1 + lp.y * c2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float2 op = pair(o[g][e]);
        o[g][e] = op.x * c1 + op.y * c2;
      }
      m[g] = mn;
    }
  }
  __syncthreads();  // the candidate region becomes red_o
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      if (g >= G) break;
      if (lane == 0) {
        red_ml[wave][g][0] = m[g];
        red_ml[wave][g][1] = l[g];
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) red_o[(wave * GMAX + g) * D + lane * EPL + e] = o[g][e];
    }
  }
  __syncthreads();
  for (int i = t; i < G * D; i += NT) {
    const int g = i / D, c = i % D;
    float mm = -INFINITY;
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, red_ml[w][g][0]);
    float ll = 0.f, oo = 0.f;
    if (mm != -INFINITY) {
      for (int w = 0; w < NW; ++w) {
        const float wt = exp2f(red_ml[w][g][0] - mm);
        ll += red_ml[w][g][1] * wt;
        oo += red_o[(w * GMAX + g) * D + c] * wt;
      }
    }
    const long long pi = (static_cast<long long>(b) * Hq + h * G + g) * nsplit + split;
    a.part_o[pi * D + c] = oo;
    if (c == 0) {
      a.part_ml[pi * 2] = mm;
      a.part_ml[pi * 2 + 1] = ll;
    }
  }
}

// Merge the split states of one query head.  grid (B*Hq), 256 threads.
// Thread t owns column block c = t % (D/4) (four output elements) of the
// splits so, so + SP, ... (so = t / (D/4)); the (m, l) pairs and the partial
// outputs are loaded together (one round trip), then weighted by
// 2^(m_s - max m) and summed; the sum of weights times l is the denominator.
template <int D>
__global__ void __launch_bounds__(256)
combine_kernel(int nsplit, const float* __restrict__ part_o, const float* __restrict__ part_ml,
               float* __restrict__ out, float* __restrict__ lse) {
  constexpr int NT = 256, CW = D / 4, SP = NT / CW, NW = NT / 64;
  constexpr int B8 = 8;  // partial-output loads per thread per batch
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[2][NW];
  __shared__ u32x4 accs[SP][CW];
  const long long qh = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int c = t % CW, so = t / CW;
  const float* po = part_o + qh * nsplit * D;
  // first batch of partial outputs and this thread's (m, l) pair, together
  u32x4 ov[B8];
#pragma unroll
  for (int i = 0; i < B8; ++i) {
    const int sp = so + i * SP;
    ov[i] = reinterpret_cast<const u32x4*>(po)[(sp < nsplit ? sp : nsplit - 1) * CW + c];
  }
  const float2 ml = t < nsplit ? reinterpret_cast<const float2*>(part_ml)[qh * nsplit + t]
                               : make_float2(-INFINITY, 0.f);
  // M = max m; weights; L = sum w * l
  float M = ml.x;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  if (lane == 0) red[0][wave] = M;
  __syncthreads();
  M = red[0][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, red[0][w]);
  const float wv = (ml.x == -INFINITY || M == -INFINITY) ? 0.f : exp2f(ml.x - M);
  if (t < nsplit) wgt[t] = wv;
  float Ls = wv * ml.y;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) Ls += __shfl_xor(Ls, o, 64);
  if (lane == 0) red[1][wave] = Ls;
  __syncthreads();
  Ls = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) Ls += red[1][w];
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int i0 = 0; i0 < nsplit; i0 += B8 * SP) {
    if (i0 > 0) {
#pragma unroll
      for (int i = 0; i < B8; ++i) {
        const int sp = so + i0 + i * SP;
        ov[i] = reinterpret_cast<const u32x4*>(po)[(sp < nsplit ? sp : nsplit - 1) * CW + c];
      }
    }
#pragma unroll
    for (int i = 0; i < B8; ++i) {
      const int sp = so + i0 + i * SP;
      if (sp < nsplit) {
        const float w = wgt[sp];
        a0 += w * __uint_as_float(ov[i].x);
        a1 += w * __uint_as_float(ov[i].y);
        a2 += w * __uint_as_float(ov[i].z);
        a3 += w * __uint_as_float(ov[i].w);
      }
    }
  }
  accs[so][c] = u32x4{__float_as_uint(a0), __float_as_uint(a1), __float_as_uint(a2), __float_as_uint(a3)};
  __syncthreads();
  if (t < CW) {
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
#pragma unroll
    for (int k = 0; k < SP; ++k) {
      const u32x4 v = accs[k][t];
      r0 += __uint_as_float(v.x);
      r1 += __uint_as_float(v.y);
      r2 += __uint_as_float(v.z);
      r3 += __uint_as_float(v.w);
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    reinterpret_cast<float4*>(out + qh * D)[t] = make_float4(r0 * inv, r1 * inv, r2 * inv, r3 * inv);
  }
  if (t == 0 && lse != nullptr) lse[qh] = Ls > 0.f ? (M + log2f(Ls)) * kLn2F : -INFINITY;
}

// Stand-alone top-k: one workgroup per (sequence, kv head) writes the row.
__global__ void __launch_bounds__(kSelNT)
select_kernel(int32_t* __restrict__ idx, const void* __restrict__ scores, int scores_int, int chunk,
              const int32_t* __restrict__ seq_lens, FusedArgs a) {
  extern __shared__ __align__(16) unsigned char sm[];
  __shared__ BlockScratch<kSelNT> sc;
  const int bh = blockIdx.x, b = bh / a.Hkv;
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int k_eff = a.heads[bh].k_eff;
  SelectScratch ws{reinterpret_cast<uint32_t*>(sm), reinterpret_cast<int32_t*>(sm + 4 * kSelCap),
                   reinterpret_cast<uint32_t*>(sm + 65536), reinterpret_cast<int*>(sm + 65536 + 8192)};
  int M = 0;
  const void* srow =
      scores != nullptr ? static_cast<const char*>(scores) + static_cast<long long>(bh) * a.Nmax * 4 : nullptr;
  const int path = select_range<kSelNT>(a, bh, n, k_eff, chunk, srow, scores_int != 0, ws, 0, a.kcap,
                                        idx + static_cast<long long>(bh) * a.kcap, nullptr, sc, &M);
  if (threadIdx.x == 0) {
    a.heads[bh].path = static_cast<uint32_t>(path);
    a.heads[bh].cand_total = static_cast<uint32_t>(M);
  }
}

// The candidates the filtering scan left for each head, in index order: the
// (order key, index) pairs of its chunk slots, up to cap of them, their count
// and the head's threshold.  One workgroup per (sequence, kv head).
__global__ void __launch_bounds__(256)
candidates_kernel(FusedArgs a, int chunk, const int32_t* __restrict__ seq_lens, uint32_t* __restrict__ keys,
                  int32_t* __restrict__ index, int32_t* __restrict__ count, uint32_t* __restrict__ theta,
                  int cap) {
  __shared__ int offs[kMaxChunks + 1];
  const int bh = blockIdx.x, b = bh / a.Hkv;
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int nch = (n + a.span - 1) / a.span;
  const uint32_t* cnt = a.counts + static_cast<long long>(bh) * a.nchunks;
  const uint2* slots = a.slots + static_cast<long long>(bh) * a.nchunks * chunk;
  if (threadIdx.x == 0) {
    int run = 0;
    for (int c = 0; c < nch; ++c) {
      offs[c] = run;
      run += static_cast<int>(cnt[c]);
    }
    offs[nch] = run;
    count[bh] = run;
    theta[bh] = a.heads[bh].theta;
  }
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int m = offs[c + 1] - offs[c];
    for (int i = threadIdx.x; i < m; i += blockDim.x) {
      const int p = offs[c] + i;
      if (p < cap) {
        const uint2 v = slots[static_cast<long long>(c) * chunk + i];
        keys[static_cast<long long>(bh) * cap + p] = v.x;
        index[static_cast<long long>(bh) * cap + p] = static_cast<int32_t>(v.y);
      }
    }
  }
}

hipError_t launch_candidates(const hst_shape& s, const FusedArgs& a, int chunk, uint32_t* keys, int32_t* index,
                             int32_t* count, uint32_t* theta, int cap, hipStream_t st) {
  if (a.nchunks > kMaxChunks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(candidates_kernel, dim3(s.B * s.Hkv), dim3(256), 0, st, a, chunk, s.seq_lens, keys, index,
                     count, theta, cap);
  return hipGetLastError();
}

// Raises a kernel's dynamic LDS limit (kept per kernel and device).
template <typename K>
static hipError_t lds_limit(K kern, size_t bytes) {
  return raise_lds_limit(reinterpret_cast<const void*>(kern), bytes);
}

template <typename T, int D, bool SELECT>
static hipError_t launch_attend_t(const hst_shape& s, const FusedArgs& a, const void* q, const void* K,
                                  const void* V, int32_t* idx, const void* scores, int scores_int,
                                  int chunk, float sl2, hipStream_t st) {
  const int G = s.Hq / s.Hkv;
  dim3 grid(a_nsplit(a), s.B * s.Hkv);
  const size_t smem = attend_smem(a.nchunks, a.rps);
#define HST_ATT(GM)                                                                             \
  do {                                                                                          \
    auto kern = attend_kernel<T, D, GM, SELECT>;                                                \
    hipError_t e = lds_limit(kern, smem);                                                       \
    if (e != hipSuccess) return e;                                                              \
    hipLaunchKernelGGL(kern, grid, dim3(kAttNT), smem, st, static_cast<const T*>(q),            \
                       static_cast<const T*>(K), static_cast<const T*>(V), idx, scores,         \
                       scores_int, chunk, s.seq_lens, sl2, a);                                  \
  } while (0)
  if (G <= 1) HST_ATT(1);
  else if (G <= 2) HST_ATT(2);
  else if (G <= 4) HST_ATT(4);
  else HST_ATT(8);
#undef HST_ATT
  return hipGetLastError();
}

template <int D>
static hipError_t launch_combine_t(const hst_shape& s, const FusedArgs& a, float* out, float* lse,
                                   hipStream_t st) {
  hipLaunchKernelGGL((combine_kernel<D>), dim3(s.B * s.Hq), dim3(256), 0, st, a_nsplit(a), a.part_o,
                     a.part_ml, out, lse);
  return hipGetLastError();
}

hipError_t launch_attend(const hst_shape& s, const FusedArgs& a, const void* q, const void* K,
                         const void* V, int32_t* idx, bool select, const void* scores, int scores_int,
                         int chunk, float scale, float* out, float* lse, hipStream_t st) {
  const float sl2 = scale * kLog2eF;
  hipError_t e;
  if (s.kv_dtype == HST_F32) {
    if (s.d == 64)
      e = select ? launch_attend_t<float, 64, true>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, st)
                 : launch_attend_t<float, 64, false>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, st);
    else
      e = select ? launch_attend_t<float, 128, true>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, st)
                 : launch_attend_t<float, 128, false>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, st);
  } else {
    if (s.d == 64)
      e = select ? launch_attend_t<bf16, 64, true>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, st)
                 : launch_attend_t<bf16, 64, false>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, st);
    else
      e = select ? launch_attend_t<bf16, 128, true>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, st)
                 : launch_attend_t<bf16, 128, false>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, st);
  }
  if (e != hipSuccess) return e;
  return s.d == 64 ? launch_combine_t<64>(s, a, out, lse, st) : launch_combine_t<128>(s, a, out, lse, st);
}

hipError_t launch_select_only(const hst_shape& s, const FusedArgs& a, int32_t* idx, const void* scores,
                              int scores_int, int chunk, hipStream_t st) {
  const size_t smem = 65536 + 8192 + static_cast<size_t>(a.nchunks + 1) * 4;
  hipError_t e = lds_limit(select_kernel, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, dim3(s.B * s.Hkv), dim3(kSelNT), smem, st, idx, scores, scores_int,
                     chunk, s.seq_lens, a);
  return hipGetLastError();
}

}  // namespace hst
