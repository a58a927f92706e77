// Selection and exact attention over the selected keys.
//  * Top-k (SOCKET overview page, "Core mechanism: soft LSH", item 4: the
//    top-k keys by soft score, chosen deterministically; ties go to the lower
//    index): each workgroup derives the head's selection from the candidate
//    slots itself and keeps the part of the ascending index row that falls in
//    its split, so no workgroup waits for another before the merge.
//  * Attention (same item: exact attention on that subset): a split-K flash
//    decode; each gathered K/V row is read once per kv head and used for all G
//    query heads of the group (grouped-query attention), with an online
//    softmax in the base-2 exponent domain.  The split states are merged
//    through their log-sum-exp (by the last split of a head to finish, or by
//    a second kernel when the rows are given).
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

// Device-coherent stores and loads of the split states (relaxed atomics at
// agent scope: they go to and come from the level every XCD shares, so no
// cache-wide write-back or invalidation is needed around them).
__device__ __forceinline__ void store_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The merge of the splits of one kv head's query heads, done by whichever
// split of the head finishes last.  Each split stores its state with
// store_dev, waits until those stores are complete, then adds one to the
// head's arrival count (an agent-scope atomic); the split that brings the
// count to nsplit reads the states with load_dev, merges the nsplit states of
// each query head through their log-sum-exp (weights 2^(m_s - max m); the
// weighted sum of l is the denominator) and resets the count for the next
// step.  smem: the workgroup's LDS (>= 16 KB + 64 B, free at this point).
template <int D, int NT>
__device__ __forceinline__ void merge_splits(const FusedArgs& a, int bh, long long qh0, int G, int nsplit,
                                             float* __restrict__ out, float* __restrict__ lse,
                                             unsigned char* smem, BlockScratch<NT>& sc) {
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's state stores are complete
  __syncthreads();
  if (t == 0)
    sc.found[0] = __hip_atomic_fetch_add(&a.heads[bh].arrive, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                          static_cast<uint32_t>(nsplit - 1)
                      ? 1
                      : 0;
  __syncthreads();
  if (sc.found[0] == 0) return;  // uniform
  const int GS = G * nsplit;
  HST_DCHECK(GS + 16 <= 16384, kDbgMergeLds);
  float* wt = reinterpret_cast<float*>(smem);  // [G][nsplit]: the weights
  float* ls = wt + GS;                         // [G]: sum of weighted l
  float* mx = ls + 8;                          // [G]: max m
  // this thread's first output: its partial outputs are in flight while the
  // weights are formed
  constexpr int PL = 32;
  const bool has0 = t < G * D;
  const int g0 = has0 ? t / D : 0, c0 = t % D;
  const float* po0 = a.part_o + (qh0 + g0) * nsplit * D + c0;
  float pv[PL];
#pragma unroll
  for (int u = 0; u < PL; ++u) pv[u] = has0 && u < nsplit ? load_dev(po0 + static_cast<long long>(u) * D) : 0.f;
  // wave g forms the weights of query head g (lanes over the splits).  The
  // (m, l) pairs of the first 64 * SPL splits are loaded together, in one
  // round trip; splits past those (nsplit > 128) are read twice.
  constexpr int SPL = 2;
  for (int g = wave; g < G; g += NW) {
    const float* pml = a.part_ml + (qh0 + g) * nsplit * 2;
    float mv[SPL], lv[SPL];
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int s = lane + 64 * u;
      mv[u] = s < nsplit ? load_dev(pml + 2 * s) : -INFINITY;
      lv[u] = s < nsplit ? load_dev(pml + 2 * s + 1) : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int u = 0; u < SPL; ++u) M = fmaxf(M, mv[u]);
    for (int s = lane + 64 * SPL; s < nsplit; s += 64) M = fmaxf(M, load_dev(pml + 2 * s));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float L = 0.f;
#pragma unroll
    for (int u = 0; u < SPL; ++u) {
      const int s = lane + 64 * u;
      if (s < nsplit) {
        const float w = mv[u] == -INFINITY || M == -INFINITY ? 0.f : exp2f(mv[u] - M);
        wt[g * nsplit + s] = w;
        L += w * lv[u];
      }
    }
    for (int s = lane + 64 * SPL; s < nsplit; s += 64) {
      const float m1 = load_dev(pml + 2 * s);
      const float w = m1 == -INFINITY || M == -INFINITY ? 0.f : exp2f(m1 - M);
      wt[g * nsplit + s] = w;
      L += w * load_dev(pml + 2 * s + 1);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) L += __shfl_xor(L, o, 64);
    if (lane == 0) {
      mx[g] = M;
      ls[g] = L;
    }
  }
  __syncthreads();
  for (int i = t; i < G * D; i += NT) {
    const int g = i / D, c = i % D;
    const float* po = a.part_o + (qh0 + g) * nsplit * D + c;
    const float* wg = wt + g * nsplit;
    float acc = 0.f;
    int s = 0;
    if (i == t) {
#pragma unroll
      for (int u = 0; u < PL; ++u)
        if (u < nsplit) acc += wg[u] * pv[u];
      s = PL;
    }
    for (; s < nsplit; ++s) acc += wg[s] * load_dev(po + static_cast<long long>(s) * D);
    const float L = ls[g];
    out[(qh0 + g) * D + c] = acc * (L > 0.f ? 1.f / L : 0.f);
    if (c == 0) lse[qh0 + g] = L > 0.f ? (mx[g] + log2f(L)) * kLn2F : -INFINITY;
  }
  if (t == 0) a.heads[bh].arrive = 0u;
}

// 1-D grid of nsplit * B*Hkv workgroups: workgroup i takes split s of head
// bh with xcd_item(i) = bh * nsplit + s, so that the splits of a head run on
// one XCD and share its L2 (the head's candidate slots, its partial states).
// Rows outside [0, N_b) are skipped.
//  * SELECT: every split derives the head's exact selection from the
//    candidate slots (in LDS when they fit; see select_from_candidates),
//    keeps the rows of its part [r0, r1) of the ascending index row, attends
//    over them and writes that part of the row (-1 past k_eff); the split
//    that finishes last merges the head's split states (merge_splits).
//  * !SELECT: rows come from idx; a second kernel merges the split states.
// Rows are gathered in batches of NG*U, the next batch in flight while one
// is consumed.  Without the selection, bf16 rows with up to four query heads
// per kv head fit 128 VGPRs, so that two workgroups share a CU.
template <typename T, int GMAX, bool SELECT>
constexpr bool kAttOcc2 = !SELECT && sizeof(T) == 2 && GMAX <= 4;  // two workgroups per CU

template <typename T, int D, int GMAX, bool SELECT>
__global__ void __launch_bounds__(kAttNT)
__attribute__((amdgpu_waves_per_eu(kAttOcc2<T, GMAX, SELECT> ? 4 : 1)))
attend_kernel(const T* __restrict__ q, const T* __restrict__ K, const T* __restrict__ V,
              int32_t* __restrict__ idx, const void* __restrict__ scores, int scores_int, int chunk,
              const int32_t* __restrict__ seq_lens, float scale_log2, FusedArgs a, float* __restrict__ out,
              float* __restrict__ lse) {
  constexpr int NT = kAttNT;
  constexpr int EPL = D / 16;
  constexpr int NW = NT / 64;
  constexpr int NG = NT / 16;
  constexpr int U = 4;
  // bf16 rows: q stays in packed bf16 pairs and each lane's part of a score is
  // a chain of pair dot products, scaled once after the row-group sum
  constexpr bool PK = sizeof(T) == 2;
  typedef typename RowLd<T, EPL>::raw Raw;
  extern __shared__ __align__(16) unsigned char sm[];
  __shared__ BlockScratch<NT> sc;
  __shared__ float red_ml[NW][GMAX][2];
  float* red_o = reinterpret_cast<float*>(sm);  // [NW][GMAX][D], after the selection
  const int nchunks = a.nchunks;
  int* offs = reinterpret_cast<int*>(sm + 65536 + 8192);
  int32_t* rows = reinterpret_cast<int32_t*>(sm + 65536 + 8192 + (nchunks + 1) * 4);
  const int Hq = a.Hq, Hkv = a.Hkv, G = Hq / Hkv;
  const int nsplit = a.nsplit;
  const int item = xcd_item(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
  const int bh = item / nsplit, split = item % nsplit, b = bh / Hkv, h = bh % Hkv;
  const int n = seq_len(seq_lens, b, a.Nmax) + (SELECT ? 0 : a.np);
  const int r0 = split * a.rps, r1 = min(r0 + a.rps, a.kcap);
  const int t = threadIdx.x, sub = t & 15, grp = t >> 4, lane = t & 63, wave = t >> 6;
  int32_t* irow = idx + static_cast<long long>(bh) * a.kcap;
  // the query rows, in flight during the selection
  Raw qr[GMAX];
#pragma unroll
  for (int g = 0; g < GMAX; ++g)
    if (g < G) qr[g] = RowLd<T, EPL>::load(q + (static_cast<long long>(b) * Hq + h * G + g) * D + sub * EPL);
  int nrows;
  SelectScratch ws{reinterpret_cast<uint32_t*>(sm), reinterpret_cast<int32_t*>(sm + 4 * kSelCap),
                   reinterpret_cast<uint32_t*>(sm + 65536), offs};
  if (SELECT) {
    // the head's k_eff, threshold and histogram shift, read before anything
    // else is in flight
    const HeadState& hs = a.heads[bh];
    const int k_eff = hs.k_eff;
    const uint32_t h_theta = hs.theta, h_shift = hs.shift;
    const int M = candidates_to_lds<NT>(a, bh, n, chunk, k_eff, ws, sc);
    const void* srow =
        scores != nullptr ? static_cast<const char*>(scores) + static_cast<long long>(bh) * a.Nmax * 4 : nullptr;
    const int path = select_from_candidates<NT>(a, bh, n, k_eff, chunk, M, h_theta, h_shift, srow,
                                                scores_int != 0, ws, r0, r1, nullptr, rows, sc);
    nrows = max(0, min(k_eff, r1) - r0);
    HST_DCHECK(nrows <= a.rps, kDbgRowLds);
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
  float m[GMAX], l[GMAX], o[GMAX][EPL];
#pragma unroll
  for (int g = 0; g < GMAX; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[g][e] = 0.f;
  }
  const long long kvb = static_cast<long long>(bh) * a.Nmax;
  // A batch: rows rb + u*NG (u < U) of this 16-lane group.  All loads of a
  // batch are issued back to back, without branches: a row that is absent or
  // out of range reads row 0 of the head (allocated whenever the head
  // exists) and is masked at use.
  const auto issue = [&](int rb, Raw (&kr)[U], Raw (&vr)[U], bool (&valid)[U]) {
    const T* kp[U];
    const T* vp[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = rb + u * NG;
      const int j = r < nrows ? rows[r] : -1;
      HST_DCHECK(!SELECT || r >= nrows || (j >= 0 && j < n), kDbgGatherRow);
      valid[u] = j >= 0 && j < n;
      const int jj = valid[u] ? j : 0;
      // a shared prefix row, or a row of the sequence's own cache
      const bool pre = !SELECT && jj < a.np;
      const long long off = pre ? (static_cast<long long>(h) * a.np + jj) * D + sub * EPL
                                : (kvb + (jj - (SELECT ? 0 : (valid[u] ? a.np : 0)))) * D + sub * EPL;
      kp[u] = (pre ? static_cast<const T*>(a.pk) : K) + off;
      vp[u] = (pre ? static_cast<const T*>(a.pv) : V) + off;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      kr[u] = RowLd<T, EPL>::load(kp[u]);
      vr[u] = RowLd<T, EPL>::load(vp[u]);
    }
  };
  // scores of a batch's rows for every query head slot (slots past G hold a
  // zero query and are never written out; an absent row scores -inf), then
  // one online-softmax step: the running state of each head is rescaled once
  // to the batch's new maximum, then the rows are added.  While a head has
  // seen no row its maximum stays -inf and the exponents are taken against
  // 0, so that every weight is exactly 0 (never NaN).
  const auto consume = [&](const Raw (&kr)[U], const Raw (&vr)[U], const bool (&ok)[U]) {
    float sc2[U][GMAX];
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
        sc2[u][g] = ok[u] ? s : -INFINITY;
      }
    }
    float pw[U][GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g) {
      float mx = m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) mx = fmaxf(mx, sc2[u][g]);
      const float ms = mx == -INFINITY ? 0.f : mx;
      const float c = __builtin_amdgcn_exp2f(m[g] - ms);
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pw[u][g] = __builtin_amdgcn_exp2f(sc2[u][g] - ms);
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
  };

  // Batches of BR rows.  Where the registers hold two batches, the next one
  // is in flight while one is consumed; where two workgroups share a CU (or
  // the registers hold one batch), batches go one at a time.
  constexpr int BR = NG * U;
  constexpr bool PIPE = !kAttOcc2<T, GMAX, SELECT> &&
                        (sizeof(T) == 2 ? !(D == 128 && GMAX == 8) : (D == 64 || GMAX <= 2));
  if constexpr (PIPE) {
    Raw ka[U], va[U], kb[U], vb[U];
    bool oka[U], okb[U];
    if (nrows > 0) issue(grp, ka, va, oka);
    for (int b0 = 0; b0 < nrows; b0 += 2 * BR) {
      if (b0 + BR < nrows) issue(b0 + BR + grp, kb, vb, okb);
      consume(ka, va, oka);
      if (b0 + 2 * BR < nrows) issue(b0 + 2 * BR + grp, ka, va, oka);
      if (b0 + BR < nrows) consume(kb, vb, okb);
    }
  } else {
    for (int b0 = 0; b0 < nrows; b0 += BR) {
      Raw ka[U], va[U];
      bool oka[U];
      issue(b0 + grp, ka, va, oka);
      consume(ka, va, oka);
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
  const long long qh0 = static_cast<long long>(b) * Hq + h * G;  // the group's first query head
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
    const long long pi = (qh0 + g) * nsplit + split;
    if (SELECT) {  // read by the merging split of the head (merge_splits)
      store_dev(a.part_o + pi * D + c, oo);
      if (c == 0) {
        store_dev(a.part_ml + pi * 2, mm);
        store_dev(a.part_ml + pi * 2 + 1, ll);
      }
    } else {
      a.part_o[pi * D + c] = oo;
      if (c == 0) {
        a.part_ml[pi * 2] = mm;
        a.part_ml[pi * 2 + 1] = ll;
      }
    }
  }
  if (SELECT)  // the split's part of the ascending index row, -1 past k_eff
    for (int i = r0 + t; i < r1; i += NT) irow[i] = i - r0 < nrows ? rows[i - r0] : -1;
  if constexpr (SELECT) merge_splits<D, NT>(a, bh, qh0, G, nsplit, out, lse, sm, sc);
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
                                  int chunk, float sl2, float* out, float* lse, hipStream_t st) {
  const int G = s.Hq / s.Hkv;
  const dim3 grid(static_cast<unsigned>(a_nsplit(a) * s.B * s.Hkv));
  const size_t smem = attend_smem(a.nchunks, a.rps);
#define HST_ATT(GM)                                                                             \
  do {                                                                                          \
    auto kern = attend_kernel<T, D, GM, SELECT>;                                                \
    hipError_t e = lds_limit(kern, smem);                                                       \
    if (e != hipSuccess) return e;                                                              \
    hipLaunchKernelGGL(kern, grid, dim3(kAttNT), smem, st, static_cast<const T*>(q),            \
                       static_cast<const T*>(K), static_cast<const T*>(V), idx, scores,         \
                       scores_int, chunk, s.seq_lens, sl2, a, out, lse);                        \
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
      e = select ? launch_attend_t<float, 64, true>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, out, lse, st)
                 : launch_attend_t<float, 64, false>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, out, lse, st);
    else
      e = select ? launch_attend_t<float, 128, true>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, out, lse, st)
                 : launch_attend_t<float, 128, false>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, out, lse, st);
  } else {
    if (s.d == 64)
      e = select ? launch_attend_t<bf16, 64, true>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, out, lse, st)
                 : launch_attend_t<bf16, 64, false>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, out, lse, st);
    else
      e = select ? launch_attend_t<bf16, 128, true>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, out, lse, st)
                 : launch_attend_t<bf16, 128, false>(s, a, q, K, V, idx, scores, scores_int, chunk, sl2, out, lse, st);
  }
  if (e != hipSuccess || select) return e;
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
