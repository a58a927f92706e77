// The key scan, the bandwidth-dominant stage of a decode step: every cached
// key's metadata is read from HBM exactly once, scored, and (when a top-k
// follows) appended to its chunk's candidate slots if it scores >= theta.
//  * Soft-collision score (SOCKET overview page, "Core mechanism: soft LSH",
//    item 3): score_j = ||v_j|| * sum_l T[id_{j,l}][l], the kv head's
//    bucket-major table T resident in LDS.  Each key's L ids are split over
//    L/16 lanes; lane groups visit their 16 tables in an order rotated by the
//    key's slot in the wave so the 64 lanes of a wave hit distinct LDS banks.
//  * Code similarity (HATA explainer page, section 3): XOR + popcount of
//    128-bit codes against the G query codes.
//  * Given scores (the stand-alone top-k): the scores are only filtered.
//
// The candidate threshold of each head is derived from the key sample prep
// gathered by a small kernel that runs before the scan (threshold_kernel).
#include "fused_device.h"
#include "hst_launch.h"

namespace hst {

constexpr int kScanNT = 1024;
constexpr int kSoftChunk = 2048;
constexpr int kLaneChunk = 4096;
static_assert(kSoftChunk >= kSample && kLaneChunk >= kSample && kSample >= 2048,
              "chunk tile holds the sample scores and doubles as the select histogram");
constexpr int kThetaSpin = 1 << 16;
constexpr int kScanSoftU = 2;  // key batches per lane group in flight (two workgroups fit a CU)  // polls of the threshold word before falling back

template <int LANES, int NT, int U>
struct SoftScorer {
  static constexpr int L = 16 * LANES;
  static constexpr int KPI = NT / LANES;  // keys per batch
  static constexpr int TILE = KPI * U;
  const uint4* idv;
  const void* vnorm;
  int norm_f16;
  const float* tbl;  // LDS
  uint32_t idmask;   // 2^P - 1: ids outside the table cannot leave it
  int sub, grp;

  __device__ __forceinline__ void setup() {
    sub = threadIdx.x % LANES;
    grp = threadIdx.x / LANES;
  }
  __device__ __forceinline__ void load(uint4 (&w)[U], float (&nr)[U], long long base, int jb,
                                       int jend) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * KPI;
      if (j < jend) {
        w[u] = idv[(base + j) * LANES + sub];
        nr[u] = norm_f16 ? f16_bits_to_f32(static_cast<const uint16_t*>(vnorm)[base + j])
                         : static_cast<const float*>(vnorm)[base + j];
      }
    }
  }
  // scores of the batch held in (w, nr) into out[j - j0]
  __device__ __forceinline__ void compute(const uint4 (&w)[U], const float (&nr)[U], int jb, int jend,
                                          int j0, float* out) const {
    const int k = grp & 15;
    const int qw = k >> 2, sh = k & 3;
    const char* tb = reinterpret_cast<const char*>(tbl);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * KPI;
      if (j < jend) {  // uniform over the LANES lanes of a key
        const uint32_t a0 = w[u].x, a1 = w[u].y, a2 = w[u].z, a3 = w[u].w;
        const uint32_t u0 = qw == 0 ? a0 : qw == 1 ? a1 : qw == 2 ? a2 : a3;
        const uint32_t u1 = qw == 0 ? a1 : qw == 1 ? a2 : qw == 2 ? a3 : a0;
        const uint32_t u2 = qw == 0 ? a2 : qw == 1 ? a3 : qw == 2 ? a0 : a1;
        const uint32_t u3 = qw == 0 ? a3 : qw == 1 ? a0 : qw == 2 ? a1 : a2;
        uint32_t c[4];
        c[0] = __builtin_amdgcn_alignbyte(u1, u0, sh);
        c[1] = __builtin_amdgcn_alignbyte(u2, u1, sh);
        c[2] = __builtin_amdgcn_alignbyte(u3, u2, sh);
        c[3] = __builtin_amdgcn_alignbyte(u0, u3, sh);
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const uint32_t id0 = (c[i >> 2] >> ((i & 3) * 8)) & idmask;
          const uint32_t id1 = (c[(i + 1) >> 2] >> (((i + 1) & 3) * 8)) & idmask;
          const int l0 = sub * 16 + ((i + k) & 15), l1 = sub * 16 + ((i + 1 + k) & 15);
          acc0 += *reinterpret_cast<const float*>(tb + (id0 * L + l0) * 4);
          acc1 += *reinterpret_cast<const float*>(tb + (id1 * L + l1) * 4);
        }
        const float sv = group_sum<LANES>(acc0 + acc1) * nr[u];
        if (sub == 0) out[j - j0] = sv;
      }
    }
  }
};

// Scores of keys [j0, jend) (rows base + j) into out[j - j0]; (w, nr) hold the
// first batch, already loaded.  The next batch is in flight during each
// batch's table lookups.
template <class S, int U>
__device__ __forceinline__ void soft_score_range(const S& sco, long long base, int j0, int jend,
                                                 uint4 (&w)[U], float (&nr)[U], float* out) {
  uint4 wn[U];
  float nn[U];
  for (int t0 = j0; t0 < jend; t0 += S::TILE) {
    const int jb = t0 + sco.grp;
    const bool more = t0 + S::TILE < jend;
    if (more) sco.load(wn, nn, base, jb + S::TILE, jend);
    sco.compute(w, nr, jb, jend, j0, out);
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        w[u] = wn[u];
        nr[u] = nn[u];
      }
    }
  }
}

// The chunk's scores sit in LDS (tile[0..cnt)): write them out (coalesced)
// and append the keys scoring >= theta, in index order, to the chunk's
// candidate slots.  Returns the candidate count (every thread).
template <int NT, bool KINT>
__device__ __forceinline__ int scan_chunk_epilogue(const uint32_t* tile, int cnt, int j0,
                                                   long long base, uint32_t* scores_out,
                                                   uint32_t theta, bool filter, uint2* slot,
                                                   BlockScratch<NT>& sc) {
  if (scores_out != nullptr)
    for (int i = threadIdx.x; i < cnt; i += NT) scores_out[base + j0 + i] = tile[i];
  if (!filter) return 0;
  const int per = (cnt + NT - 1) / NT;  // thread t owns [t*per, t*per + per)
  const int i0 = threadIdx.x * per;
  int nc = 0;
  for (int e = 0; e < per; ++e) {
    const int i = i0 + e;
    if (i < cnt) {
      const uint32_t key = KINT ? order_key_i32(static_cast<int32_t>(tile[i]))
                                : order_key_f32(__uint_as_float(tile[i]));
      nc += key >= theta;
    }
  }
  int tot;
  int pos = block_excl_scan<NT>(nc, sc, tot);
  for (int e = 0; e < per && nc > 0; ++e) {
    const int i = i0 + e;
    if (i < cnt) {
      const uint32_t key = KINT ? order_key_i32(static_cast<int32_t>(tile[i]))
                                : order_key_f32(__uint_as_float(tile[i]));
      if (key >= theta) {
        slot[pos++] = make_uint2(key, static_cast<uint32_t>(j0 + i));
        --nc;
      }
    }
  }
  return tot;
}


// Candidate threshold of head bh from the sample prep gathered; every thread
// of the workgroup calls.  LDS: the head's table (soft-LSH, as the scan holds
// it), the query codes (binary codes), kSample words of scratch in tile.
template <int KIND, int LANES>
__device__ uint32_t sample_theta(const FusedArgs& a, int bh, int n, int k_eff, const float* tbl,
                                 const uint32_t* qc, uint32_t* tile, BlockScratch<kScanNT>& sc) {
  // (the whole sample in one batch: every lane's loads in flight together)
  constexpr int NT = kScanNT;
  constexpr int PER = kSample / NT;
  const int S = a.sample > n ? n : a.sample;
  const int r = sample_rank(k_eff, n, S);
  if (!(S > 0 && k_eff > 0 && r < S)) return 0u;
  const int t = threadIdx.x;
  const long long sb = static_cast<long long>(bh) * kSample;
  uint32_t key[PER];
  if (KIND == kScanSoftFast) {
    constexpr int U = kSample * LANES / NT;
    SoftScorer<LANES, NT, U> ss;
    ss.idv = reinterpret_cast<const uint4*>(a.samp);
    ss.vnorm = a.samp_vn;
    ss.norm_f16 = 0;
    ss.tbl = tbl;
    ss.idmask = (1u << a.P) - 1u;
    ss.setup();
    uint4 w[U];
    float nr[U];
    ss.load(w, nr, sb, ss.grp, S);
    ss.compute(w, nr, ss.grp, S, 0, reinterpret_cast<float*>(tile));
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = t + e * NT;
      key[e] = i < S ? order_key_f32(__uint_as_float(tile[i])) : 0u;
    }
  } else if (KIND == kScanSoftAny) {
    const uint32_t idm = (1u << a.P) - 1u;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = t + e * NT;
      float sv = 0.f;
      if (i < S) {
        const uint8_t* row = a.samp + (sb + i) * a.L;
        for (int l = 0; l < a.L; ++l) sv += tbl[(row[l] & idm) * a.L + l];
        sv *= a.samp_vn[sb + i];
      }
      key[e] = order_key_f32(sv);
    }
  } else if (KIND == kScanHamming) {
    const int G = a.Hq / a.Hkv;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = t + e * NT;
      int ham = 0;
      if (i < S) {
        const u32x4 cv = reinterpret_cast<const u32x4*>(a.samp)[sb + i];
        for (int g = 0; g < G; ++g)
          ham += __popc(cv.x ^ qc[4 * g]) + __popc(cv.y ^ qc[4 * g + 1]) +
                 __popc(cv.z ^ qc[4 * g + 2]) + __popc(cv.w ^ qc[4 * g + 3]);
      }
      key[e] = order_key_i32(128 * G - ham);
    }
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = t + e * NT;
      key[e] = i < S ? reinterpret_cast<const uint32_t*>(a.samp)[sb + i] : 0u;
    }
  }
  __syncthreads();  // tile becomes the histogram
  return rank_lower_bound_regs<NT, PER>(key, S, r, tile, sc);
}

// grid (B*Hkv): each head's candidate threshold and state.
template <int KIND, int LANES>
__global__ void __launch_bounds__(kScanNT)
threshold_kernel(const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_seq, FusedArgs a) {
  constexpr int NT = kScanNT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ BlockScratch<NT> sc;
  __shared__ uint32_t qc[64 * 4];
  float* tbl = reinterpret_cast<float*>(smem_raw);
  uint32_t* tile = reinterpret_cast<uint32_t*>(smem_raw + a.region_bytes);  // kSample words
  const int bh = blockIdx.x, b = bh / a.Hkv;
  const int t = threadIdx.x;
  if (KIND == kScanSoftFast || KIND == kScanSoftAny) {
    const int nflt = a.L << a.P;
    const float* src = a.tables + static_cast<long long>(bh) * nflt;
    if ((nflt & 3) == 0) {  // 16-byte loads, four in flight per thread
      const int nv = nflt / 4;
      for (int i0 = 0; i0 < nv; i0 += NT * 4) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (i0 + u * NT + t < nv) v[u] = reinterpret_cast<const u32x4*>(src)[i0 + u * NT + t];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (i0 + u * NT + t < nv) reinterpret_cast<u32x4*>(tbl)[i0 + u * NT + t] = v[u];
      }
    } else {
      for (int i = t; i < nflt; i += NT) tbl[i] = src[i];
    }
  }
  if (KIND == kScanHamming) {
    const int G = a.Hq / a.Hkv;
    for (int i = t; i < G * 4; i += NT) qc[i] = a.qcodes[static_cast<long long>(bh) * G * 4 + i];
  }
  __syncthreads();
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int k_eff = keff_of(a.kcap, k_per_seq, b, n);
  const uint32_t theta = sample_theta<KIND, LANES>(a, bh, n, k_eff, tbl, qc, tile, sc);
  if (t == 0) {
    HeadState* hs = a.heads + bh;
    hs->theta = theta;
    hs->k_eff = k_eff;
    hs->n = n;
  }
}

// Soft-LSH scan, L a multiple of 16.  grid (B*Hkv*nch), chunk-major per head.
template <int LANES, int U, bool FILTER>
__global__ void __launch_bounds__(kScanNT) __attribute__((amdgpu_waves_per_eu(8, 8)))  // two workgroups per CU
scan_softlsh_kernel(const uint8_t* __restrict__ ids, const void* __restrict__ vnorm, int norm_f16,
                    const int32_t* __restrict__ seq_lens, float* __restrict__ scores_out, int nch,
                    FusedArgs a) {
  constexpr int NT = kScanNT;
  using S = SoftScorer<LANES, NT, U>;
  constexpr int CH = kSoftChunk;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ BlockScratch<NT> sc;
  float* tbl = reinterpret_cast<float*>(smem_raw);                      // table region
  float* tile = reinterpret_cast<float*>(smem_raw + a.region_bytes);    // CH scores
  constexpr bool filt = FILTER;
  const int bh = blockIdx.x / nch, chunk = blockIdx.x % nch, b = bh / a.Hkv;
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int j0 = chunk * CH;
  if (j0 >= n) return;
  const int jend = min(j0 + CH, n);
  const long long base = static_cast<long long>(bh) * a.Nmax;
  S sco;
  sco.idv = reinterpret_cast<const uint4*>(ids);
  sco.vnorm = vnorm;
  sco.norm_f16 = norm_f16;
  sco.tbl = tbl;
  sco.idmask = (1u << a.P) - 1u;
  sco.setup();
  uint4 w[U];
  float nr[U];
  sco.load(w, nr, base, j0 + sco.grp, jend);  // first batch in flight during the table load
  {
    const int nflt = S::L << a.P;
    const float4* src = reinterpret_cast<const float4*>(a.tables + static_cast<long long>(bh) * nflt);
    for (int i = threadIdx.x; i < nflt / 4; i += NT) reinterpret_cast<float4*>(tbl)[i] = src[i];
  }
  const uint32_t theta = filt ? a.heads[bh].theta : 0u;
  __syncthreads();
  soft_score_range(sco, base, j0, jend, w, nr, tile);
  __syncthreads();
  uint2* slot = a.slots + static_cast<long long>(bh) * a.nchunks * CH + static_cast<long long>(chunk) * CH;
  const int count = scan_chunk_epilogue<NT, false>(reinterpret_cast<const uint32_t*>(tile), jend - j0, j0, base,
                                                   reinterpret_cast<uint32_t*>(scores_out), theta, filt,
                                                   slot, sc);
  if (filt && threadIdx.x == 0) a.counts[static_cast<long long>(bh) * a.nchunks + chunk] = count;
}

// One-lane-per-key scans: soft-LSH with any L, binary codes, given scores.
template <int KIND>
__global__ void __launch_bounds__(kScanNT)
scan_lane_kernel(const void* __restrict__ src, const void* __restrict__ vnorm, int norm_f16,
                 const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_seq,
                 uint32_t* __restrict__ scores_out, int filter, int nch, FusedArgs a) {
  constexpr int NT = kScanNT;
  constexpr bool KINT = KIND == kScanHamming || KIND == kScanGivenI32;
  constexpr int CH = kLaneChunk;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ BlockScratch<NT> sc;
  __shared__ uint32_t qc[64 * 4];
  float* tbl = reinterpret_cast<float*>(smem_raw);
  uint32_t* tile = reinterpret_cast<uint32_t*>(smem_raw + a.region_bytes);
  const bool filt = filter != 0;
  const int bh = blockIdx.x / nch, chunk = blockIdx.x % nch, b = bh / a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int j0 = chunk * CH;
  if (j0 >= n) return;
  const int jend = min(j0 + CH, n);
  const long long base = static_cast<long long>(bh) * a.Nmax;
  if (KIND == kScanSoftAny) {
    const int nflt = a.L << a.P;
    const float* s = a.tables + static_cast<long long>(bh) * nflt;
    for (int i = threadIdx.x; i < nflt; i += NT) tbl[i] = s[i];
  }
  if (KIND == kScanHamming)
    for (int i = threadIdx.x; i < G * 4; i += NT) qc[i] = a.qcodes[static_cast<long long>(bh) * G * 4 + i];
  const uint32_t theta = filt ? a.heads[bh].theta : 0u;
  __syncthreads();
  if (KIND == kScanSoftAny) {
    const uint32_t idmask = (1u << a.P) - 1u;
    for (int j = j0 + static_cast<int>(threadIdx.x); j < jend; j += NT) {
      const uint8_t* r = static_cast<const uint8_t*>(src) + (base + j) * a.L;
      float acc = 0.f;
      for (int l = 0; l < a.L; ++l) acc += tbl[(r[l] & idmask) * a.L + l];
      const float vn = norm_f16 ? f16_bits_to_f32(static_cast<const uint16_t*>(vnorm)[base + j])
                                : static_cast<const float*>(vnorm)[base + j];
      tile[j - j0] = __float_as_uint(acc * vn);
    }
  } else {
    // four keys per thread in flight
    for (int jb = j0 + static_cast<int>(threadIdx.x); jb < jend; jb += 4 * NT) {
      uint4 c[4];
      uint32_t gv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jb + u * NT;
        if (j < jend) {
          if (KIND == kScanHamming) c[u] = static_cast<const uint4*>(src)[base + j];
          else gv[u] = static_cast<const uint32_t*>(src)[base + j];
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = jb + u * NT;
        if (j >= jend) continue;
        if (KIND == kScanHamming) {
          int ham = 0;
          for (int g = 0; g < G; ++g)
            ham += __popc(c[u].x ^ qc[4 * g]) + __popc(c[u].y ^ qc[4 * g + 1]) +
                   __popc(c[u].z ^ qc[4 * g + 2]) + __popc(c[u].w ^ qc[4 * g + 3]);
          tile[j - j0] = static_cast<uint32_t>(128 * G - ham);
        } else {
          tile[j - j0] = gv[u];
        }
      }
    }
  }
  __syncthreads();
  uint2* slot = a.slots + static_cast<long long>(bh) * a.nchunks * CH + static_cast<long long>(chunk) * CH;
  const int count = scan_chunk_epilogue<NT, KINT>(tile, jend - j0, j0, base, scores_out, theta, filt,
                                                  slot, sc);
  if (filt && threadIdx.x == 0) a.counts[static_cast<long long>(bh) * a.nchunks + chunk] = count;
}

int scan_chunk(int L) {
  return (L == 16 || L == 32 || L == 64 || L == 128) ? kSoftChunk : kLaneChunk;
}

size_t scan_smem(int region, int chunk) { return static_cast<size_t>(region) + static_cast<size_t>(chunk) * 4; }

// Raises a kernel's dynamic LDS limit once per device (the largest size
// requested so far).
template <typename K>
static hipError_t lds_limit(K kern, size_t bytes) {
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

template <int LANES, bool FILTER>
static hipError_t launch_scan_soft_f(dim3 grid, const FusedArgs& a, const uint8_t* ids,
                                     const void* vnorm, int f16, const int32_t* sl, float* sout, int nch,
                                     hipStream_t st) {
  const size_t smem = scan_smem(a.region_bytes, kSoftChunk);
  auto kern = scan_softlsh_kernel<LANES, kScanSoftU, FILTER>;
  hipError_t e = lds_limit(kern, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kScanNT), smem, st, ids, vnorm, f16, sl, sout, nch, a);
  return hipGetLastError();
}

template <int LANES>
static hipError_t launch_scan_soft_t(dim3 grid, const FusedArgs& a, const uint8_t* ids,
                                     const void* vnorm, int f16, const int32_t* sl, float* sout,
                                     int filter, int nch, hipStream_t st) {
  return filter ? launch_scan_soft_f<LANES, true>(grid, a, ids, vnorm, f16, sl, sout, nch, st)
                : launch_scan_soft_f<LANES, false>(grid, a, ids, vnorm, f16, sl, sout, nch, st);
}

template <int KIND>
static hipError_t launch_scan_lane_t(dim3 grid, const FusedArgs& a, const void* src, const void* vnorm,
                                     int f16, const int32_t* sl, const int32_t* kps, void* sout,
                                     int filter, int nch, hipStream_t st) {
  const size_t smem = scan_smem(a.region_bytes, kLaneChunk);
  auto kern = scan_lane_kernel<KIND>;
  hipError_t e = lds_limit(kern, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kScanNT), smem, st, src, vnorm, f16, sl, kps,
                     static_cast<uint32_t*>(sout), filter, nch, a);
  return hipGetLastError();
}

template <int KIND, int LANES>
static hipError_t launch_threshold_t(const hst_shape& s, const FusedArgs& a, const int32_t* kps,
                                     hipStream_t st) {
  const size_t smem = static_cast<size_t>(a.region_bytes) + kSample * 4;
  auto kern = threshold_kernel<KIND, LANES>;
  hipError_t e = lds_limit(kern, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(s.B * s.Hkv), dim3(kScanNT), smem, st, s.seq_lens, kps, a);
  return hipGetLastError();
}

static hipError_t launch_threshold(const hst_shape& s, const FusedArgs& a, int kind, const int32_t* kps,
                                   hipStream_t st) {
  switch (kind) {
    case kScanSoftFast:
      switch (a.L) {
        case 16: return launch_threshold_t<kScanSoftFast, 1>(s, a, kps, st);
        case 32: return launch_threshold_t<kScanSoftFast, 2>(s, a, kps, st);
        case 64: return launch_threshold_t<kScanSoftFast, 4>(s, a, kps, st);
        default: return launch_threshold_t<kScanSoftFast, 8>(s, a, kps, st);
      }
    case kScanSoftAny: return launch_threshold_t<kScanSoftAny, 1>(s, a, kps, st);
    case kScanHamming: return launch_threshold_t<kScanHamming, 1>(s, a, kps, st);
    default: return launch_threshold_t<kScanGivenF32, 1>(s, a, kps, st);
  }
}

hipError_t launch_scan(const hst_shape& s, const FusedArgs& a_in, int kind, const void* src,
                       const void* vnorm, int norm_f16, void* scores_out, int filter,
                       const int32_t* kps, hipStream_t st) {
  const int chunk = kind == kScanSoftFast ? kSoftChunk : kLaneChunk;
  // LDS ahead of the chunk tile: the kv head's table (soft-LSH) or nothing
  FusedArgs a = a_in;
  a.region_bytes = (kind == kScanSoftFast || kind == kScanSoftAny)
                       ? static_cast<int>(hst_align16(static_cast<size_t>(a.L << a.P) * 4))
                       : 0;
  const int nch = static_cast<int>((s.Nmax + chunk - 1) / chunk);
  const long long BH = static_cast<long long>(s.B) * s.Hkv;
  const long long nblk = BH * nch;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(nblk));
  const uint8_t* ids = static_cast<const uint8_t*>(src);
  float* sout = static_cast<float*>(scores_out);
  const int32_t* sl = s.seq_lens;
  if (filter) {
    hipError_t e = launch_threshold(s, a, kind, kps, st);
    if (e != hipSuccess) return e;
  }
  switch (kind) {
    case kScanSoftFast:
      switch (a.L) {
        case 16: return launch_scan_soft_t<1>(grid, a, ids, vnorm, norm_f16, sl, sout, filter, nch, st);
        case 32: return launch_scan_soft_t<2>(grid, a, ids, vnorm, norm_f16, sl, sout, filter, nch, st);
        case 64: return launch_scan_soft_t<4>(grid, a, ids, vnorm, norm_f16, sl, sout, filter, nch, st);
        default: return launch_scan_soft_t<8>(grid, a, ids, vnorm, norm_f16, sl, sout, filter, nch, st);
      }
    case kScanSoftAny:
      return launch_scan_lane_t<kScanSoftAny>(grid, a, src, vnorm, norm_f16, sl, kps, scores_out, filter, nch, st);
    case kScanHamming:
      return launch_scan_lane_t<kScanHamming>(grid, a, src, nullptr, 0, sl, kps, scores_out, filter, nch, st);
    case kScanGivenF32:
      return launch_scan_lane_t<kScanGivenF32>(grid, a, src, nullptr, 0, sl, kps, nullptr, filter, nch, st);
    default:
      return launch_scan_lane_t<kScanGivenI32>(grid, a, src, nullptr, 0, sl, kps, nullptr, filter, nch, st);
  }
}

}  // namespace hst
