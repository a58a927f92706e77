// The key scan, the bandwidth-dominant stage of a decode step: every cached
// key's metadata is read from HBM exactly once, scored, and (when a top-k
// follows) appended to its chunk's candidate slots if it scores >= theta.
//  * Soft-collision score (SOCKET overview page, "Core mechanism: soft LSH",
//    item 3): score_j = ||v_j|| * sum_l T[id_{j,l}][l], the kv head's
//    bucket-major table T resident in LDS.  Each key's L ids are split over
//    L/16 lanes; lane groups visit their 16 tables in an order rotated (L = 64:
//    XOR-skewed) by the key's slot in the wave so the 64 lanes of a wave hit
//    distinct LDS banks.
//  * Code similarity (HATA explainer page, section 3): XOR + popcount of
//    128-bit codes against the G query codes.
//  * Given scores (the stand-alone top-k): the scores are only filtered.
//
// When filtering, B*Hkv extra workgroups (the first ones of the grid, which
// the dispatcher starts first) derive the heads' candidate thresholds from the
// partial sample scores prep wrote, while the others stream their chunks; a
// chunk workgroup waits for its head's threshold only before its epilogue.
// The threshold is handed over in one 64-bit atomic word (flag and value), so
// no other memory needs ordering.  Every wait is bounded: past the bound it
// falls back to threshold 0 (every key a candidate), which leaves the
// selection exact, so no dispatch order can stall the kernel.
#include <atomic>

#include "fused_device.h"
#include "hst_launch.h"

namespace hst {

constexpr int kScanNT = 1024;
constexpr int kSoftChunk = 2048;  // default keys per chunk (table lookups)
constexpr int kSoftCap = 2560;    // longest chunk: candidate slots per chunk, LDS score tile
constexpr int kLaneChunk = 4096;  // the same for one-lane-per-key scans
constexpr int kLaneCap = 5120;
static_assert(kSoftChunk >= kSample && kLaneChunk >= kSample && kSample >= 2048,
              "chunk tile holds the sample scores and doubles as the select histogram");
static_assert(kSoftCap >= kSoftChunk && kLaneCap >= kLaneChunk, "chunk caps");
// block scratch of a scan workgroup, after its table and score tile in LDS
template <int NT>
struct ScanTail {
  BlockScratch<NT> sc;
  uint32_t theta;
};
constexpr int kScanSoftU = 2;        // key batches per lane group in flight (two workgroups fit a CU)
constexpr int kThetaSpin = 1 << 16;  // polls of the threshold word before falling back
constexpr int kMaxParts = 16;        // partial sample scores per head (prep workgroups)

// LDS offset of an LDS-resident object, and a float read at an LDS byte
// address (no base to add).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<size_t>((const __attribute__((address_space(3))) char*)p));
}
__device__ __forceinline__ float lds_f32_at(uint32_t addr) {
  return *(const __attribute__((address_space(3))) float*)static_cast<size_t>(addr);
}

// Element i of a global array, loaded as a global (not flat) access also
// where the compiler cannot infer the pointer's address space.
template <typename T>
__device__ __forceinline__ T ld_global(const void* p, long long i) {
#if defined(__HIP_DEVICE_COMPILE__)
  return ((const __attribute__((address_space(1))) T*)p)[i];
#else
  return static_cast<const T*>(p)[i];
#endif
}

// F16: value norms stored as binary16 (else float32); the raw bits are loaded
// and converted only when used, so a load never waits for its own result.
template <int LANES, int NT, int U, bool F16>
struct SoftScorer {
  static constexpr int L = 16 * LANES;
  static constexpr int KPI = NT / LANES;  // keys per batch
  static constexpr int TILE = KPI * U;
  const uint4* idv;
  const void* vnorm;
  const float* tbl;  // LDS
  uint32_t idmask;   // 2^P - 1: ids outside the table cannot leave it
  int sub, grp;
  // L = 64 (LANES == 4): lookup i of a lane reads table 16*sub + (i ^ k), k
  // the key's slot among the 16 keys of its wave, so the 64 lanes of a wave
  // hit 64 distinct banks.  Entry (id, l) of the bucket-major table sits at
  // byte id*256 + 4l: the address is the id byte over the byte 4l, one byte
  // permutation (v_perm) of the lane's id word and a word of four 4l bytes.
  uint32_t lc[4];   // byte b of lc[m]: 4 * (16*sub + ((4m + b) ^ k))
  uint32_t sel[4];  // permutation of lookup i (by i & 3): byte 0 <- lc byte, byte 1 <- id byte, 0, 0
  uint32_t idm4;    // idmask in every byte
  bool x1, x2;      // the lane's id words are taken XOR-permuted by (k >> 2)
  bool at0;         // the table starts at LDS address 0: a permuted address is the LDS address

  __device__ __forceinline__ void setup() {
    sub = threadIdx.x % LANES;
    grp = threadIdx.x / LANES;
    if constexpr (LANES == 4) {
      const int k = grp & 15;
      x1 = ((k >> 2) & 1) != 0;
      x2 = ((k >> 3) & 1) != 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t v = 0u;
#pragma unroll
        for (int b = 0; b < 4; ++b) v |= static_cast<uint32_t>((sub * 16 + ((4 * m + b) ^ k)) * 4) << (8 * b);
        lc[m] = v;
      }
#pragma unroll
      for (int b = 0; b < 4; ++b)
        sel[b] = static_cast<uint32_t>(b) | (static_cast<uint32_t>(4 + (b ^ (k & 3))) << 8) | 0x0c0c0000u;
      idm4 = idmask * 0x01010101u;
      at0 = lds_offset(tbl) == 0u;
    }
  }
  // Loads of a batch; keys past jend (>= 1) read key jend - 1 instead, so the
  // loads carry no branch and all are in flight together.
  __device__ __forceinline__ void load(uint4 (&w)[U], uint32_t (&nr)[U], long long base, int jb,
                                       int jend) const {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j0 = jb + u * KPI;
      const long long j = base + (j0 < jend ? j0 : jend - 1);
      w[u] = ld_global<uint4>(idv, j * LANES + sub);
      nr[u] = F16 ? static_cast<uint32_t>(ld_global<uint16_t>(vnorm, j)) : ld_global<uint32_t>(vnorm, j);
    }
  }
  // scores of the batch held in (w, nr) into out[j - j0]
  __device__ __forceinline__ void compute(const uint4 (&w)[U], const uint32_t (&nr)[U], int jb, int jend,
                                          int j0, float* out) const {
    if constexpr (LANES == 4) {
      if (at0) compute64<true>(w, nr, jb, jend, j0, out);
      else compute64<false>(w, nr, jb, jend, j0, out);
      return;
    }
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
        const float vn = F16 ? f16_bits_to_f32(static_cast<uint16_t>(nr[u])) : __uint_as_float(nr[u]);
        const float sv = group_sum<LANES>(acc0 + acc1) * vn;
        if (sub == 0) out[j - j0] = sv;
      }
    }
  }
  template <bool AT0>
  __device__ __forceinline__ void compute64(const uint4 (&w)[U], const uint32_t (&nr)[U], int jb, int jend,
                                            int j0, float* out) const {
    const char* tb = reinterpret_cast<const char*>(tbl);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jb + u * KPI;
      if (j < jend) {  // uniform over the LANES lanes of a key
        // id words in the order (m ^ (k >> 2)), ids clamped into the table
        const uint32_t e0 = x1 ? w[u].y : w[u].x, e1 = x1 ? w[u].x : w[u].y;
        const uint32_t e2 = x1 ? w[u].w : w[u].z, e3 = x1 ? w[u].z : w[u].w;
        uint32_t d[4];
        d[0] = (x2 ? e2 : e0) & idm4;
        d[1] = (x2 ? e3 : e1) & idm4;
        d[2] = (x2 ? e0 : e2) & idm4;
        d[3] = (x2 ? e1 : e3) & idm4;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const uint32_t o0 = __builtin_amdgcn_perm(d[i >> 2], lc[i >> 2], sel[i & 3]);
          const uint32_t o1 = __builtin_amdgcn_perm(d[(i + 1) >> 2], lc[(i + 1) >> 2], sel[(i + 1) & 3]);
          acc0 += AT0 ? lds_f32_at(o0) : *reinterpret_cast<const float*>(tb + o0);
          acc1 += AT0 ? lds_f32_at(o1) : *reinterpret_cast<const float*>(tb + o1);
        }
        const float vn = F16 ? f16_bits_to_f32(static_cast<uint16_t>(nr[u])) : __uint_as_float(nr[u]);
        const float sv = group_sum<LANES>(acc0 + acc1) * vn;
        if (sub == 0) out[j - j0] = sv;
      }
    }
  }
};

// Scores of keys [j0, min(jend, j0 + NTILES * TILE)) into out[j - j0];
// (wa, na) hold the first batch, already loaded.  Two register sets
// alternate, so the next batch is in flight during each batch's table
// lookups without register copies (a copy, or a loop back edge, would make
// the compiler wait for the loads first): the tile loop is unrolled and every
// load is unconditional, only the lookups are skipped past jend.
template <int NTILES, class S, int U>
__device__ __forceinline__ void soft_score_tiles(const S& sco, long long base, int j0, int jend,
                                                 uint4 (&wa)[U], uint32_t (&na)[U], float* out) {
  uint4 wb[U];
  uint32_t nb[U];
#pragma unroll
  for (int it = 0; it < NTILES; it += 2) {
    const int t0 = j0 + it * S::TILE, t1 = t0 + S::TILE;
    if (it + 1 < NTILES) sco.load(wb, nb, base, t1 + sco.grp, jend);
    if (t0 < jend) sco.compute(wa, na, t0 + sco.grp, jend, j0, out);
    if (it + 2 < NTILES) sco.load(wa, na, base, t1 + S::TILE + sco.grp, jend);
    if (it + 1 < NTILES && t1 < jend) sco.compute(wb, nb, t1 + sco.grp, jend, j0, out);
  }
}

// The same with the first two batches already loaded, (wa, na) and (wb, nb):
// each set is reloaded right after its lookups, so one batch stays in flight
// during each batch's lookups as above.  late() runs once, before the
// lookups of tile NTILES - 2 (or of the only tile).
template <int NTILES, class S, int U, class F>
__device__ __forceinline__ void soft_score_tiles2(const S& sco, long long base, int j0, int jend,
                                                  uint4 (&wa)[U], uint32_t (&na)[U], uint4 (&wb)[U],
                                                  uint32_t (&nb)[U], float* out, F&& late) {
  constexpr int kLate = NTILES >= 2 ? NTILES - 2 : 0;
#pragma unroll
  for (int it = 0; it < NTILES; it += 2) {
    const int t0 = j0 + it * S::TILE, t1 = t0 + S::TILE;
    if (it == kLate) late();
    if (t0 < jend) sco.compute(wa, na, t0 + sco.grp, jend, j0, out);
    if (it + 2 < NTILES) sco.load(wa, na, base, t1 + S::TILE + sco.grp, jend);
    if (it + 1 == kLate) late();
    if (it + 1 < NTILES && t1 < jend) sco.compute(wb, nb, t1 + sco.grp, jend, j0, out);
    if (it + 3 < NTILES) sco.load(wb, nb, base, t1 + 2 * S::TILE + sco.grp, jend);
  }
}

// Table copy of exactly NT * 4 vectors: its loads, then the loads of the
// scorer's second batch, then the LDS stores and a barrier that orders LDS
// only.  The stores wait for the table's loads alone (the memory counter
// counts loads in issue order), and the barrier does not wait for the
// batch, which is still in flight when the lookups start.
template <int NT, class S, int U>
__device__ __forceinline__ void copy_table_then_load(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                     const S& sco, uint4 (&wb)[U], uint32_t (&nb)[U],
                                                     long long base, int jb, int jend) {
  u32x4 v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = src[u * NT + threadIdx.x];
  sco.load(wb, nb, base, jb, jend);
  asm volatile("" ::: "memory");  // the loads above stay ahead of the stores
#pragma unroll
  for (int u = 0; u < 4; ++u) dst[u * NT + threadIdx.x] = v[u];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The chunk's scores sit in LDS (tile[0..cnt)): write them out (coalesced)
// when a score row is asked for, and append the keys scoring >= theta, in
// index order, to the chunk's candidate slots.  Returns the candidate count
// (every thread).
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


// Work of a scan workgroup: a chunk of one head, or (filtering) the
// threshold of one head.  Filtering grids start with theta_groups(BH)
// threshold workgroups (those past BH have no work); the chunks of one head
// then run on one XCD (xcd_item), which fetches the head's table once.
struct ScanWork {
  int bh, chunk;
  bool theta, none;
};
__device__ __forceinline__ ScanWork scan_work(bool filt, int BH, int nch) {
  const int lid = blockIdx.x;
  const int nth = filt ? static_cast<int>(theta_groups(BH)) : 0;
  ScanWork w;
  w.theta = lid < nth;
  w.none = w.theta && lid >= BH;
  const int x = w.theta ? 0 : xcd_item(lid - nth, BH * nch);
  w.bh = w.theta ? lid : x / nch;
  w.chunk = w.theta ? 0 : x % nch;
  return w;
}

// Candidate threshold of head bh: the sample scores are the sums of the
// parts prep wrote (times the sampled key's value norm, read from a.meta_vn,
// for soft-LSH), and theta is
// a lower bound of the sample score at a high-margin rank.  The bin width of
// the selection's candidate histogram (shift) spreads [theta, the sample's
// largest key] over half the bins.  Every thread of the workgroup calls;
// tile: kSample words of LDS scratch.
template <int KIND>
__device__ uint32_t sample_theta(const FusedArgs& a, int bh, int n, int k_eff, uint32_t* tile,
                                 BlockScratch<kScanNT>& sc, int& shift) {
  constexpr int NT = kScanNT;
  constexpr int PER = kSample / NT;
  const int S = a.sample > n ? n : a.sample;
  const int r = sample_rank(k_eff, n, S);
  shift = 21;  // no usable sample: every key is a candidate, bins of 2^21 keys
  if (!(S > 0 && k_eff > 0 && r < S)) return 0u;
  const int t = threadIdx.x;
  const float* part = a.spart + static_cast<long long>(bh) * a.xparts * kSample;
  const int X = a.xparts;
  uint32_t key[PER];
  if (KIND == kScanGivenF32 || KIND == kScanGivenI32) {
#pragma unroll
    for (int e = 0; e < PER; ++e) key[e] = __float_as_uint(part[t + e * NT]);  // order keys' bits
  } else {
    // every part of both keys in flight together (indices clamped to the parts
    // that exist; entries past S are ignored by the rank)
    float pv[PER][kMaxParts];
#pragma unroll
    for (int e = 0; e < PER; ++e)
#pragma unroll
      for (int x = 0; x < kMaxParts; ++x) pv[e][x] = part[(x < X ? x : X - 1) * kSample + t + e * NT];
    // soft-LSH: the sampled keys' value norms, read at their positions
    // (issued with the parts; this workgroup starts before the chunk
    // workgroups' key stream)
    float vn[PER];
    if (KIND != kScanHamming) {
      uint32_t vb[PER];
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int i = t + e * NT;
        const long long row = static_cast<long long>(bh) * a.Nmax + sample_pos(i < S ? i : S - 1, S, n);
        vb[e] = a.meta_f16 ? static_cast<uint32_t>(static_cast<const uint16_t*>(a.meta_vn)[row])
                           : static_cast<const uint32_t*>(a.meta_vn)[row];
      }
#pragma unroll
      for (int e = 0; e < PER; ++e)
        vn[e] = a.meta_f16 ? f16_bits_to_f32(static_cast<uint16_t>(vb[e])) : __uint_as_float(vb[e]);
    }
    const int G = a.Hq / a.Hkv;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int x = 0; x < kMaxParts; ++x)
        if (x < X) acc += pv[e][x];
      key[e] = KIND == kScanHamming ? order_key_i32(128 * G - static_cast<int>(acc))
                                    : order_key_f32(acc * vn[e]);
    }
  }
  uint32_t kmax = 0u;
  const uint32_t theta = rank_lower_bound_regs<NT, PER>(key, S, r, tile, sc, &kmax);
  shift = hist_shift(theta, kmax);
  return theta;
}

// Threshold workgroup: derive and publish head bh's threshold and state.
template <int KIND>
__device__ void theta_publish(const FusedArgs& a, int bh, const int32_t* seq_lens, const int32_t* k_per_seq,
                              uint32_t* tile, BlockScratch<kScanNT>& sc) {
  const int b = bh / a.Hkv;
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int k_eff = keff_of(a.kcap, k_per_seq, b, n);
  int shift;
  const uint32_t theta = sample_theta<KIND>(a, bh, n, k_eff, tile, sc, shift);
  if (threadIdx.x == 0) {
    HeadState* hs = a.heads + bh;
    hs->theta = theta;
    hs->k_eff = k_eff;
    hs->n = n;
    hs->shift = static_cast<uint32_t>(shift);
    __hip_atomic_store(&hs->thr_word, (1ull << 32) | theta, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Chunk workgroup: the head's threshold, once published (see above).  Past
// the bounded wait the chunk filters with threshold 0 (every key a
// candidate), which leaves the selection exact.
// pre: the threshold word as thread 0 read it earlier (0 if not read).
__device__ __forceinline__ uint32_t theta_wait(const FusedArgs& a, int bh, ScanTail<kScanNT>& tl,
                                               uint64_t pre = 0) {
  if (threadIdx.x == 0) {
    uint64_t v = pre;
    for (int i = 0; (v >> 32) == 0 && i < kThetaSpin; ++i) {
      v = __hip_atomic_load(&a.heads[bh].thr_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (v >> 32) break;
      __builtin_amdgcn_s_sleep(4);
    }
    tl.theta = (v >> 32) ? static_cast<uint32_t>(v) : 0u;
  }
  __syncthreads();
  return tl.theta;
}

// Soft-LSH scan, L a multiple of 16.  grid (B*Hkv*nch [+ B*Hkv when filtering]);
// chunk c of a head holds keys [c*span, (c+1)*span), span at most the default
// chunk length (LONG false) or kSoftCap (LONG true).
template <int LANES, int U, bool FILTER, bool F16, bool LONG, bool FULL>
__global__ void __launch_bounds__(kScanNT) __attribute__((amdgpu_waves_per_eu(8, 8)))  // two workgroups per CU
scan_softlsh_kernel(const uint8_t* __restrict__ ids, const void* __restrict__ vnorm,
                    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_seq,
                    float* __restrict__ scores_out, int nch, FusedArgs a) {
  constexpr int NT = kScanNT;
  using S = SoftScorer<LANES, NT, U, F16>;
  static_assert(kSoftChunk % S::TILE == 0, "whole tiles per default chunk");
  constexpr int NTILES = LONG ? (kSoftCap + S::TILE - 1) / S::TILE : kSoftChunk / S::TILE;
  // no static LDS: the table starts at LDS address 0, so a lookup's address
  // is the byte permutation alone
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* tbl = reinterpret_cast<float*>(smem_raw);                      // table region
  float* tile = reinterpret_cast<float*>(smem_raw + a.region_bytes);    // the chunk's scores
  ScanTail<NT>& tl = *reinterpret_cast<ScanTail<NT>*>(smem_raw + a.region_bytes + kSoftCap * 4);
  BlockScratch<NT>& sc = tl.sc;
  constexpr bool filt = FILTER;
  const ScanWork wk = scan_work(filt, a.nbh, nch);
  if (wk.none) return;
  if (filt && wk.theta) {
    theta_publish<kScanSoftFast>(a, wk.bh, seq_lens, k_per_seq, reinterpret_cast<uint32_t*>(tile), sc);
    return;
  }
  const int bh = wk.bh, chunk = wk.chunk, b = bh / a.Hkv;
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int j0 = chunk * a.span;
  if (j0 >= n) return;
  const int jend = min(j0 + a.span, n);
  const long long base = static_cast<long long>(bh) * a.Nmax;
  S sco;
  sco.idv = reinterpret_cast<const uint4*>(ids);
  sco.vnorm = vnorm;
  sco.tbl = tbl;
  sco.idmask = (1u << a.P) - 1u;
  sco.setup();
  uint4 w[U];
  uint32_t nr[U];
  uint64_t thv = 0;  // the threshold word, when read ahead
  const int nflt = S::L << a.P;               // a multiple of 16: L is
  const u32x4* tsrc = reinterpret_cast<const u32x4*>(a.tables + static_cast<long long>(bh) * nflt);
  if constexpr (FULL && NTILES >= 2) {  // a full table (L = 64, P = 8): two batches in flight during its copy
    // The metadata arguments are read-only and unaliased, so their loads
    // count as invariant and the compiler may sink them past the barrier to
    // their first use; pointers it cannot see through keep them where issued.
    asm volatile("" : "+s"(sco.idv), "+s"(sco.vnorm));
    uint4 w2[U];
    uint32_t nr2[U];
    sco.load(w, nr, base, j0 + sco.grp, jend);
    copy_table_then_load<NT>(reinterpret_cast<u32x4*>(tbl), tsrc, sco, w2, nr2, base, j0 + S::TILE + sco.grp,
                             jend);
    // thread 0 reads the threshold word before the last full tile: a chunk
    // that finishes late then finds theta without another round trip
    soft_score_tiles2<NTILES>(sco, base, j0, jend, w, nr, w2, nr2, tile, [&] {
      if (filt && threadIdx.x == 0)
        thv = __hip_atomic_load(&a.heads[bh].thr_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    });
  } else {
    sco.load(w, nr, base, j0 + sco.grp, jend);  // first batch in flight during the table load
    copy_to_lds<NT, 4>(reinterpret_cast<u32x4*>(tbl), tsrc, nflt / 4);
    __syncthreads();
    soft_score_tiles<NTILES>(sco, base, j0, jend, w, nr, tile);
  }
  __syncthreads();
  const uint32_t theta = filt ? theta_wait(a, bh, tl, thv) : 0u;
  uint2* slot = a.slots + (static_cast<long long>(bh) * a.nchunks + chunk) * kSoftCap;
  const int count = scan_chunk_epilogue<NT, false>(reinterpret_cast<const uint32_t*>(tile), jend - j0, j0, base,
                                                   reinterpret_cast<uint32_t*>(scores_out), theta, filt,
                                                   slot, sc);
  HST_DCHECK(count <= kSoftCap, kDbgChunkCount);
  if (filt && threadIdx.x == 0) a.counts[static_cast<long long>(bh) * a.nchunks + chunk] = count;
}

// Soft-LSH scan of a batch that shares a prefix (scores only).  The
// context of sequence b is the Np prefix keys (metadata [Hkv][Np], one copy)
// then its own suffix (metadata [B*Hkv][Ns]); scores of (b, h) go to row
// bh of `scores_out` (pitch Np + Ns): prefix key j at j, suffix key j at
// Np + j.  1-D grid: prefix chunks first, B workgroups per (kv head, chunk)
// with block ids congruent modulo 8 and within 8*B consecutive ids, so they
// run on one XCD at about the same time and the prefix metadata is fetched
// from HBM once; then B*Hkv*nchs suffix chunks.
template <int LANES, int U, bool F16>
__global__ void __launch_bounds__(kScanNT) __attribute__((amdgpu_waves_per_eu(8, 8)))
scan_shared_kernel(const uint8_t* __restrict__ ids_p, const void* __restrict__ vn_p, int Np,
                   const uint8_t* __restrict__ ids_s, const void* __restrict__ vn_s,
                   const int32_t* __restrict__ s_lens, int Ns, int B, int nchp, int pitems_pad,
                   int nchs, float* __restrict__ scores_out, FusedArgs a) {
  constexpr int NT = kScanNT;
  using S = SoftScorer<LANES, NT, U, F16>;
  constexpr int CH = kSoftChunk;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* tbl = reinterpret_cast<float*>(smem_raw);
  float* tile = reinterpret_cast<float*>(smem_raw + a.region_bytes);
  BlockScratch<NT>& sc = reinterpret_cast<ScanTail<NT>*>(smem_raw + a.region_bytes + kSoftCap * 4)->sc;
  const int w = blockIdx.x, Hkv = a.Hkv;
  const int npre = pitems_pad * B;
  int b, h, chunk;
  bool pre;
  if (w < npre) {
    const int grp = w / (8 * B), rem = w % (8 * B);
    b = rem / 8;
    const int item = grp * 8 + rem % 8;
    if (item >= Hkv * nchp) return;  // padding of the last group
    h = item / nchp;
    chunk = item % nchp;
    pre = true;
  } else {
    const int v = w - npre, bhv = v / nchs;
    chunk = v % nchs;
    b = bhv / Hkv;
    h = bhv % Hkv;
    pre = false;
  }
  const int bh = b * Hkv + h;
  const int n = pre ? Np : seq_len(s_lens, b, Ns);
  const int j0 = chunk * CH;
  if (j0 >= n) return;
  const int jend = min(j0 + CH, n);
  const long long mbase = pre ? static_cast<long long>(h) * Np : static_cast<long long>(bh) * Ns;
  S sco;
  sco.idv = reinterpret_cast<const uint4*>(pre ? ids_p : ids_s);
  sco.vnorm = pre ? vn_p : vn_s;
  sco.tbl = tbl;
  sco.idmask = (1u << a.P) - 1u;
  sco.setup();
  uint4 wv[U];
  uint32_t nr[U];
  sco.load(wv, nr, mbase, j0 + sco.grp, jend);
  {
    const int nflt = S::L << a.P;
    copy_to_lds<NT, 4>(reinterpret_cast<u32x4*>(tbl),
                       reinterpret_cast<const u32x4*>(a.tables + static_cast<long long>(bh) * nflt), nflt / 4);
  }
  __syncthreads();
  soft_score_tiles<CH / S::TILE>(sco, mbase, j0, jend, wv, nr, tile);
  __syncthreads();
  const long long obase = static_cast<long long>(bh) * (Np + Ns) + (pre ? 0 : Np);
  scan_chunk_epilogue<NT, false>(reinterpret_cast<const uint32_t*>(tile), jend - j0, j0, obase,
                                 reinterpret_cast<uint32_t*>(scores_out), 0u, false, nullptr, sc);
}

// One-lane-per-key scans: soft-LSH with any L, binary codes, given scores.
template <int KIND>
__global__ void __launch_bounds__(kScanNT)
scan_lane_kernel(const void* __restrict__ src, const void* __restrict__ vnorm, int norm_f16,
                 const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_seq,
                 uint32_t* __restrict__ scores_out, int filter, int nch, FusedArgs a) {
  constexpr int NT = kScanNT;
  constexpr bool KINT = KIND == kScanHamming || KIND == kScanGivenI32;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  __shared__ ScanTail<NT> tl;
  BlockScratch<NT>& sc = tl.sc;
  __shared__ uint32_t qc[64 * 4];
  float* tbl = reinterpret_cast<float*>(smem_raw);
  uint32_t* tile = reinterpret_cast<uint32_t*>(smem_raw + a.region_bytes);
  const bool filt = filter != 0;
  const ScanWork wk = scan_work(filt, a.nbh, nch);
  if (wk.none) return;
  if (filt && wk.theta) {
    theta_publish<KIND>(a, wk.bh, seq_lens, k_per_seq, tile, sc);
    return;
  }
  const int bh = wk.bh, chunk = wk.chunk, b = bh / a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int n = seq_len(seq_lens, b, a.Nmax);
  const int j0 = chunk * a.span;
  if (j0 >= n) return;
  const int jend = min(j0 + a.span, n);
  const long long base = static_cast<long long>(bh) * a.Nmax;
  // codes / given scores: the first four keys of each thread are loaded
  // before the query codes, so both arrive in one round trip
  uint4 c[4];
  uint32_t gv[4];
  const auto load4 = [&](int jb) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = jb + u * NT;
      if (j < jend) {
        if (KIND == kScanHamming) c[u] = static_cast<const uint4*>(src)[base + j];
        else gv[u] = static_cast<const uint32_t*>(src)[base + j];
      }
    }
  };
  const int jfirst = j0 + static_cast<int>(threadIdx.x);
  if (KIND != kScanSoftAny) load4(jfirst);
  // the threshold word, read ahead: workgroups that start after the
  // threshold workgroups have published it skip the epilogue's round trip
  uint64_t thv = 0;
  if (filt && threadIdx.x == 0)
    thv = __hip_atomic_load(&a.heads[bh].thr_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (KIND == kScanSoftAny) {
    const int nflt = a.L << a.P;
    const float* s = a.tables + static_cast<long long>(bh) * nflt;
    for (int i = threadIdx.x; i < nflt; i += NT) tbl[i] = s[i];
  }
  if (KIND == kScanHamming)
    for (int i = threadIdx.x; i < G * 4; i += NT) qc[i] = a.qcodes[static_cast<long long>(bh) * G * 4 + i];
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
    // four keys per thread in flight (the first four already loaded)
    for (int jb = jfirst; jb < jend; jb += 4 * NT) {
      if (jb != jfirst) load4(jb);
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
  const uint32_t theta = filt ? theta_wait(a, bh, tl, thv) : 0u;
  uint2* slot = a.slots + (static_cast<long long>(bh) * a.nchunks + chunk) * kLaneCap;
  const int count = scan_chunk_epilogue<NT, KINT>(tile, jend - j0, j0, base, scores_out, theta, filt,
                                                  slot, sc);
  if (filt && threadIdx.x == 0) a.counts[static_cast<long long>(bh) * a.nchunks + chunk] = count;
}

int scan_chunk(int L) {
  return (L == 16 || L == 32 || L == 64 || L == 128) ? kSoftChunk : kLaneChunk;
}

int scan_cap(int L) {
  return (L == 16 || L == 32 || L == 64 || L == 128) ? kSoftCap : kLaneCap;
}

// Scan workgroups resident at once on the current device: two 1024-thread
// workgroups per CU.  The count is cached per device in an atomic: threads
// that race on the first call all store the same value.
static int resident_scan_groups() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 512;
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    v = 2 * cus;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// A filtering scan runs B*Hkv*nch chunk workgroups plus B*Hkv threshold
// workgroups.  When the threshold workgroups add a round of resident
// workgroups that the chunks alone would not need, the chunks left over for
// it start only once earlier workgroups finish and end the kernel late.
// Lengthening the chunks (up to the slot capacity) so that the chunks and
// thresholds fit the chunks' own rounds removes that tail.
int scan_span(const hst_shape& s, int chunk, int cap, bool filter) {
  const long long BH = static_cast<long long>(s.B) * s.Hkv;
  const long long N = s.Nmax;
  if (!filter || BH <= 0 || N <= 0) return chunk;
  const long long R0 = resident_scan_groups();
  const long long nch0 = (N + chunk - 1) / chunk;
  const long long r_chunks = (BH * nch0 + R0 - 1) / R0;        // rounds of the chunks alone
  const long long TH = theta_groups(BH);
  const long long r_all = (BH * nch0 + TH + R0 - 1) / R0;      // with the threshold workgroups
  if (r_all == r_chunks) return chunk;
  const long long nch = (r_chunks * R0 - TH) / BH;
  if (nch < 1) return chunk;
  const long long span = ((N + nch - 1) / nch + 63) / 64 * 64;
  return span <= cap ? static_cast<int>(span) : chunk;
}

size_t scan_smem(int region, int chunk) {
  return static_cast<size_t>(region) + static_cast<size_t>(chunk) * 4 + hst_align16(sizeof(ScanTail<kScanNT>));
}

// Raises a kernel's dynamic LDS limit (kept per kernel and device).
template <typename K>
static hipError_t lds_limit(K kern, size_t bytes) {
  return raise_lds_limit(reinterpret_cast<const void*>(kern), bytes);
}

template <int LANES, bool FILTER, bool F16>
static hipError_t launch_scan_soft_f(dim3 grid, const FusedArgs& a, const uint8_t* ids,
                                     const void* vnorm, const int32_t* sl, const int32_t* kps,
                                     float* sout, int nch, hipStream_t st) {
  const size_t smem = scan_smem(a.region_bytes, kSoftCap);
  // chunks up to the default length take the default tile count
  auto kern = a.span > kSoftChunk ? scan_softlsh_kernel<LANES, kScanSoftU, FILTER, F16, true, false>
                                  : scan_softlsh_kernel<LANES, kScanSoftU, FILTER, F16, false, false>;
  if constexpr (LANES == 4)
    if (a.P == 8)  // the full table: 16 * kScanNT vectors
      kern = a.span > kSoftChunk ? scan_softlsh_kernel<LANES, kScanSoftU, FILTER, F16, true, true>
                                 : scan_softlsh_kernel<LANES, kScanSoftU, FILTER, F16, false, true>;
  hipError_t e = lds_limit(kern, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kScanNT), smem, st, ids, vnorm, sl, kps, sout, nch, a);
  return hipGetLastError();
}

template <int LANES>
static hipError_t launch_scan_soft_t(dim3 grid, const FusedArgs& a, const uint8_t* ids,
                                     const void* vnorm, int f16, const int32_t* sl, const int32_t* kps,
                                     float* sout, int filter, int nch, hipStream_t st) {
  if (filter)
    return f16 ? launch_scan_soft_f<LANES, true, true>(grid, a, ids, vnorm, sl, kps, sout, nch, st)
               : launch_scan_soft_f<LANES, true, false>(grid, a, ids, vnorm, sl, kps, sout, nch, st);
  return f16 ? launch_scan_soft_f<LANES, false, true>(grid, a, ids, vnorm, sl, kps, sout, nch, st)
             : launch_scan_soft_f<LANES, false, false>(grid, a, ids, vnorm, sl, kps, sout, nch, st);
}

template <int KIND>
static hipError_t launch_scan_lane_t(dim3 grid, const FusedArgs& a, const void* src, const void* vnorm,
                                     int f16, const int32_t* sl, const int32_t* kps, void* sout,
                                     int filter, int nch, hipStream_t st) {
  const size_t smem = scan_smem(a.region_bytes, kLaneCap);
  auto kern = scan_lane_kernel<KIND>;
  hipError_t e = lds_limit(kern, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kScanNT), smem, st, src, vnorm, f16, sl, kps,
                     static_cast<uint32_t*>(sout), filter, nch, a);
  return hipGetLastError();
}

hipError_t launch_scan(const hst_shape& s, const FusedArgs& a_in, int kind, const void* src,
                       const void* vnorm, int norm_f16, void* scores_out, int filter,
                       const int32_t* kps, hipStream_t st) {
  // LDS ahead of the chunk tile: the kv head's table (soft-LSH) or nothing
  FusedArgs a = a_in;
  const int chunk = a.span;
  if (chunk < 1 || chunk > (kind == kScanSoftFast ? kSoftCap : kLaneCap)) return hipErrorInvalidValue;
  a.region_bytes = (kind == kScanSoftFast || kind == kScanSoftAny)
                       ? static_cast<int>(hst_align16(static_cast<size_t>(a.L << a.P) * 4))
                       : 0;
  const int nch = static_cast<int>((s.Nmax + chunk - 1) / chunk);
  const long long BH = static_cast<long long>(s.B) * s.Hkv;
  const long long nblk = BH * nch + (filter ? theta_groups(BH) : 0);
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  dim3 grid(static_cast<unsigned>(nblk));
  const uint8_t* ids = static_cast<const uint8_t*>(src);
  float* sout = static_cast<float*>(scores_out);
  const int32_t* sl = s.seq_lens;
  if (kind == kScanSoftFast || kind == kScanSoftAny) {  // the threshold reads the sampled norms
    a.meta_vn = vnorm;
    a.meta_f16 = norm_f16;
  }
  switch (kind) {
    case kScanSoftFast:
      switch (a.L) {
        case 16: return launch_scan_soft_t<1>(grid, a, ids, vnorm, norm_f16, sl, kps, sout, filter, nch, st);
        case 32: return launch_scan_soft_t<2>(grid, a, ids, vnorm, norm_f16, sl, kps, sout, filter, nch, st);
        case 64: return launch_scan_soft_t<4>(grid, a, ids, vnorm, norm_f16, sl, kps, sout, filter, nch, st);
        default: return launch_scan_soft_t<8>(grid, a, ids, vnorm, norm_f16, sl, kps, sout, filter, nch, st);
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

template <int LANES, bool F16>
static hipError_t launch_scan_shared_t(dim3 grid, const FusedArgs& a, const uint8_t* ids_p,
                                       const void* vn_p, int Np, const uint8_t* ids_s,
                                       const void* vn_s, const int32_t* sl, int Ns, int B,
                                       int nchp, int pitems_pad, int nchs, float* sout,
                                       hipStream_t st) {
  const size_t smem = scan_smem(a.region_bytes, kSoftCap);  // the scratch sits past a longest tile
  auto kern = scan_shared_kernel<LANES, kScanSoftU, F16>;
  hipError_t e = lds_limit(kern, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(kScanNT), smem, st, ids_p, vn_p, Np, ids_s, vn_s, sl, Ns, B,
                     nchp, pitems_pad, nchs, sout, a);
  return hipGetLastError();
}

hipError_t launch_scan_shared(const hst_shape& s, const FusedArgs& a_in, int Np,
                              const uint8_t* ids_p, const void* vn_p, const uint8_t* ids_s,
                              const void* vn_s, int norm_f16, float* scores_out, hipStream_t st) {
  FusedArgs a = a_in;
  a.region_bytes = static_cast<int>(hst_align16(static_cast<size_t>(a.L << a.P) * 4));
  const int nchp = (Np + kSoftChunk - 1) / kSoftChunk;
  const int nchs = (s.Nmax + kSoftChunk - 1) / kSoftChunk;
  const int pitems_pad = (s.Hkv * nchp + 7) / 8 * 8;
  const long long nblk = static_cast<long long>(pitems_pad) * s.B +
                         static_cast<long long>(s.B) * s.Hkv * nchs;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<unsigned>(nblk));
#define HST_SSH(LN)                                                                           \
  return norm_f16 ? launch_scan_shared_t<LN, true>(grid, a, ids_p, vn_p, Np, ids_s, vn_s,     \
                                                  s.seq_lens, s.Nmax, s.B, nchp, pitems_pad, \
                                                  nchs, scores_out, st)                      \
                  : launch_scan_shared_t<LN, false>(grid, a, ids_p, vn_p, Np, ids_s, vn_s,    \
                                                   s.seq_lens, s.Nmax, s.B, nchp,            \
                                                   pitems_pad, nchs, scores_out, st)
  switch (a.L) {
    case 16: HST_SSH(1);
    case 32: HST_SSH(2);
    case 64: HST_SSH(4);
    default: HST_SSH(8);
  }
#undef HST_SSH
}

}  // namespace hst
