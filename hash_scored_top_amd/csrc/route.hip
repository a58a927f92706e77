// Two-level chunk -> token routing.
// HGA explainer page ("Hierarchical Global Attention"), section 2: the
// context is cut into 64-token chunks, each summarised on a small index
// card; the query first scans the cards to find the relevant chunks (chunk
// routing), then goes back to the exact tokens of those chunks (token
// routing), and the answer is computed over the original tokens.
//
// Here a card is itself a stored key: the chunk's key sum (float64, index
// order) rounded to the key storage type, hashed by the ordinary soft-LSH
// kernels, and weighted by the largest stored value norm of the chunk.  The
// decode step then scores N/64 cards instead of N keys, keeps C chunks, and
// scores only their C * 64 keys.
//
//   card_sum_kernel    grid (ceil(Nc / (256 / d)), B*Hkv): one thread per
//                      (chunk, channel) sums the chunk's keys in index
//                      order; one wave per chunk takes the max norm.
//   route_scan_kernel  grid (ceil(C / 16), B*Hkv), 1024 threads: the head's
//                      table, transposed to table-major in LDS (bank =
//                      bucket), scores the 64 keys of each of 16 chosen
//                      chunks, one key per thread.
//   card_route_kernel  one 1024-thread workgroup per (sequence, kv head):
//                      every card's score from the partial scores the
//                      prep workgroups wrote (each on its own tables, see
//                      prep.hip) times the card weight, then the exact
//                      top C is cut and compacted.
//   token_route_kernel one 1024-thread workgroup per (sequence, kv head):
//                      the exact top k of the scored keys, mapped from
//                      positions in the kept chunks to key indices.
// Both cut with the selection of the attention kernel (keys held in
// registers, radix passes, a direct rank of a small boundary bin, ballot
// compaction); a card cut over more than 2048 cards uses a radix select of
// count histograms (12, 10, 10 bits; after the first level only the
// crossing bucket's items are visited) instead.  Ties go to the lower
// position, which is the lower index; output ascending.
#include "fused_device.h"
#include "hst_launch.h"
#include "table_lds.h"

namespace hst {

constexpr int kChunkTok = kCardKeys;  // tokens per chunk
constexpr int kMaxCardParts = 16;     // partial card scores per head (prep workgroups)
constexpr int kTopNT = 1024;        // threads of the small top-k
constexpr int kRouteNT = 1024;      // threads of the routed scan (16 chunks)

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  return static_cast<uint16_t>((b + 0x7fffu + ((b >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ void store_key(float* p, double v) { *p = static_cast<float>(v); }
__device__ __forceinline__ void store_key(bf16* p, double v) {
  p->bits = f32_to_bf16_rne(static_cast<float>(v));
}

template <typename T>
__global__ void __launch_bounds__(256)
card_sum_kernel(const T* __restrict__ K, const void* __restrict__ vnorm, int norm_f16,
                const int32_t* __restrict__ seq_lens, int B, int Hkv, int Nmax, int Nc, int d,
                T* __restrict__ ckeys, void* __restrict__ cw, int32_t* __restrict__ clens) {
  const int bh = blockIdx.y, b = bh / Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int nc = (n + kChunkTok - 1) / kChunkTok;
  const int t = threadIdx.x, per = 256 / d;
  const int c = blockIdx.x * per + t / d, ch = t % d;
  if (blockIdx.x == 0 && bh % Hkv == 0 && t == 0) clens[b] = nc;
  if (c >= nc) return;  // whole waves: d is a multiple of 64
  const int j0 = c * kChunkTok, j1 = min(j0 + kChunkTok, n);
  const T* kp = K + (static_cast<long long>(bh) * Nmax + j0) * d + ch;
  double acc = 0.0;
  for (int j = j0; j < j1; ++j, kp += d) acc += to_f64(*kp);
  store_key(ckeys + (static_cast<long long>(bh) * Nc + c) * d + ch, acc);
  // card weight: the largest stored value norm of the chunk (lane = row);
  // norms are non-negative, so their bit patterns order like their values
  if (ch < 64) {
    const long long row = static_cast<long long>(bh) * Nmax + j0 + ch;
    uint32_t v = 0;
    if (j0 + ch < j1)
      v = norm_f16 ? static_cast<uint32_t>(static_cast<const uint16_t*>(vnorm)[row])
                   : static_cast<const uint32_t*>(vnorm)[row];
    for (int x = 32; x >= 1; x >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), x)));
    if (ch == 0) {
      const long long o = static_cast<long long>(bh) * Nc + c;
      if (norm_f16)
        static_cast<uint16_t*>(cw)[o] = static_cast<uint16_t>(v);
      else
        static_cast<uint32_t*>(cw)[o] = v;
    }
  }
}

// Scores of the keys of the chosen chunks: out[bh][slot * 64 + i] for key
// chunk * 64 + i of the slot-th chosen chunk; -1 where there is no key.
template <int L>
__global__ void __launch_bounds__(kRouteNT)
route_scan_kernel(const float* __restrict__ tables, const int32_t* __restrict__ chunks, int C,
                  const uint8_t* __restrict__ ids, const void* __restrict__ vnorm, int norm_f16,
                  const int32_t* __restrict__ seq_lens, int Hkv, int Nmax, int P, int out_stride,
                  float* __restrict__ out) {
  extern __shared__ __align__(16) float tl[];  // [L][2^P + 1], table-major
  const int bh = blockIdx.y, b = bh / Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int nb = 1 << P, t = threadIdx.x;
  const float* Tg = tables + static_cast<long long>(bh) * nb * L;
  const int slot = blockIdx.x * (kRouteNT / kChunkTok) + t / kChunkTok;
  const int c = slot < C ? chunks[static_cast<long long>(bh) * C + slot] : -1;
  const int j = c * kChunkTok + (t % kChunkTok);
  const bool ok = c >= 0 && j < n;
  // this key's ids and norm first, then the table
  u32x4 idv[L / 16];
  const u32x4* ip = reinterpret_cast<const u32x4*>(ids + (static_cast<long long>(bh) * Nmax + (ok ? j : 0)) * L);
#pragma unroll
  for (int i = 0; i < L / 16; ++i) idv[i] = ip[i];
  const long long row = static_cast<long long>(bh) * Nmax + (ok ? j : 0);
  const float w = norm_f16 ? f16_bits_to_f32(static_cast<const uint16_t*>(vnorm)[row])
                           : static_cast<const float*>(vnorm)[row];
  load_table_t<kRouteNT>(Tg, tl, L, nb);
  __syncthreads();
  const float s = table_sum<L>(idv, tl, nb);
  if (slot < C)
    out[static_cast<long long>(bh) * out_stride + slot * kChunkTok + (t % kChunkTok)] = ok ? w * s : -1.0f;
}

// Order key of a score: larger scores give larger keys, 0 marks no item.
__device__ __forceinline__ uint32_t score_key(float s) {
  return (s >= 0.0f) ? (__float_as_uint(s) & 0x7fffffffu) + 1u : 0u;  // -0 counts as +0
}

template <typename V>
__device__ __forceinline__ V block_excl_scan_r(V v, V* red) {
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

// Exact cut of a top-`want` selection over order keys in LDS (0 = no
// item; valid > want >= 1 items): the threshold key and how many items equal
// to it are taken.  Three radix levels (12, 10, 10 bits) of count
// histograms; after the first, only the items of the crossing bucket are
// visited again (gathered into `cand`, in any order: only counts matter).
struct Cut {
  uint32_t thr, need;
};

struct CutScratch {
  uint32_t* hist;  // 4096
  uint32_t* cand;  // as many as the items
  uint32_t* red;   // kTopNT / 64
  uint32_t* vars;  // 4
};

__device__ Cut block_radix_cut(const uint32_t* key, int nitems, uint32_t want, CutScratch sc) {
  const int t = threadIdx.x;
  // level 0: bits 31..20
  for (int i = t; i < 4096; i += kTopNT) sc.hist[i] = 0;
  if (t == 0) sc.vars[2] = 0;
  __syncthreads();
  for (int r = t; r < nitems; r += kTopNT) {
    const uint32_t k = key[r];
    if (k) atomicAdd(&sc.hist[k >> 20], 1u);
  }
  __syncthreads();
  // buckets from the top, four per thread: thread t owns 4095 - 4t .. 4092 - 4t
  uint32_t part = 0;
  for (int u = 0; u < 4; ++u) part += sc.hist[4095 - 4 * t - u];
  uint32_t above = block_excl_scan_r<uint32_t>(part, sc.red);
  if (above < want && above + part >= want) {
    int b0 = 4092 - 4 * t;
    for (int u = 0; u < 4; ++u) {
      const int bk = 4095 - 4 * t - u;
      if (above + sc.hist[bk] >= want) {
        b0 = bk;
        break;
      }
      above += sc.hist[bk];
    }
    sc.vars[0] = static_cast<uint32_t>(b0);
    sc.vars[1] = above;
  }
  __syncthreads();
  const uint32_t b0 = sc.vars[0];
  uint32_t abv = sc.vars[1];
  // gather the crossing bucket: one counter update per wave and row
  const int lane = t & 63;
  for (int base = t - lane; base < nitems; base += kTopNT) {
    const int r = base + lane;
    const uint32_t k = r < nitems ? key[r] : 0u;
    const bool in = k && (k >> 20) == b0;
    const unsigned long long m = __ballot(in);
    if (m == 0) continue;
    uint32_t at = 0;
    if (lane == __ffsll(static_cast<long long>(m)) - 1) at = atomicAdd(&sc.vars[2], static_cast<uint32_t>(__popcll(m)));
    at = __shfl(at, __ffsll(static_cast<long long>(m)) - 1);
    if (in) sc.cand[at + __popcll(m & ((1ull << lane) - 1))] = k;
  }
  __syncthreads();
  const int m = static_cast<int>(sc.vars[2]);
  uint32_t prefix = b0;
  // levels 1 and 2: bits 19..10, then 9..0, over the gathered items
  for (int level = 1; level <= 2; ++level) {
    const int shift = level == 1 ? 10 : 0;
    sc.hist[t] = 0;  // 1024 buckets, one per thread
    __syncthreads();
    for (int i = t; i < m; i += kTopNT) {
      const uint32_t k = sc.cand[i];
      if ((k >> (shift + 10)) == prefix) atomicAdd(&sc.hist[(k >> shift) & 1023u], 1u);
    }
    __syncthreads();
    const uint32_t c = sc.hist[1023 - t];
    const uint32_t ex = block_excl_scan_r<uint32_t>(c, sc.red);
    if (abv + ex < want && abv + ex + c >= want) {
      sc.vars[0] = static_cast<uint32_t>(1023 - t);
      sc.vars[1] = abv + ex;
    }
    __syncthreads();
    prefix = (prefix << 10) | sc.vars[0];
    abv = sc.vars[1];
    __syncthreads();
  }
  return Cut{prefix, want - abv};
}

// Positions in [0, nitems) taken by (thr, need), ascending: every key above
// thr and the first `need` equal to it.  Writes out[i] = map(position) for
// the i-th, then -1 up to out_len; returns the count.  Wave w owns a
// contiguous run of rows of 64 items; lanes read consecutive items (no bank
// conflicts) and place them by ballot counts.
template <typename Map>
__device__ int block_cut_compact(const uint32_t* key, int nitems, Cut cut, int32_t* out,
                                 int out_len, uint64_t* red64, uint32_t* total, Map map) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  constexpr int NW = kTopNT / 64;
  const int rows = (nitems + 63) / 64, rpw = (rows + NW - 1) / NW;
  const int r0 = min(wv * rpw, rows), r1 = min(r0 + rpw, rows);
  const unsigned long long below = (1ull << lane) - 1;
  uint32_t gtw = 0, eqw = 0;
  for (int row = r0; row < r1; ++row) {
    const int r = row * 64 + lane;
    const uint32_t k = r < nitems ? key[r] : 0u;
    gtw += __popcll(__ballot(k != 0 && k > cut.thr));
    eqw += __popcll(__ballot(k != 0 && k == cut.thr));
  }
  // exclusive scan over the waves (lane 0 of each wave contributes)
  const uint64_t mine = (static_cast<uint64_t>(eqw) << 32) | gtw;
  const uint64_t before = block_excl_scan_r<uint64_t>(lane == 0 ? mine : 0ull, red64);
  uint64_t wb = __shfl(before, 0);  // lane 0 of this wave: sum over earlier waves
  uint32_t gt_run = static_cast<uint32_t>(wb & 0xffffffffu), eq_run = static_cast<uint32_t>(wb >> 32);
  if (t == kTopNT - 1) {
    const uint64_t all = wb + mine;  // mine is the same in every lane of the wave
    *total = static_cast<uint32_t>(all & 0xffffffffu) + min(static_cast<uint32_t>(all >> 32), cut.need);
  }
  for (int row = r0; row < r1; ++row) {
    const int r = row * 64 + lane;
    const uint32_t k = r < nitems ? key[r] : 0u;
    const bool gt = k != 0 && k > cut.thr, eq = k != 0 && k == cut.thr;
    const unsigned long long mg = __ballot(gt), me = __ballot(eq);
    const uint32_t gb = gt_run + __popcll(mg & below), eb = eq_run + __popcll(me & below);
    if (gt || (eq && eb < cut.need)) out[gb + min(eb, cut.need)] = map(r);
    gt_run += __popcll(mg);
    eq_run += __popcll(me);
  }
  __syncthreads();
  const int n = static_cast<int>(*total);
  for (int r = n + t; r < out_len; r += kTopNT) out[r] = -1;
  return n;
}

// Top-`want` cut over keys[0, nitems) with `valid` non-zero keys.
__device__ Cut block_cut(const uint32_t* key, int nitems, uint32_t valid, uint32_t want,
                         CutScratch sc) {
  if (want >= valid) return Cut{1u, 0xffffffffu};  // every item (keys are >= 1)
  if (want == 0) return Cut{0xffffffffu, 0u};      // none
  return block_radix_cut(key, nitems, want, sc);
}

// Count, smallest and largest of the non-zero keys in LDS (0 marks no item),
// in one pass.  red3: 3 * kTopNT / 64 words of LDS.
struct KeyStats {
  uint32_t valid, kmin, kmax;
};
__device__ __forceinline__ KeyStats block_key_stats(const uint32_t* key, int nitems, uint32_t* red3) {
  constexpr int NW = kTopNT / 64;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  uint32_t v = 0, mn = 0xffffffffu, mx = 0u;
  for (int r = t; r < nitems; r += kTopNT) {
    const uint32_t k = key[r];
    if (k != 0u) {
      ++v;
      mn = min(mn, k);
      mx = max(mx, k);
    }
  }
  for (int m = 32; m >= 1; m >>= 1) {
    v += static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), m));
    mn = min(mn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mn), m)));
    mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), m)));
  }
  __syncthreads();
  if (lane == 0) {
    red3[wv] = v;
    red3[NW + wv] = mn;
    red3[2 * NW + wv] = mx;
  }
  __syncthreads();
  KeyStats s{0u, 0xffffffffu, 0u};
  for (int w = 0; w < NW; ++w) {
    s.valid += red3[w];
    s.kmin = min(s.kmin, red3[NW + w]);
    s.kmax = max(s.kmax, red3[2 * NW + w]);
  }
  return s;
}

// A card's position is its chunk index.
struct PosIdx {
  __device__ __forceinline__ int32_t operator[](int r) const { return r; }
};

// Chunk routing for one (sequence, kv head): the score of card c is its
// weight times the sum of the xparts partial scores the prep workgroups
// wrote (each over its own group of tables, added in group order), and the
// C best cards (score descending, chunk ascending) are written ascending to
// chunks[bh][0..C), then -1.  REGS: the selection on register-held keys, two
// cards per lane (Nc <= 2048); else the count-histogram cut (more cards
// would spill the registers).
template <bool REGS>
__global__ void __launch_bounds__(kTopNT)
card_route_kernel(const float* __restrict__ cpart, int xparts, const void* __restrict__ cw, int norm_f16,
                  const int32_t* __restrict__ seq_lens, int Hkv, int Nmax, int Nc, int C,
                  int32_t* __restrict__ chunks) {
  extern __shared__ __align__(16) unsigned char sm[];
  uint32_t* cand = reinterpret_cast<uint32_t*>(sm);  // the count-histogram cut's candidates
  uint32_t* key = cand + Nc;
  uint32_t* hist = key + Nc;  // 4096
  __shared__ uint32_t red[3 * (kTopNT / 64)];
  __shared__ BlockScratch<kTopNT> tsc;
  __shared__ uint64_t red64[kTopNT / 64];
  __shared__ uint32_t vars[4], total;
  const int bh = blockIdx.x, b = bh / Hkv, t = threadIdx.x;
  const int n = seq_len(seq_lens, b, Nmax);
  const int nc = (n + kChunkTok - 1) / kChunkTok;
  const float* pp = cpart + static_cast<long long>(bh) * xparts * Nc;
  for (int c0 = 0; c0 < Nc; c0 += 2 * kTopNT) {
    // two cards per thread, every part of both in flight together
    float pv[2][kMaxCardParts];
    float w[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = min(c0 + t + u * kTopNT, max(nc - 1, 0));
      const long long row = static_cast<long long>(bh) * Nc + c;
#pragma unroll
      for (int x = 0; x < kMaxCardParts; ++x) pv[u][x] = x < xparts ? pp[static_cast<long long>(x) * Nc + c] : 0.f;
      w[u] = norm_f16 ? f16_bits_to_f32(static_cast<const uint16_t*>(cw)[row]) : static_cast<const float*>(cw)[row];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = c0 + t + u * kTopNT;
      if (c >= Nc) continue;
      float s = 0.0f;
#pragma unroll
      for (int x = 0; x < kMaxCardParts; ++x)
        if (x < xparts) s += pv[u][x];
      key[c] = c < nc ? score_key(w[u] * s) : 0u;
    }
  }
  __syncthreads();
  const KeyStats kst = block_key_stats(key, Nc, red);
  const uint32_t valid = kst.valid;
  int32_t* orow = chunks + static_cast<long long>(bh) * C;
  if constexpr (REGS) {
    // the C best cards (fewer if fewer chunks exist), ascending, then -1, by
    // the selection's histogram over the keys' own range (radix passes only
    // when a bin is too full to rank)
    const int ks = min(min(C, nc), static_cast<int>(valid));
    const HistInfo hi{kst.kmin, hist_shift(kst.kmin, kst.kmax), true};
    if (ks > 0)
      select_lds_core<kTopNT, 2, PosIdx, true>(key, PosIdx{}, Nc, ks, 0, ks, orow, nullptr, hist, tsc, hi);
    for (int p = ks + t; p < C; p += kTopNT) orow[p] = -1;
  } else {
    const Cut cut = block_cut(key, Nc, valid, static_cast<uint32_t>(min(C, nc)),
                              CutScratch{hist, cand, red, vars});
    block_cut_compact(key, Nc, cut, orow, C, red64, &total, [](int r) { return r; });
  }
}

// Position r of the scored keys of the kept chunks (slot r / 64, token r % 64)
// as a key index.
struct ChunkIdx {
  const int32_t* cl;  // kept chunks, ascending (LDS)
  __device__ __forceinline__ int32_t operator[](int r) const { return cl[r / kChunkTok] * kChunkTok + (r % kChunkTok); }
};

// Token routing: the k (or k_per_seq[b]) best of the scored keys of the kept
// chunks, as key indices, ascending.
__global__ void __launch_bounds__(kTopNT)
token_route_kernel(const float* __restrict__ scores, int nitems,
                   const int32_t* __restrict__ chunks, int C, int k,
                   const int32_t* __restrict__ k_per_seq, int Hkv, int32_t* __restrict__ out) {
  extern __shared__ __align__(16) uint32_t keybuf[];  // [nitems] keys, [2048] hist
  __shared__ uint32_t red[3 * (kTopNT / 64)];
  __shared__ BlockScratch<kTopNT> tsc;
  const int bh = blockIdx.x, b = bh / Hkv, t = threadIdx.x;
  uint32_t* key = keybuf;
  uint32_t* hist = keybuf + nitems;  // 2048 words of radix histogram
  __shared__ int32_t cl[kRouteMaxChunks];
  const float* sr = scores + static_cast<long long>(bh) * nitems;
  const int32_t* crow = chunks + static_cast<long long>(bh) * C;
  if (t < C) cl[t] = crow[t];
  {
    const int n4 = nitems / 4;  // nitems is a multiple of 64
    const u32x4* src = reinterpret_cast<const u32x4*>(sr);
    for (int base = 0; base < n4; base += 4 * kTopNT) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * kTopNT + t;
        if (i < n4) v[u] = src[i];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = base + u * kTopNT + t;
        if (i < n4) {
          u32x4 kv;
#pragma unroll
          for (int q = 0; q < 4; ++q) kv[q] = score_key(__uint_as_float(v[u][q]));
          reinterpret_cast<u32x4*>(key)[i] = kv;
        }
      }
    }
  }
  __syncthreads();
  const KeyStats kst = block_key_stats(key, nitems, red);
  const uint32_t valid = kst.valid;
  int kb = k_per_seq != nullptr ? k_per_seq[b] : k;
  kb = max(0, min(kb, k));
  // the kb best (fewer if fewer keys exist: a missing key's order key 0 is
  // below every real one, so it is never among them), by the selection on
  // register-held keys, radix passes from the keys' common prefix (a
  // histogram over [min, max] crowds these skewed scores into a few bins);
  // positions map to key indices through the kept chunks
  const int ks = min(kb, static_cast<int>(valid));
  int32_t* orow = out + static_cast<long long>(bh) * k;
  if (ks > 0)
    select_lds_regs<kTopNT, kRouteMaxChunks * kChunkTok / kTopNT>(key, ChunkIdx{cl}, nitems, ks, 0, ks, orow,
                                                                   nullptr, hist, tsc);
  for (int p = ks + t; p < k; p += kTopNT) orow[p] = -1;
}

template <typename K>
static hipError_t route_lds_limit(K kern, size_t bytes) {
  return raise_lds_limit(reinterpret_cast<const void*>(kern), bytes);
}

int route_chunks(int Nmax) { return (Nmax + kChunkTok - 1) / kChunkTok; }


hipError_t launch_card_sums(const hst_shape& s, const void* K, const void* vnorm, int norm_f16,
                            void* ckeys, void* cw, int32_t* clens, hipStream_t st) {
  const int Nc = route_chunks(s.Nmax);
  const int per = 256 / s.d;
  const dim3 grid(static_cast<unsigned>((Nc + per - 1) / per), static_cast<unsigned>(s.B * s.Hkv));
  if (s.kv_dtype == HST_F32)
    hipLaunchKernelGGL(card_sum_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(K),
                       vnorm, norm_f16, s.seq_lens, s.B, s.Hkv, s.Nmax, Nc, s.d,
                       static_cast<float*>(ckeys), cw, clens);
  else
    hipLaunchKernelGGL(card_sum_kernel<bf16>, grid, dim3(256), 0, st, static_cast<const bf16*>(K),
                       vnorm, norm_f16, s.seq_lens, s.B, s.Hkv, s.Nmax, Nc, s.d,
                       static_cast<bf16*>(ckeys), cw, clens);
  return hipGetLastError();
}

hipError_t launch_route_scan(const hst_shape& s, const float* tables, const int32_t* chunks, int C,
                             const uint8_t* ids, const void* vnorm, int norm_f16, int L, int P,
                             int out_stride, float* out, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((C + 15) / 16), static_cast<unsigned>(s.B * s.Hkv));
  const size_t smem = static_cast<size_t>(L) * ((1u << P) + 1) * 4;
  hipError_t e;
#define HST_ROUTE_L(LL)                                                                          \
  case LL:                                                                                       \
    e = route_lds_limit(route_scan_kernel<LL>, smem);                                            \
    if (e != hipSuccess) return e;                                                               \
    hipLaunchKernelGGL(route_scan_kernel<LL>, grid, dim3(kRouteNT), smem, st, tables, chunks, C, \
                       ids, vnorm, norm_f16, s.seq_lens, s.Hkv, s.Nmax, P, out_stride, out);     \
    break;
  switch (L) {
    HST_ROUTE_L(16)
    HST_ROUTE_L(32)
    HST_ROUTE_L(64)
    HST_ROUTE_L(128)
    default: return hipErrorInvalidValue;
  }
#undef HST_ROUTE_L
  return hipGetLastError();
}

size_t card_route_smem(int Nc) {
  return static_cast<size_t>(Nc) * 8 + 4096 * 4;  // candidates, keys, histogram
}

hipError_t launch_card_route(const hst_shape& s, const float* cpart, int xparts, const void* cw,
                             int norm_f16, int C, int32_t* chunks, hipStream_t st) {
  const int Nc = route_chunks(s.Nmax);
  if (xparts < 1 || xparts > kMaxCardParts) return hipErrorInvalidValue;
  const size_t smem = card_route_smem(Nc);
  hipError_t e;
#define HST_CARD(RG)                                                                                \
  do {                                                                                              \
    e = route_lds_limit(card_route_kernel<RG>, smem);                                               \
    if (e != hipSuccess) return e;                                                                  \
    hipLaunchKernelGGL((card_route_kernel<RG>), dim3(s.B * s.Hkv), dim3(kTopNT), smem, st, cpart,    \
                       xparts, cw, norm_f16, s.seq_lens, s.Hkv, s.Nmax, Nc, C, chunks);             \
  } while (0)
  if (Nc <= 2 * kTopNT) HST_CARD(true);
  else HST_CARD(false);
#undef HST_CARD
  return hipGetLastError();
}

hipError_t launch_token_route(const hst_shape& s, const float* scores, int nitems,
                              const int32_t* chunks, int C, int k, const int32_t* kps,
                              int32_t* out, hipStream_t st) {
  const size_t smem = static_cast<size_t>(nitems) * 4 + 2048 * 4;
  hipError_t e = route_lds_limit(token_route_kernel, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(token_route_kernel, dim3(s.B * s.Hkv), dim3(kTopNT), smem, st, scores, nitems,
                     chunks, C, k, kps, s.Hkv, out);
  return hipGetLastError();
}

}  // namespace hst
