// Device helpers shared by the decode-path kernels (internal).
#pragma once

#include "block_select.h"
#include "hst_common.h"
#include "hst_fused.h"

namespace hst {

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLn2F = 0.6931471805599453f;

__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  // integer finalizer ("lowbias32", C. Wellons): a fixed pseudo-random
  // offset per stratum of the key sample
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Position of sample i among n keys.  When n > kSample the sample is
// kSample / kRunLen runs of kRunLen consecutive keys, run r at a fixed
// pseudo-random offset inside stratum r = [r*n/R, (r+1)*n/R) (every stratum
// is at least kRunLen keys wide), so a workgroup can read the sampled keys'
// metadata in short contiguous pieces; otherwise every key is taken.
static_assert((kSample & (kSample - 1)) == 0 && kSample % kRunLen == 0, "sample shape");
__device__ __forceinline__ int sample_pos(int i, int S, int n) {
  if (S >= n) return i;
  constexpr int kRuns = kSample / kRunLen;
  constexpr int kShift = __builtin_ctz(kRuns);
  const int r = i / kRunLen, o = i % kRunLen;
  const unsigned long long nn = static_cast<unsigned long long>(n);
  const uint32_t lo = static_cast<uint32_t>((static_cast<unsigned long long>(r) * nn) >> kShift);
  const uint32_t hi = static_cast<uint32_t>((static_cast<unsigned long long>(r + 1) * nn) >> kShift);
  const uint32_t span = hi - lo - kRunLen + 1;  // >= 1
  return static_cast<int>(lo + mix32(static_cast<uint32_t>(r) * 0x9e3779b9u + 0x632be5abu) % span) + o;
}

__device__ __forceinline__ int keff_of(int kcap, const int32_t* k_per_seq, int b, int n) {
  int k = kcap;
  if (k_per_seq != nullptr) {
    const int kb = k_per_seq[b];
    k = kb < 0 ? 0 : (kb < kcap ? kb : kcap);
  }
  return k < n ? k : n;
}

// Rank in a sample of S_eff keys whose score bounds the top-k threshold from
// below with a wide margin (mean + 4 sd of the binomial count + 8).
__device__ __forceinline__ int sample_rank(int k, int n, int S_eff) {
  if (n <= 0 || k <= 0) return 0;
  const double f = static_cast<double>(k) / n;
  const double mu = f * S_eff;
  const double r = ceil(mu + 4.0 * sqrt(mu * (1.0 - f)) + 8.0);
  return r >= S_eff ? S_eff : static_cast<int>(r);
}

template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
  if (LANES >= 2)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  if (LANES >= 4)
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  if (LANES >= 8) v += __shfl_xor(v, 4, 8);
  return v;
}

// Copies n >= 1 16-byte vectors from global memory to LDS with NT threads.
// Each thread moves runs of B consecutive vectors (one address, immediate
// offsets), so its B loads are issued back to back; a run past the end is
// clamped to the last vector and only the stores are predicated.
template <int NT, int B>
__device__ __forceinline__ void copy_to_lds(u32x4* __restrict__ dst, const u32x4* __restrict__ src, int n) {
  for (int r0 = 0; r0 < n; r0 += NT * B) {
    const int i = r0 + static_cast<int>(threadIdx.x) * B;
    const u32x4* p = src + (i + B <= n ? i : n - B >= 0 ? n - B : 0);
    u32x4 v[B];
#pragma unroll
    for (int u = 0; u < B; ++u) v[u] = p[u < n ? u : 0];
    const int base = i + B <= n ? i : (n - B >= 0 ? n - B : 0);
#pragma unroll
    for (int u = 0; u < B; ++u)
      if (base + u < n && base + u >= i) dst[base + u] = v[u];
  }
}

constexpr int kSelCap = 8192;  // candidates a workgroup selects from in LDS

// Candidate slots of one head seen as one array in index order; entry i lives
// in the chunk c with offs[c] <= i < offs[c+1].
__device__ __forceinline__ int chunk_of(const int* offs, int nch, int i) {
  int lo = 0, hi = nch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= i) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
struct SlotSrc {
  const uint2* slots;
  const int* offs;
  int nch, chunk;
  __device__ __forceinline__ uint2 at(int i) const {
    const int c = chunk_of(offs, nch, i);
    return slots[static_cast<long long>(c) * chunk + (i - offs[c])];
  }
  __device__ __forceinline__ uint32_t key(int i) const { return at(i).x; }
  __device__ __forceinline__ int32_t idx(int i) const { return static_cast<int32_t>(at(i).y); }
};

// Stable compaction restricted to output positions [r0, r1): entry i of the
// selection goes to out_g[p] (global, nullable) and out_l[p - r0] (LDS,
// nullable) when its position p lies in the range.  Stops once r1 is passed.
template <int NT, class Src>
__device__ void block_compact_range(const Src& src, int M, const SelRule& rule, int r0, int r1,
                                    int32_t* out_g, int32_t* out_l, BlockScratch<NT>& sc) {
  int out_pos = 0, eq_seen = 0;
  for (int base = 0; base < M && out_pos < r1; base += NT) {
    const int i = base + threadIdx.x;
    bool gt = false, eq = false;
    if (i < M) {
      const uint32_t m = src.key(i) & rule.mask;
      gt = m > rule.prefix;
      eq = m == rule.prefix;
    }
    int eqtot;
    const int eqx = block_excl_scan<NT>(eq ? 1 : 0, sc, eqtot);
    const bool sel = gt || (eq && eq_seen + eqx < rule.krem);
    int seltot;
    const int selx = block_excl_scan<NT>(sel ? 1 : 0, sc, seltot);
    const int p = out_pos + selx;
    if (sel && p >= r0 && p < r1) {
      const int32_t v = src.idx(i);
      if (out_g != nullptr) out_g[p] = v;
      if (out_l != nullptr) out_l[p - r0] = v;
    }
    out_pos += seltot;
    eq_seen += eqtot;
  }
}

__device__ __forceinline__ int lanes_below(unsigned long long m) {
  return static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
}

// Radix search for the k-th largest (1 <= k <= count) of the keys held PER
// per thread (entry e of thread t is entry t + e * NT; entries >= count are
// ignored), 11-bit digits below the common prefix of the keys, at most
// max_pass passes.  On return an entry with masked key m = key & mask is
// above the k-th iff m > prefix; when all passes ran, exactly krem of the
// entries with m == prefix are needed to complete the k largest.  After fewer
// passes (max_pass reached), prefix (with its unresolved low bits zero) is a
// lower bound of the k-th largest key.  hist: 2048 words of LDS.
template <int NT, int PER>
__device__ void radix_select_regs(const uint32_t (&key)[PER], int count, int k, int max_pass,
                                  uint32_t* hist, BlockScratch<NT>& sc, uint32_t& mask,
                                  uint32_t& prefix, int& krem, uint32_t* kmin = nullptr) {
  const int t = threadIdx.x;
  mask = 0u;
  prefix = 0u;
  krem = k;
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (t + e * NT < count) {
      mn = min(mn, key[e]);
      mx = max(mx, key[e]);
    }
  block_minmax<NT>(mn, mx, sc);
  if (kmin != nullptr) *kmin = mn;
  if (mn == mx) return;  // every key equal: mask 0 selects krem of them
  const int hb = 31 - __clz(static_cast<int>(mn ^ mx));
  mask = hb == 31 ? 0u : ~((1u << (hb + 1)) - 1u);
  prefix = mn & mask;
  int lo = hb + 1;
  for (int pass = 0; lo > 0 && pass < max_pass; ++pass) {
    const int width = lo < 11 ? lo : 11;
    const int sh = lo - width;
    const int nb = 1 << width;
    for (int i = t; i < nb; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < PER; ++e)
      if (t + e * NT < count && (key[e] & mask) == prefix) atomicAdd(&hist[(key[e] >> sh) & (nb - 1)], 1u);
    __syncthreads();
    // thread t owns bins [t*per, t*per + per) counted from the top digit down;
    // wave-level inclusive scan, then every thread adds the totals of the
    // waves before its own
    constexpr int NW = NT / 64;
    constexpr int MAXPER = (2048 + NT - 1) / NT;
    const int per = (nb + NT - 1) / NT;
    int c[MAXPER];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < MAXPER; ++i) {
      const int r = t * per + i;
      c[i] = (i < per && r < nb) ? static_cast<int>(hist[nb - 1 - r]) : 0;
      mine += c[i];
    }
    const int lane = t & 63, w = t >> 6;
    const int incl = wave_incl_scan(mine);
    if (lane == 63) sc.wsum[w] = incl;
    __syncthreads();
    int above = incl - mine;
#pragma unroll
    for (int i = 0; i < NW; ++i)
      if (i < w) above += sc.wsum[i];
    if (above < krem && krem <= above + mine) {
      int cum = above;
#pragma unroll
      for (int i = 0; i < MAXPER; ++i) {
        if (i < per && cum + c[i] >= krem) {
          sc.found[0] = nb - 1 - (t * per + i);
          sc.found[1] = krem - cum;
          sc.found[2] = c[i];
          break;
        }
        cum += c[i];
      }
    }
    __syncthreads();
    const int digit = sc.found[0];
    krem = sc.found[1];
    const int cnt = sc.found[2];
    prefix |= static_cast<uint32_t>(digit) << sh;
    mask |= static_cast<uint32_t>(nb - 1) << sh;
    lo = sh;
    if (cnt == krem) break;  // the whole bin is taken
  }
}

// Exact selection over M <= NT * PERW candidates held in LDS in index order,
// on keys held in registers: wave w holds the entries at positions
// [lo_w, hi_w) (lane l's entry u at lo_w + 64u + l), the order in which the
// compaction walks them, so the counts and the compaction come from ballots
// over registers instead of a second pass over LDS.  Radix passes of up to
// 11 bits below the keys' common prefix narrow the bin of the k-th largest
// key; once that bin holds at most kRankBin entries they are ranked directly
// by (key descending, position ascending), which resolves the k-th key and
// how many keys equal to it are taken, without further passes.  The result
// is the masked-prefix rule of radix_select_regs.  Writes the selected
// indices at output positions [r0, r1).  hist: 2048 words of LDS.
// candi: the entries' key indices, anything indexable by position (an LDS
// array, or a map from positions to indices).
constexpr int kRankBin = 64;
template <int NT, int PERW, class Idx>
__device__ void select_lds_regs(const uint32_t* candk, const Idx& candi, int M, int k, int r0, int r1,
                                int32_t* out_g, int32_t* out_l, uint32_t* hist, BlockScratch<NT>& sc) {
  constexpr int NW = NT / 64;
  constexpr int MAXPER = (2048 + NT - 1) / NT;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int span = ((M + NW - 1) / NW + 63) & ~63;
  const int lo = min(M, wave * span), hi = min(M, lo + span);
  uint32_t key[PERW];
#pragma unroll
  for (int u = 0; u < PERW; ++u) {
    const int p = lo + 64 * u + lane;
    key[u] = p < hi ? candk[p] : 0u;
  }
  // rule: selected iff (key & mask) > prefix, or (key & mask) == prefix among
  // the first krem such entries in index order
  uint32_t mask = 0u, prefix = 0u;
  int krem = k < M ? k : M;
  if (k < M) {
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int u = 0; u < PERW; ++u)
      if (lo + 64 * u + lane < hi) {
        mn = min(mn, key[u]);
        mx = max(mx, key[u]);
      }
    block_minmax<NT>(mn, mx, sc);
    if (mn != mx) {
      const int hb = 31 - __clz(static_cast<int>(mn ^ mx));
      mask = hb == 31 ? 0u : ~((1u << (hb + 1)) - 1u);
      prefix = mn & mask;
      int lob = hb + 1;
      while (lob > 0) {
        const int width = lob < 11 ? lob : 11;
        const int sh = lob - width;
        const int nb = 1 << width;
        const uint32_t dm = static_cast<uint32_t>(nb - 1);
        for (int i = t; i < nb; i += NT) hist[i] = 0u;
        if (t == 0) sc.found[3] = 0;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < PERW; ++u)
          if (lo + 64 * u + lane < hi && (key[u] & mask) == prefix) atomicAdd(&hist[(key[u] >> sh) & dm], 1u);
        __syncthreads();
        // the bin holding rank krem, counted from the top digit down: thread t
        // owns bins [t*per, t*per + per) of that order
        const int per = (nb + NT - 1) / NT;
        int c[MAXPER];
        int mine = 0;
#pragma unroll
        for (int i = 0; i < MAXPER; ++i) {
          const int r = t * per + i;
          c[i] = (i < per && r < nb) ? static_cast<int>(hist[nb - 1 - r]) : 0;
          mine += c[i];
        }
        const int incl = wave_incl_scan(mine);
        if (lane == 63) sc.wsum[wave] = incl;
        __syncthreads();
        int above = incl - mine;
#pragma unroll
        for (int i = 0; i < NW; ++i)
          if (i < wave) above += sc.wsum[i];
        if (above < krem && krem <= above + mine) {
          int cum = above;
          bool hit = false;
#pragma unroll
          for (int i = 0; i < MAXPER; ++i) {
            if (!hit && i < per && cum + c[i] >= krem) {
              sc.found[0] = nb - 1 - (t * per + i);
              sc.found[1] = krem - cum;
              sc.found[2] = c[i];
              hit = true;
            }
            if (!hit) cum += c[i];
          }
        }
        __syncthreads();
        const int digit = sc.found[0], cnt = sc.found[2];
        krem = sc.found[1];
        prefix |= static_cast<uint32_t>(digit) << sh;
        mask |= dm << sh;
        lob = sh;
        if (cnt == krem || lob == 0) break;  // the whole bin is taken, or every bit is resolved
        if (cnt <= kRankBin) {
          // the bin's entries (key, position), in any order, over the histogram
          uint2* bl = reinterpret_cast<uint2*>(hist);
          __syncthreads();  // every thread has read its bins
          {
            // this wave's entries of the bin, then one slot reservation per wave
            int nw = 0;
#pragma unroll
            for (int u = 0; u < PERW; ++u) nw += __popcll(__ballot(lo + 64 * u + lane < hi && (key[u] & mask) == prefix));
            int base = 0;
            if (lane == 0 && nw > 0) base = atomicAdd(&sc.found[3], nw);
            base = __shfl(base, 0, 64);
#pragma unroll
            for (int u = 0; u < PERW; ++u) {
              const int p = lo + 64 * u + lane;
              const bool in = p < hi && (key[u] & mask) == prefix;
              const unsigned long long b = __ballot(in);
              if (in) bl[base + lanes_below(b)] = make_uint2(key[u], static_cast<uint32_t>(p));
              base += __popcll(b);
            }
          }
          __syncthreads();
          if (t < cnt) {
            // rank of this entry by (key descending, position ascending): the
            // bin's entries with a larger key, then its equal keys earlier
            const uint2 me = bl[t];
            int gt = 0, eq = 0;
            for (int j = 0; j < cnt; ++j) {
              const uint2 o = bl[j];
              gt += o.x > me.x ? 1 : 0;
              eq += (o.x == me.x && o.y < me.y) ? 1 : 0;
            }
            if (gt + eq == krem - 1) {  // the k-th entry: its key, and how many
              sc.found[0] = static_cast<int>(me.x);  // entries equal to it are taken
              sc.found[1] = eq + 1;
            }
          }
          __syncthreads();
          // the k-th key is now fully resolved: take the keys above it and the
          // first krem keys equal to it (index order)
          prefix = static_cast<uint32_t>(sc.found[0]);
          mask = 0xffffffffu;
          krem = sc.found[1];
          break;
        }
      }
    }
  }
  __syncthreads();  // sc.found is read above; sc.red is written below
  // counts per wave (strictly above, tied at the prefix), then the waves before
  int gtc = 0, eqc = 0;
#pragma unroll
  for (int u = 0; u < PERW; ++u) {
    const bool ok = lo + 64 * u + lane < hi;
    const uint32_t m = key[u] & mask;
    gtc += __popcll(__ballot(ok && m > prefix));
    eqc += __popcll(__ballot(ok && m == prefix));
  }
  if (lane == 0) {
    sc.red[0][wave] = static_cast<uint32_t>(gtc);
    sc.red[1][wave] = static_cast<uint32_t>(eqc);
  }
  __syncthreads();
  int gt_before = 0, eq_run = 0;
  for (int w = 0; w < wave; ++w) {
    gt_before += static_cast<int>(sc.red[0][w]);
    eq_run += static_cast<int>(sc.red[1][w]);
  }
  __syncthreads();  // sc is reused by the caller
  int run = gt_before + min(eq_run, krem);
#pragma unroll
  for (int u = 0; u < PERW; ++u) {
    const int p = lo + 64 * u + lane;
    const bool ok = p < hi;
    const uint32_t m = key[u] & mask;
    const bool top = ok && m > prefix;
    const bool eq = ok && m == prefix;
    const unsigned long long eqb = __ballot(eq);
    const bool sel = top || (eq && eq_run + lanes_below(eqb) < krem);
    const unsigned long long selb = __ballot(sel);
    const int pos = run + lanes_below(selb);
    if (sel && pos >= r0 && pos < r1) {
      const int32_t v = static_cast<int32_t>(candi[p]);
      if (out_g != nullptr) out_g[pos] = v;
      if (out_l != nullptr) out_l[pos - r0] = v;
    }
    run += __popcll(selb);
    eq_run += __popcll(eqb);
  }
}

// Lower bound of the r-th largest (1 <= r <= count) of the keys held PER per
// thread: two 11-bit radix passes below the common prefix of the keys, then
// the low edge of the bin holding rank r (the common key if all are equal).
template <int NT, int PER>
__device__ uint32_t rank_lower_bound_regs(const uint32_t (&key)[PER], int count, int r, uint32_t* hist,
                                          BlockScratch<NT>& sc) {
  uint32_t mask, prefix, kmin;
  int krem;
  radix_select_regs<NT, PER>(key, count, r, 2, hist, sc, mask, prefix, krem, &kmin);
  return mask == 0u ? kmin : prefix;
}

struct SelectScratch {
  uint32_t* candk;  // LDS, kSelCap entries
  int32_t* candi;   // LDS, kSelCap entries
  uint32_t* hist;   // LDS, 2048 words
  int* offs;        // LDS, nchunks + 1
};

// The head's exact top-k (k_eff keys, ties to the lower index) from the
// candidate slots the scan wrote (or, when fewer than k_eff keys passed the
// threshold, from the whole score row).  Writes the selected indices at
// output positions [r0, r1) (see block_compact_range) and -1 at positions
// in [max(r0, k_eff), r1) of out_g.  Returns the selection path taken
// (0: candidates in LDS, 1: candidates read from HBM, 2: whole score row).
template <int NT>
__device__ int select_range(const FusedArgs& a, int bh, int n, int k_eff, int chunk,
                            const void* scores_row, bool scores_int, const SelectScratch& ws,
                            int r0, int r1, int32_t* out_g, int32_t* out_l, BlockScratch<NT>& sc,
                            int* cand_total) {
  const int nch = (n + a.span - 1) / a.span;  // chunk c: keys [c*span, (c+1)*span), slots at c*chunk
  const uint32_t* cnt = a.counts + static_cast<long long>(bh) * a.nchunks;
  const uint2* slots = a.slots + static_cast<long long>(bh) * a.nchunks * chunk;
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the first counts, then the first 128 slots of the first eight chunks of
  // each wave (copied below), all in flight together: the slot addresses do
  // not depend on the counts (slots past a chunk's count are read, unused),
  // and the counts, issued first, arrive without waiting for the slots
  const int cnt0 = static_cast<int>(threadIdx.x) < nch ? static_cast<int>(cnt[threadIdx.x]) : 0;
  // (chunk indices clamped, so the loads are unconditional and the wait for
  // the counts counts exactly the slot loads behind them)
  uint2 pre[8][2];
  const int clast = nch > 0 ? nch - 1 : 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = min(wave + u * NW, clast);
#pragma unroll
    for (int x = 0; x < 2; ++x) pre[u][x] = slots[static_cast<long long>(c) * chunk + lane + 64 * x];
  }
  int run = 0;
  for (int c0 = 0; c0 < nch; c0 += NT) {
    const int c = c0 + static_cast<int>(threadIdx.x);
    const int v = c0 == 0 ? cnt0 : (c < nch ? static_cast<int>(cnt[c]) : 0);
    int tot;
    const int x = block_excl_scan<NT>(v, sc, tot);
    if (c < nch) ws.offs[c] = run + x;
    run += tot;
  }
  if (threadIdx.x == 0) ws.offs[nch] = run;
  __syncthreads();
  const int M = run;
  *cand_total = M;
  int path = 0;
  if (k_eff > 0) {
    if (M >= k_eff && M <= kSelCap) {
      // each wave copies whole chunks (coalesced): eight chunks and sixteen
      // loads per lane in flight (the first eight already loaded)
      for (int c0 = wave; c0 < nch; c0 += NW * 8) {
        uint2 v[8][2];
        int cnt[8], base[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = c0 + u * NW;
          cnt[u] = c < nch ? ws.offs[c + 1] - ws.offs[c] : 0;
          base[u] = c < nch ? ws.offs[c] : 0;
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            if (c0 == wave) v[u][x] = pre[u][x];
            else if (lane + 64 * x < cnt[u]) v[u][x] = slots[static_cast<long long>(c) * chunk + lane + 64 * x];
          }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
#pragma unroll
          for (int x = 0; x < 2; ++x)
            if (lane + 64 * x < cnt[u]) {
              ws.candk[base[u] + lane + 64 * x] = v[u][x].x;
              ws.candi[base[u] + lane + 64 * x] = static_cast<int32_t>(v[u][x].y);
            }
          const long long c = c0 + u * NW;
          for (int i = 128 + lane; i < cnt[u]; i += 64) {  // chunks with many candidates
            const uint2 w = slots[c * chunk + i];
            ws.candk[base[u] + i] = w.x;
            ws.candi[base[u] + i] = static_cast<int32_t>(w.y);
          }
        }
      }
      __syncthreads();
      select_lds_regs<NT, kSelCap / NT>(ws.candk, ws.candi, M, k_eff, r0, r1, out_g, out_l, ws.hist, sc);
    } else if (M >= k_eff) {
      path = 1;
      const SlotSrc src{slots, ws.offs, nch, chunk};
      const SelRule rule = block_select_rule<NT>(src, M, k_eff, ws.hist, sc);
      block_compact_range<NT>(src, M, rule, r0, r1, out_g, out_l, sc);
    } else {
      path = 2;  // the sample overestimated the threshold: use every score
      if (scores_int) {
        const I32RowSrc src{static_cast<const int32_t*>(scores_row)};
        const SelRule rule = block_select_rule<NT>(src, n, k_eff, ws.hist, sc);
        block_compact_range<NT>(src, n, rule, r0, r1, out_g, out_l, sc);
      } else {
        const F32RowSrc src{static_cast<const float*>(scores_row)};
        const SelRule rule = block_select_rule<NT>(src, n, k_eff, ws.hist, sc);
        block_compact_range<NT>(src, n, rule, r0, r1, out_g, out_l, sc);
      }
    }
  }
  if (out_g != nullptr)
    for (int p = max(r0, k_eff) + static_cast<int>(threadIdx.x); p < r1; p += NT) out_g[p] = -1;
  __syncthreads();
  return path;
}

}  // namespace hst
