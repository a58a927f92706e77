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
                                  uint32_t& prefix, int& krem, uint32_t* kmin = nullptr,
                                  uint32_t* kmax = nullptr) {
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
  if (kmax != nullptr) *kmax = mx;
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

// Binning of a selection's candidate histogram: key c falls in bin
// min(kHistBins - 1, (c - theta) >> shift), and keys below theta (a chunk
// that filtered with a lower threshold) in bin 0, so bins keep the key order.
struct HistInfo {
  uint32_t theta;
  int shift;
  bool ok;
  __device__ __forceinline__ int bin(uint32_t c) const {
    if (c < theta) return 0;
    const uint32_t b = (c - theta) >> shift;
    return b < static_cast<uint32_t>(kHistBins - 1) ? static_cast<int>(b) : kHistBins - 1;
  }
};

// Histogram bin width for keys from theta up to khi: [theta, khi] spans fewer
// than kHistBins / 2 bins.
__device__ __forceinline__ int hist_shift(uint32_t theta, uint32_t khi) {
  const uint32_t d = khi > theta ? khi - theta : 0u;
  int sh = 0;
  while ((d >> sh) >= static_cast<uint32_t>(kHistBins / 2)) ++sh;
  return sh;
}

// Bin of the k-th largest candidate from the histogram, counted from the top
// bin down.  hb: this thread's bins, kHistBins / NT of them, in descending
// bin order starting at bin kHistBins - 1 - threadIdx.x * (kHistBins / NT).
// Returns false when the bins do not add up to M (the histogram is not
// usable); otherwise bstar is the bin holding rank k, krem how many of its
// entries complete the k largest, cnt its size.  All threads call.
template <int NT>
__device__ __forceinline__ bool hist_boundary(const uint32_t (&hb)[kHistBins / NT], int M, int k, BlockScratch<NT>& sc,
                              int& bstar, int& krem, int& cnt) {
  constexpr int BPT = kHistBins / NT;
  constexpr int NW = NT / 64;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int mine = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) mine += static_cast<int>(hb[i]);
  const int incl = wave_incl_scan(mine);
  if (lane == 63) sc.wsum[wave] = incl;
  __syncthreads();
  int above = incl - mine, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    total += sc.wsum[w];
    if (w < wave) above += sc.wsum[w];
  }
  if (total != M) {  // uniform: every thread read the same sums
    __syncthreads();
    return false;
  }
  if (above < k && k <= above + mine) {
    int cum = above;
    bool hit = false;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      const int c = static_cast<int>(hb[i]);
      if (!hit && cum + c >= k) {
        sc.found[0] = kHistBins - 1 - (t * BPT + i);
        sc.found[1] = k - cum;
        sc.found[2] = c;
        hit = true;
      }
      if (!hit) cum += c;
    }
  }
  __syncthreads();
  bstar = sc.found[0];
  krem = sc.found[1];
  cnt = sc.found[2];
  __syncthreads();  // sc.found is rewritten by the caller
  return true;
}

// Ranks the entries of the wave-held keys that satisfy `in` (cnt of them;
// at most kRankBin) by (key descending, position ascending) and returns the
// key and the position of the krem-th (rank krem - 1 among the entries).
// The entries equal to that key that are taken are exactly those at or
// before that position.  bl: LDS, >= kRankBin uint2.
//  * cnt <= 64 (the usual case): the entries go to bl in any order (each
//    carries its position), at slots taken from the counter sc.rank_n, which
//    must be 0 on entry; a step of the pass in which no lane of a wave holds
//    an entry costs that wave one ballot.  Then lane j of wave 0 takes entry
//    j and counts the entries ranked before it, reading the others from
//    their lanes (no LDS round trip per comparison).
//  * otherwise: a ballot count per wave, one slot reservation per wave and a
//    second pass that writes the entries; thread j < cnt compares entry j
//    with all of them from LDS.
constexpr int kRankBin = 256;
template <int NT, int PERW, class In>
__device__ __forceinline__ void rank_entries(const uint32_t (&key)[PERW], int lo, int hi, const In& in, int cnt,
                                             int krem, uint2* bl, BlockScratch<NT>& sc, uint32_t& kstar,
                                             int& cut) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (cnt <= 64) {  // uniform
#pragma unroll
    for (int u = 0; u < PERW; ++u) {
      const int p = lo + 64 * u + lane;
      const bool ok = p < hi && in(key[u]);
      if (__ballot(ok) != 0ull && ok) {
        const int slot = HST_DCLAMP(atomicAdd(&sc.rank_n, 1), 0, 63, kDbgRankSlot);
        bl[slot] = make_uint2(key[u], static_cast<uint32_t>(p));
      }
    }
    __syncthreads();
    if (wave == 0) {
      const uint2 me = lane < cnt ? bl[lane] : make_uint2(0u, 0xffffffffu);
      int bf[4] = {0, 0, 0, 0};  // four independent counts
      int j = 0;
      for (; j + 4 <= cnt; j += 4) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const uint32_t ok = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(me.x), j + x));
          const uint32_t op = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(me.y), j + x));
          bf[x] += (ok > me.x || (ok == me.x && op < me.y)) ? 1 : 0;
        }
      }
      for (; j < cnt; ++j) {
        const uint32_t ok = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(me.x), j));
        const uint32_t op = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(me.y), j));
        bf[0] += (ok > me.x || (ok == me.x && op < me.y)) ? 1 : 0;
      }
      if (lane < cnt && bf[0] + bf[1] + bf[2] + bf[3] == krem - 1) {
        sc.found[0] = static_cast<int>(me.x);
        sc.found[1] = static_cast<int>(me.y);
      }
    }
  } else {
    if (t == 0) sc.found[3] = 0;
    __syncthreads();
    {
      // this wave's entries, then one slot reservation per wave
      int nw = 0;
#pragma unroll
      for (int u = 0; u < PERW; ++u) nw += __popcll(__ballot(lo + 64 * u + lane < hi && in(key[u])));
      int base = 0;
      if (lane == 0 && nw > 0) base = atomicAdd(&sc.found[3], nw);
      base = __shfl(base, 0, 64);
#pragma unroll
      for (int u = 0; u < PERW; ++u) {
        const int p = lo + 64 * u + lane;
        const bool ok = p < hi && in(key[u]);
        const unsigned long long b = __ballot(ok);
        const int slot = base + lanes_below(b);
        if (ok && slot < kRankBin) bl[slot] = make_uint2(key[u], static_cast<uint32_t>(p));
        base += __popcll(b);
      }
    }
    __syncthreads();
    const int nb = cnt < kRankBin ? cnt : kRankBin;
    if (t < nb) {
      const uint2 me = bl[t];
      int gt = 0, eq = 0;
      // four entries per step, their loads issued together (an entry past the
      // end is read as the last one and not counted)
      for (int j0 = 0; j0 < nb; j0 += 4) {
        uint2 o[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) o[u] = bl[j0 + u < nb ? j0 + u : nb - 1];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (j0 + u < nb) {
            gt += o[u].x > me.x ? 1 : 0;
            eq += (o[u].x == me.x && o[u].y < me.y) ? 1 : 0;
          }
      }
      if (gt + eq == krem - 1) {  // the krem-th entry: its key and position
        sc.found[0] = static_cast<int>(me.x);
        sc.found[1] = static_cast<int>(me.y);
      }
    }
  }
  __syncthreads();
  kstar = static_cast<uint32_t>(sc.found[0]);
  cut = sc.found[1];
  __syncthreads();
}

// Stable compaction under the rule (mask, prefix, cut): the entry at
// position p with masked key m = key & mask is selected iff m > prefix, or
// m == prefix and p <= cut.  From ballots over the wave-held keys: writes the
// selected indices at output positions [r0, r1).
template <int NT, int PERW, class Idx>
__device__ __forceinline__ void compact_regs(const uint32_t (&key)[PERW], int lo, int hi, const Idx& candi,
                                             uint32_t mask, uint32_t prefix, int cut, int r0, int r1,
                                             int32_t* out_g, int32_t* out_l, BlockScratch<NT>& sc) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const auto taken = [&](int u) {
    const int p = lo + 64 * u + lane;
    const uint32_t m = key[u] & mask;
    return p < hi && (m > prefix || (m == prefix && p <= cut));
  };
  int selc = 0;
#pragma unroll
  for (int u = 0; u < PERW; ++u) selc += __popcll(__ballot(taken(u)));
  if (lane == 0) sc.red[0][wave] = static_cast<uint32_t>(selc);
  __syncthreads();
  int run = 0;
  {
    uint32_t g[NW];  // every wave's count, loads issued together
#pragma unroll
    for (int w = 0; w < NW; ++w) g[w] = sc.red[0][w];
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) run += static_cast<int>(g[w]);
  }
  __syncthreads();  // sc is reused by the caller
  // this wave's selected entries take positions [run, run + selc): a wave
  // whose range misses [r0, r1) writes nothing (uniform per wave)
  if (run >= r1 || run + selc <= r0) return;
#pragma unroll
  for (int u = 0; u < PERW; ++u) {
    if (run < r1) {  // uniform per wave: nothing past r1 is written
      const bool sel = taken(u);
      const unsigned long long selb = __ballot(sel);
      const int pos = run + lanes_below(selb);
      if (sel && pos >= r0 && pos < r1) {
        const int32_t v = static_cast<int32_t>(candi[lo + 64 * u + lane]);
        if (out_g != nullptr) out_g[pos] = v;
        if (out_l != nullptr) out_l[pos - r0] = v;
      }
      run += __popcll(selb);
    }
  }
}

// Position (in index order) of the krem-th entry among those whose masked
// key equals prefix (-1 when krem is 0); the wave-held keys as
// select_rule_core holds them.  All threads call.
template <int NT, int PERW>
__device__ __forceinline__ int rule_cut_position(const uint32_t (&key)[PERW], int lo, int hi, uint32_t mask,
                                                 uint32_t prefix, int krem, BlockScratch<NT>& sc) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (krem <= 0) return -1;  // uniform
  int eqc = 0;
#pragma unroll
  for (int u = 0; u < PERW; ++u)
    eqc += __popcll(__ballot(lo + 64 * u + lane < hi && (key[u] & mask) == prefix));
  if (lane == 0) sc.red[1][wave] = static_cast<uint32_t>(eqc);
  __syncthreads();
  int before = 0;
  {
    uint32_t e[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) e[w] = sc.red[1][w];
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) before += static_cast<int>(e[w]);
  }
  if (before < krem && krem <= before + eqc) {  // this wave holds the krem-th
    int run = before;
#pragma unroll
    for (int u = 0; u < PERW; ++u) {
      const int p = lo + 64 * u + lane;
      const bool eq = p < hi && (key[u] & mask) == prefix;
      const unsigned long long b = __ballot(eq);
      const int n = __popcll(b);
      if (run < krem && krem <= run + n && eq && run + lanes_below(b) == krem - 1) sc.found[0] = p;
      run += n;
    }
  }
  __syncthreads();
  const int cut = sc.found[0];
  __syncthreads();  // sc is reused by the caller
  return cut;
}

// The exact top-k rule over M <= NT * PERW candidates held in LDS in index
// order, as (mask, prefix, cut): the entry at position p with masked key
// m = key & mask is among the k first in the order (key descending, position
// ascending) iff m > prefix, or m == prefix and p <= cut.  The keys are left
// in registers: wave w holds positions [lo, hi) (lane l's entry u at
// lo + 64u + l), the order a compaction walks them in.
//  * With a binning from the head's threshold (HIST): the keys go into an LDS
//    histogram as they are loaded, one block scan over the bins finds the bin
//    of the k-th key, and the rule follows at once when that bin is taken
//    whole; otherwise the bin's entries (at most kRankBin) are ranked
//    directly, which gives the k-th key and its position.  A bin of one key
//    value (shift 0) needs only the position of its kb-th entry.
//  * Otherwise, or when the bin is too full: radix passes of up to 11 bits
//    below the keys' common prefix narrow the bin of the k-th largest key
//    until it holds at most kRankBin entries, which are then ranked.
// hist: 2048 words of LDS.
template <int NT, int PERW, bool HIST>
__device__ __forceinline__ void select_rule_core(const uint32_t* candk, int M, int k, uint32_t* hist,
                                                 BlockScratch<NT>& sc, const HistInfo& hi_info,
                                                 uint32_t (&key)[PERW], int& lo, int& hi, uint32_t& mask,
                                                 uint32_t& prefix, int& cut) {
  constexpr int NW = NT / 64;
  constexpr int MAXPER = (2048 + NT - 1) / NT;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int span = ((M + NW - 1) / NW + 63) & ~63;
  lo = min(M, wave * span);
  hi = min(M, lo + span);
  mask = 0u;
  prefix = 0u;
  cut = 0x7fffffff;
  if (t == 0) sc.rank_n = 0;  // read only after the barriers below
  bool done = k >= M;  // every entry taken
  if (HIST && !done && hi_info.ok) {
    constexpr int BPT = kHistBins / NT;
    for (int i = t; i < kHistBins; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PERW; ++u) {
      const int p = lo + 64 * u + lane;
      key[u] = p < hi ? candk[p] : 0u;
      if (p < hi) atomicAdd(&hist[hi_info.bin(key[u])], 1u);
    }
    __syncthreads();
    uint32_t hb[BPT];  // this thread's bins, from the top bin down
#pragma unroll
    for (int i = 0; i < BPT; ++i) hb[i] = hist[kHistBins - 1 - (t * BPT + i)];
    int bstar, kb, cnt;
    if (hist_boundary<NT>(hb, M, k, sc, bstar, kb, cnt) && bstar >= 1) {
      const uint32_t th = hi_info.theta;
      const int sh = hi_info.shift;
      const unsigned long long klo = static_cast<unsigned long long>(th) +
                                     (static_cast<unsigned long long>(bstar) << sh);
      if (kb == cnt && klo <= 0xffffffffull) {
        // the whole bin is taken: every key >= its lower edge
        mask = 0xffffffffu;
        prefix = static_cast<uint32_t>(klo - 1ull);
        cut = -1;
        done = true;
      } else if (sh == 0 && bstar < kHistBins - 1) {
        // the bin is one key value: its first kb entries in index order
        mask = 0xffffffffu;
        prefix = static_cast<uint32_t>(klo);
        cut = rule_cut_position<NT, PERW>(key, lo, hi, mask, prefix, kb, sc);
        done = true;
      } else if (cnt <= kRankBin) {
        const HistInfo hh = hi_info;
        const auto in_bin = [hh, bstar](uint32_t c) { return hh.bin(c) == bstar; };
        rank_entries<NT, PERW>(key, lo, hi, in_bin, cnt, kb, reinterpret_cast<uint2*>(hist), sc, prefix, cut);
        mask = 0xffffffffu;
        done = true;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < PERW; ++u) {
      const int p = lo + 64 * u + lane;
      key[u] = p < hi ? candk[p] : 0u;
    }
  }
  if (!done) {
    int krem = k;
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int u = 0; u < PERW; ++u)
      if (lo + 64 * u + lane < hi) {
        mn = min(mn, key[u]);
        mx = max(mx, key[u]);
      }
    block_minmax<NT>(mn, mx, sc);
    bool resolved = false;
    if (mn != mx) {
      const int hb_ = 31 - __clz(static_cast<int>(mn ^ mx));
      mask = hb_ == 31 ? 0u : ~((1u << (hb_ + 1)) - 1u);
      prefix = mn & mask;
      int lob = hb_ + 1;
      while (lob > 0) {
        const int width = lob < 11 ? lob : 11;
        const int sh = lob - width;
        const int nb = 1 << width;
        const uint32_t dm = static_cast<uint32_t>(nb - 1);
        for (int i = t; i < nb; i += NT) hist[i] = 0u;
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
        __syncthreads();  // every thread has read sc.found and its bins
        if (cnt == krem) {  // the whole bin is taken
          cut = 0x7fffffff;
          resolved = true;
          break;
        }
        if (lob == 0) break;  // every bit is resolved: the first krem equal keys
        if (cnt <= kRankBin) {
          const uint32_t pm = mask, pp = prefix;
          rank_entries<NT, PERW>(key, lo, hi, [pm, pp](uint32_t c) { return (c & pm) == pp; }, cnt, krem,
                                 reinterpret_cast<uint2*>(hist), sc, prefix, cut);
          mask = 0xffffffffu;
          resolved = true;
          break;
        }
      }
    }
    // all keys equal, or every bit resolved: the first krem equal keys
    if (!resolved) cut = rule_cut_position<NT, PERW>(key, lo, hi, mask, prefix, krem, sc);
  }
  __syncthreads();  // sc.found is read above; sc.red may be written next
}

// Exact selection over M <= NT * PERW candidates held in LDS in index order:
// the rule of select_rule_core, then the stable compaction of compact_regs,
// which writes the selected indices at output positions [r0, r1).
template <int NT, int PERW, class Idx, bool HIST>
__device__ void select_lds_core(const uint32_t* candk, const Idx& candi, int M, int k, int r0, int r1,
                                int32_t* out_g, int32_t* out_l, uint32_t* hist, BlockScratch<NT>& sc,
                                const HistInfo& hi_info) {
  uint32_t key[PERW], mask, prefix;
  int lo, hi, cut;
  select_rule_core<NT, PERW, HIST>(candk, M, k, hist, sc, hi_info, key, lo, hi, mask, prefix, cut);
  compact_regs<NT, PERW>(key, lo, hi, candi, mask, prefix, cut, r0, r1, out_g, out_l, sc);
}

template <int NT, int PERW, class Idx>
__device__ void select_lds_regs(const uint32_t* candk, const Idx& candi, int M, int k, int r0, int r1,
                                int32_t* out_g, int32_t* out_l, uint32_t* hist, BlockScratch<NT>& sc) {
  select_lds_core<NT, PERW, Idx, false>(candk, candi, M, k, r0, r1, out_g, out_l, hist, sc,
                                        HistInfo{0u, 0, false});
}

// Lower bound of the r-th largest (1 <= r <= count) of the keys held PER per
// thread: two 11-bit radix passes below the common prefix of the keys, then
// the low edge of the bin holding rank r (the common key if all are equal).
// kmax (optional) receives the largest key.
template <int NT, int PER>
__device__ uint32_t rank_lower_bound_regs(const uint32_t (&key)[PER], int count, int r, uint32_t* hist,
                                          BlockScratch<NT>& sc, uint32_t* kmax = nullptr) {
  uint32_t mask, prefix, kmin;
  int krem;
  radix_select_regs<NT, PER>(key, count, r, 2, hist, sc, mask, prefix, krem, &kmin, kmax);
  return mask == 0u ? kmin : prefix;
}

struct SelectScratch {
  uint32_t* candk;  // LDS, kSelCap entries
  int32_t* candi;   // LDS, kSelCap entries
  uint32_t* hist;   // LDS, 2048 words
  int* offs;        // LDS, nchunks + 1
};

// Keys rescored from the metadata, for the rare selection over every key
// (fewer than k keys passed the threshold): the soft-collision score of key
// i from the query tables in the workspace, or its code similarity.  These
// scores may differ from the scan's in the last bit (the lookups are summed
// in table order); the selection is exact for them.
struct SoftRescoreSrc {
  const uint8_t* ids;  // the head's rows [n][L]
  const void* vn;      // the head's value norms
  const float* tbl;    // the head's table, bucket-major [2^P][L]
  int L;
  uint32_t idmask;
  bool f16;
  __device__ __forceinline__ uint32_t key(int i) const {
    const uint8_t* r = ids + static_cast<long long>(i) * L;
    float acc = 0.f;
    for (int l = 0; l < L; ++l) acc += tbl[(r[l] & idmask) * L + l];
    const float v = f16 ? f16_bits_to_f32(static_cast<const uint16_t*>(vn)[i]) : static_cast<const float*>(vn)[i];
    return order_key_f32(acc * v);
  }
  __device__ __forceinline__ int32_t idx(int i) const { return i; }
};
struct HamRescoreSrc {
  const uint32_t* codes;  // the head's codes [n][4]
  const uint32_t* qc;     // the head's G query codes [G][4]
  int G;
  __device__ __forceinline__ uint32_t key(int i) const {
    const uint32_t* c = codes + static_cast<long long>(i) * 4;
    int ham = 0;
    for (int g = 0; g < G; ++g)
      ham += __popc(c[0] ^ qc[4 * g]) + __popc(c[1] ^ qc[4 * g + 1]) + __popc(c[2] ^ qc[4 * g + 2]) +
             __popc(c[3] ^ qc[4 * g + 3]);
    return order_key_i32(128 * G - ham);
  }
  __device__ __forceinline__ int32_t idx(int i) const { return i; }
};

template <int NT, class Src>
__device__ void select_all_keys(const Src& src, int n, int k_eff, int r0, int r1, int32_t* out_g,
                                int32_t* out_l, uint32_t* hist, BlockScratch<NT>& sc) {
  const SelRule rule = block_select_rule<NT>(src, n, k_eff, hist, sc);
  block_compact_range<NT>(src, n, rule, r0, r1, out_g, out_l, sc);
}

// The head's candidate slots as one array in index order: the chunk offsets
// go to ws.offs (nch + 1 entries) and, when k_need <= M <= kSelCap (M the
// candidate count, returned), the candidates to ws.candk / ws.candi.  Ends
// with a barrier.  All threads call.
template <int NT>
__device__ __forceinline__ int candidates_to_lds(const FusedArgs& a, int bh, int n, int chunk, int k_need,
                                 const SelectScratch& ws, BlockScratch<NT>& sc) {
  const int nch = (n + a.span - 1) / a.span;  // chunk c: keys [c*span, (c+1)*span), slots at c*chunk
  const uint32_t* cnt = a.counts + static_cast<long long>(bh) * a.nchunks;
  const uint2* slots = a.slots + static_cast<long long>(bh) * a.nchunks * chunk;
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // the first counts, then the first 64*PX slots of the first eight chunks
  // of each wave (copied below), all in flight together: the slot addresses
  // do not depend on the counts (slots past a chunk's count are read,
  // unused), and the counts, issued first, arrive without waiting for the
  // slots
  constexpr int PX = NT >= 1024 ? 2 : 3;  // (1024-thread workgroups hold 128 VGPRs)
  // (the loads are bounded by the workspace's chunk count, not by nch, so
  // they do not wait for the sequence length; entries past nch are unused)
  const int cnt_ld = static_cast<int>(threadIdx.x) < a.nchunks ? static_cast<int>(cnt[threadIdx.x]) : 0;
  const int cnt0 = static_cast<int>(threadIdx.x) < nch ? cnt_ld : 0;
  // (chunk indices clamped, so the loads are unconditional)
  uint2 pre[8][PX];
  const int clast = a.nchunks > 0 ? a.nchunks - 1 : 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = min(wave + u * NW, clast);
#pragma unroll
    for (int x = 0; x < PX; ++x) pre[u][x] = slots[static_cast<long long>(c) * chunk + lane + 64 * x];
  }
  int run = 0;
  for (int c0 = 0; c0 < nch; c0 += NT) {
    const int c = c0 + static_cast<int>(threadIdx.x);
    const int v = c0 == 0 ? cnt0 : (c < nch ? static_cast<int>(cnt[c]) : 0);
    HST_DCHECK(v <= chunk, kDbgChunkCount);
    int tot;
    const int x = block_excl_scan<NT>(v, sc, tot);
    if (c < nch) ws.offs[c] = run + x;
    run += tot;
  }
  if (threadIdx.x == 0) ws.offs[nch] = run;
  __syncthreads();
  const int M = run;
  if (M >= k_need && M <= kSelCap) {
    // each wave copies whole chunks (coalesced): eight chunks and 8*PX
    // loads per lane in flight (the first eight chunks already loaded)
    for (int c0 = wave; c0 < nch; c0 += NW * 8) {
      uint2 v[8][PX];
      int cn[8], base[8];
      int cmax = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u * NW;
        cn[u] = c < nch ? ws.offs[c + 1] - ws.offs[c] : 0;
        base[u] = c < nch ? ws.offs[c] : 0;
        cmax = max(cmax, cn[u]);
#pragma unroll
        for (int x = 0; x < PX; ++x) {
          if (c0 == wave) v[u][x] = pre[u][x];
          else if (lane + 64 * x < cn[u]) v[u][x] = slots[static_cast<long long>(c) * chunk + lane + 64 * x];
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        HST_DCHECK(base[u] + cn[u] <= kSelCap, kDbgCandLds);
#pragma unroll
        for (int x = 0; x < PX; ++x)
          if (lane + 64 * x < cn[u]) {
            ws.candk[base[u] + lane + 64 * x] = v[u][x].x;
            ws.candi[base[u] + lane + 64 * x] = static_cast<int32_t>(v[u][x].y);
          }
        if constexpr (NT >= 1024) {  // chunks with more candidates, one by one (registers)
          const long long c = c0 + u * NW;
          for (int i = 64 * PX + lane; i < cn[u]; i += 64) {
            const uint2 w = slots[c * chunk + i];
            ws.candk[base[u] + i] = w.x;
            ws.candi[base[u] + i] = static_cast<int32_t>(w.y);
          }
        }
      }
      if constexpr (NT < 1024) {
        // chunks with more candidates: the next 64 of all eight chunks per
        // round trip (cmax is the same in every lane of the wave)
        for (int i0 = 64 * PX; i0 < cmax; i0 += 64) {
          uint2 w[8];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (i0 + lane < cn[u]) w[u] = slots[static_cast<long long>(c0 + u * NW) * chunk + i0 + lane];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (i0 + lane < cn[u]) {
              ws.candk[base[u] + i0 + lane] = w[u].x;
              ws.candi[base[u] + i0 + lane] = static_cast<int32_t>(w[u].y);
            }
        }
      }
    }
  }
  __syncthreads();
  return M;
}

// The head's exact top-k (k_eff keys, ties to the lower index) from the M
// candidates candidates_to_lds prepared.  Writes the selected indices at
// output positions [r0, r1) and -1 at positions in [max(r0, k_eff), r1) of
// out_g.  h_theta and h_shift are the head's threshold and histogram shift
// (read by the caller ahead of its own loads).  Returns the selection path
// taken:
//   0: candidates in LDS (a histogram over a binning from the head's
//      threshold gives the bin of the k-th key; radix passes only when it
//      cannot);
//   1: more candidates than LDS holds: selected from the slots in HBM;
//   2: fewer than k_eff keys passed the threshold: every key, from the given
//      score row (scores_row) or rescored from the metadata (a.meta).
template <int NT>
__device__ __forceinline__ int select_from_candidates(const FusedArgs& a, int bh, int n, int k_eff, int chunk, int M,
                                      uint32_t h_theta, uint32_t h_shift, const void* scores_row,
                                      bool scores_int, const SelectScratch& ws, int r0, int r1,
                                      int32_t* out_g, int32_t* out_l, BlockScratch<NT>& sc) {
  const int nch = (n + a.span - 1) / a.span;
  const uint2* slots = a.slots + static_cast<long long>(bh) * a.nchunks * chunk;
  int path = 0;
  if (k_eff > 0) {
    if (M >= k_eff && M <= kSelCap) {
      const HistInfo hi{h_theta, static_cast<int>(h_shift), h_shift < 32u};
      select_lds_core<NT, kSelCap / NT, const int32_t*, true>(ws.candk, ws.candi, M, k_eff, r0, r1, out_g,
                                                              out_l, ws.hist, sc, hi);
    } else if (M >= k_eff) {
      path = 1;
      const SlotSrc src{slots, ws.offs, nch, chunk};
      const SelRule rule = block_select_rule<NT>(src, M, k_eff, ws.hist, sc);
      block_compact_range<NT>(src, M, rule, r0, r1, out_g, out_l, sc);
    } else {
      path = 2;  // the sample overestimated the threshold: use every key
      const long long base = static_cast<long long>(bh) * a.Nmax;
      if (scores_row != nullptr && scores_int) {
        select_all_keys<NT>(I32RowSrc{static_cast<const int32_t*>(scores_row)}, n, k_eff, r0, r1, out_g, out_l,
                            ws.hist, sc);
      } else if (scores_row != nullptr) {
        select_all_keys<NT>(F32RowSrc{static_cast<const float*>(scores_row)}, n, k_eff, r0, r1, out_g, out_l,
                            ws.hist, sc);
      } else if (a.meta_kind == kScanHamming) {
        const int G = a.Hq / a.Hkv;
        const HamRescoreSrc src{static_cast<const uint32_t*>(a.meta) + base * 4,
                                a.qcodes + static_cast<long long>(bh) * G * 4, G};
        select_all_keys<NT>(src, n, k_eff, r0, r1, out_g, out_l, ws.hist, sc);
      } else {
        const bool f16 = a.meta_f16 != 0;
        const char* vnb = static_cast<const char*>(a.meta_vn) + base * (f16 ? 2 : 4);
        const SoftRescoreSrc src{static_cast<const uint8_t*>(a.meta) + base * a.L, vnb,
                                 a.tables + static_cast<long long>(bh) * (static_cast<long long>(a.L) << a.P),
                                 a.L, (1u << a.P) - 1u, f16};
        select_all_keys<NT>(src, n, k_eff, r0, r1, out_g, out_l, ws.hist, sc);
      }
    }
  }
  if (out_g != nullptr)
    for (int p = max(r0, k_eff) + static_cast<int>(threadIdx.x); p < r1; p += NT) out_g[p] = -1;
  __syncthreads();
  return path;
}

template <int NT>
__device__ int select_range(const FusedArgs& a, int bh, int n, int k_eff, int chunk,
                            const void* scores_row, bool scores_int, const SelectScratch& ws,
                            int r0, int r1, int32_t* out_g, int32_t* out_l, BlockScratch<NT>& sc,
                            int* cand_total) {
  const HeadState& hs = a.heads[bh];
  const uint32_t h_theta = hs.theta, h_shift = hs.shift;
  const int M = candidates_to_lds<NT>(a, bh, n, chunk, k_eff, ws, sc);
  *cand_total = M;
  return select_from_candidates<NT>(a, bh, n, k_eff, chunk, M, h_theta, h_shift, scores_row, scores_int, ws,
                                    r0, r1, out_g, out_l, sc);
}

}  // namespace hst
