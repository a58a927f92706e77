// Deterministic top-k per (sequence, kv head): the k keys first in the order
// (score descending, index ascending), written in ascending index order.
// SOCKET overview page, "Core mechanism: soft LSH", item 4 (top-k chosen
// deterministically from the soft scores).
//
// Exact radix selection on order-preserving 32-bit keys, spread over many
// workgroups per head:
//   init    - per-head state, histogram cleared, idx rows set to -1
//   minmax  - the key range; bits shared by every key need no pass
//   plan    - start below the highest bit in which min and max differ
//   hist/pick (at most 3 rounds of 11 bits) - narrow the threshold digit by
//             digit until the threshold bin is taken whole or every bit is
//             fixed; afterwards `prefix`/`mask` describe the threshold T and
//             `krem` how many keys equal to T (lowest indices first) are kept
//   count   - per chunk: keys above T and keys equal to T
//   write   - ordered compaction with a prefix over the preceding chunks
#include "hst_common.h"
#include "hst_launch.h"

namespace hst {

constexpr int kSelChunk = 4096;   // keys per workgroup
constexpr int kSelBits = 11;      // radix digit width
constexpr int kSelBins = 1 << kSelBits;

struct SelState {
  uint32_t prefix;   // fixed high bits of the threshold
  uint32_t mask;     // which bits are fixed
  int32_t krem;      // keys still to take among those equal to prefix under mask
  int32_t lo;        // bits [0, lo) are not fixed yet
  int32_t done;
  int32_t n;         // N_b
  int32_t keff;      // number of keys to select
  uint32_t umin;
  uint32_t umax;
  int32_t pad[7];
};
static_assert(sizeof(SelState) == 64, "state stride");

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t order_key(int32_t v) {
  return static_cast<uint32_t>(v) ^ 0x80000000u;
}

__global__ void __launch_bounds__(256)
sel_init_kernel(SelState* __restrict__ st, uint32_t* __restrict__ hist,
                const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ k_per_seq,
                int Hkv, int Nmax, int kcap, int32_t* __restrict__ idx) {
  const int head = blockIdx.x;
  const int b = head / Hkv;
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x)
    hist[static_cast<long long>(head) * kSelBins + i] = 0u;
  for (int i = threadIdx.x; i < kcap; i += blockDim.x)
    idx[static_cast<long long>(head) * kcap + i] = -1;
  if (threadIdx.x == 0) {
    const int n = seq_len(seq_lens, b, Nmax);
    int k = kcap;
    if (k_per_seq != nullptr) {
      const int kb = k_per_seq[b];
      k = kb < 0 ? 0 : (kb < kcap ? kb : kcap);
    }
    if (k > n) k = n;
    SelState s;
    s.prefix = 0u;
    s.mask = 0u;
    s.krem = k;
    s.lo = 32;
    s.done = 0;
    s.n = n;
    s.keff = k;
    s.umin = 0xffffffffu;
    s.umax = 0u;
    for (int i = 0; i < 7; ++i) s.pad[i] = 0;
    st[head] = s;
  }
}

template <typename KT>
__global__ void __launch_bounds__(256)
sel_minmax_kernel(const KT* __restrict__ scores, SelState* __restrict__ st, int Nmax) {
  const int head = blockIdx.y;
  const int n = st[head].n;
  const int j0 = blockIdx.x * kSelChunk;
  if (j0 >= n) return;
  const int jend = min(j0 + kSelChunk, n);
  const KT* row = scores + static_cast<long long>(head) * Nmax;
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int j = j0 + threadIdx.x; j < jend; j += blockDim.x) {
    const uint32_t u = order_key(row[j]);
    mn = min(mn, u);
    mx = max(mx, u);
  }
  for (int m = 32; m >= 1; m >>= 1) {
    mn = min(mn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mn), m, 64)));
    mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), m, 64)));
  }
  if ((threadIdx.x & 63) == 0) {
    atomicMin(&st[head].umin, mn);
    atomicMax(&st[head].umax, mx);
  }
}

__global__ void sel_plan_kernel(SelState* __restrict__ st) {
  const int head = blockIdx.x * blockDim.x + threadIdx.x;
  if (head >= static_cast<int>(gridDim.x * blockDim.x)) return;
  SelState s = st[head];
  if (s.keff == 0 || s.keff == s.n || s.umin == s.umax) {
    // nothing to rank: take the first keff keys (all of them are "equal")
    s.mask = 0u;
    s.prefix = 0u;
    s.krem = s.keff;
    s.lo = 0;
    s.done = 1;
  } else {
    const int hb = 31 - __clz(static_cast<int>(s.umin ^ s.umax));
    s.mask = hb == 31 ? 0u : ~((1u << (hb + 1)) - 1u);
    s.prefix = s.umin & s.mask;
    s.krem = s.keff;
    s.lo = hb + 1;
    s.done = 0;
  }
  st[head] = s;
}

template <typename KT>
__global__ void __launch_bounds__(256)
sel_hist_kernel(const KT* __restrict__ scores, const SelState* __restrict__ st,
                uint32_t* __restrict__ hist, int Nmax) {
  __shared__ uint32_t lh[kSelBins];
  const int head = blockIdx.y;
  const SelState s = st[head];
  if (s.done) return;
  const int j0 = blockIdx.x * kSelChunk;
  if (j0 >= s.n) return;
  const int width = s.lo < kSelBits ? s.lo : kSelBits;
  const int sh = s.lo - width;
  const uint32_t dmask = (1u << width) - 1u;
  for (int i = threadIdx.x; i < kSelBins; i += blockDim.x) lh[i] = 0u;
  __syncthreads();
  const int jend = min(j0 + kSelChunk, s.n);
  const KT* row = scores + static_cast<long long>(head) * Nmax;
  for (int j = j0 + threadIdx.x; j < jend; j += blockDim.x) {
    const uint32_t u = order_key(row[j]);
    if ((u & s.mask) == s.prefix) atomicAdd(&lh[(u >> sh) & dmask], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i <= static_cast<int>(dmask); i += blockDim.x)
    if (lh[i]) atomicAdd(&hist[static_cast<long long>(head) * kSelBins + i], lh[i]);
}

// One block per head: find the digit holding the krem-th largest key.
__global__ void __launch_bounds__(256)
sel_pick_kernel(SelState* __restrict__ st, uint32_t* __restrict__ hist) {
  __shared__ uint32_t part[256];
  const int head = blockIdx.x;
  SelState s = st[head];
  if (s.done) return;
  const int width = s.lo < kSelBits ? s.lo : kSelBits;
  const int sh = s.lo - width;
  const int nbins = 1 << width;
  uint32_t* hh = hist + static_cast<long long>(head) * kSelBins;
  // thread t owns bins [t*per, (t+1)*per) counted from the top digit down
  const int per = (nbins + 255) / 256;
  const int t = threadIdx.x;
  uint32_t mine = 0;
  for (int i = 0; i < per; ++i) {
    const int r = t * per + i;  // rank from the top
    if (r < nbins) mine += hh[nbins - 1 - r];
  }
  part[t] = mine;
  __syncthreads();
  // inclusive scan over threads (Hillis-Steele, 256 entries)
  for (int off = 1; off < 256; off <<= 1) {
    uint32_t v = t >= off ? part[t - off] : 0u;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  const uint32_t above = t > 0 ? part[t - 1] : 0u;
  const uint32_t need = static_cast<uint32_t>(s.krem);
  if (above < need && need <= above + mine) {
    uint32_t cum = above;
    for (int i = 0; i < per; ++i) {
      const int r = t * per + i;
      if (r >= nbins) break;
      const int digit = nbins - 1 - r;
      const uint32_t c = hh[digit];
      if (cum + c >= need) {
        s.krem = static_cast<int>(need - cum);
        s.prefix |= static_cast<uint32_t>(digit) << sh;
        s.mask |= static_cast<uint32_t>(nbins - 1) << sh;
        s.lo = sh;
        s.done = (static_cast<uint32_t>(s.krem) == c || sh == 0) ? 1 : 0;
        st[head] = s;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  for (int i = t; i < kSelBins; i += 256) hh[i] = 0u;
}

template <typename KT>
__global__ void __launch_bounds__(256)
sel_count_kernel(const KT* __restrict__ scores, const SelState* __restrict__ st,
                 int2* __restrict__ cnt, int nchunks, int Nmax) {
  __shared__ int red[2][4];
  const int head = blockIdx.y;
  const SelState s = st[head];
  const int j0 = blockIdx.x * kSelChunk;
  const int jend = min(j0 + kSelChunk, s.n);
  const KT* row = scores + static_cast<long long>(head) * Nmax;
  int gt = 0, eq = 0;
  for (int j = j0 + threadIdx.x; j < jend; j += blockDim.x) {
    const uint32_t m = order_key(row[j]) & s.mask;
    gt += m > s.prefix;
    eq += m == s.prefix;
  }
  for (int o = 32; o >= 1; o >>= 1) {
    gt += __shfl_xor(gt, o, 64);
    eq += __shfl_xor(eq, o, 64);
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][w] = gt;
    red[1][w] = eq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int g = 0, e = 0;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) {
      g += red[0][i];
      e += red[1][i];
    }
    cnt[static_cast<long long>(head) * nchunks + blockIdx.x] = make_int2(g, e);
  }
}

template <typename KT>
__global__ void __launch_bounds__(256)
sel_write_kernel(const KT* __restrict__ scores, const SelState* __restrict__ st,
                 const int2* __restrict__ cnt, int nchunks, int Nmax, int kcap,
                 int32_t* __restrict__ idx) {
  __shared__ int wsum[2][4];
  __shared__ int base[2];
  const int head = blockIdx.y;
  const SelState s = st[head];
  const int j0 = blockIdx.x * kSelChunk;
  if (j0 >= s.n || s.keff == 0) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // selected keys and equal keys in the chunks before this one
  int gtb = 0, eqb = 0;
  for (int c = threadIdx.x; c < static_cast<int>(blockIdx.x); c += blockDim.x) {
    const int2 v = cnt[static_cast<long long>(head) * nchunks + c];
    gtb += v.x;
    eqb += v.y;
  }
  for (int o = 32; o >= 1; o >>= 1) {
    gtb += __shfl_xor(gtb, o, 64);
    eqb += __shfl_xor(eqb, o, 64);
  }
  if (lane == 0) {
    wsum[0][w] = gtb;
    wsum[1][w] = eqb;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int g = 0, e = 0;
    for (int i = 0; i < 4; ++i) {
      g += wsum[0][i];
      e += wsum[1][i];
    }
    base[0] = g + min(e, s.krem);  // output slot of this chunk's first selected key
    base[1] = e;                   // equal keys before this chunk
  }
  __syncthreads();
  int out_pos = base[0];
  int eq_rank = base[1];
  const int jend = min(j0 + kSelChunk, s.n);
  const KT* row = scores + static_cast<long long>(head) * Nmax;
  int32_t* orow = idx + static_cast<long long>(head) * kcap;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int jt = j0; jt < jend; jt += blockDim.x) {
    const int j = jt + threadIdx.x;
    bool gt = false, eq = false;
    if (j < jend) {
      const uint32_t m = order_key(row[j]) & s.mask;
      gt = m > s.prefix;
      eq = m == s.prefix;
    }
    const unsigned long long beq = __ballot(eq);
    __syncthreads();  // wsum reuse
    if (lane == 0) wsum[1][w] = __popcll(beq);
    __syncthreads();
    int eq_off = eq_rank;
    int eq_tot = 0;
    for (int i = 0; i < 4; ++i) {
      if (i < w) eq_off += wsum[1][i];
      eq_tot += wsum[1][i];
    }
    const int my_eq_rank = eq_off + __popcll(beq & below);
    const bool sel = gt || (eq && my_eq_rank < s.krem);
    const unsigned long long bsel = __ballot(sel);
    if (lane == 0) wsum[0][w] = __popcll(bsel);
    __syncthreads();
    int sel_off = out_pos;
    int sel_tot = 0;
    for (int i = 0; i < 4; ++i) {
      if (i < w) sel_off += wsum[0][i];
      sel_tot += wsum[0][i];
    }
    if (sel) {
      const int pos = sel_off + __popcll(bsel & below);
      if (pos < kcap) orow[pos] = j;
    }
    out_pos += sel_tot;
    eq_rank += eq_tot;
  }
}

size_t select_ws_bytes(const hst_shape& s) {
  const size_t nheads = static_cast<size_t>(s.B) * s.Hkv;
  const size_t nchunks = (static_cast<size_t>(s.Nmax) + kSelChunk - 1) / kSelChunk;
  return nheads * sizeof(SelState) + nheads * kSelBins * sizeof(uint32_t) +
         nheads * nchunks * sizeof(int2) + 256;
}

template <typename KT>
static hipError_t launch_select_t(const hst_shape& s, const KT* scores, int kcap,
                                  const int32_t* k_per_seq, int32_t* idx, void* ws,
                                  hipStream_t stm) {
  const int nheads = s.B * s.Hkv;
  const int nchunks = (s.Nmax + kSelChunk - 1) / kSelChunk;
  char* p = static_cast<char*>(ws);
  SelState* st = reinterpret_cast<SelState*>(p);
  p += static_cast<size_t>(nheads) * sizeof(SelState);
  uint32_t* hist = reinterpret_cast<uint32_t*>(p);
  p += static_cast<size_t>(nheads) * kSelBins * sizeof(uint32_t);
  int2* cnt = reinterpret_cast<int2*>(p);
  dim3 gch(nchunks, nheads);
  hipLaunchKernelGGL(sel_init_kernel, dim3(nheads), dim3(256), 0, stm, st, hist, s.seq_lens,
                     k_per_seq, s.Hkv, s.Nmax, kcap, idx);
  hipLaunchKernelGGL(sel_minmax_kernel<KT>, gch, dim3(256), 0, stm, scores, st, s.Nmax);
  hipLaunchKernelGGL(sel_plan_kernel, dim3(nheads), dim3(1), 0, stm, st);
  for (int pass = 0; pass < 3; ++pass) {
    hipLaunchKernelGGL(sel_hist_kernel<KT>, gch, dim3(256), 0, stm, scores, st, hist, s.Nmax);
    hipLaunchKernelGGL(sel_pick_kernel, dim3(nheads), dim3(256), 0, stm, st, hist);
  }
  hipLaunchKernelGGL(sel_count_kernel<KT>, gch, dim3(256), 0, stm, scores, st, cnt, nchunks,
                     s.Nmax);
  hipLaunchKernelGGL(sel_write_kernel<KT>, gch, dim3(256), 0, stm, scores, st, cnt, nchunks,
                     s.Nmax, kcap, idx);
  return hipGetLastError();
}

hipError_t launch_select(const hst_shape& s, int score_dtype, const void* scores, int kcap,
                         const int32_t* k_per_seq, int32_t* idx, void* ws, hipStream_t st) {
  if (score_dtype == HST_F32)
    return launch_select_t(s, static_cast<const float*>(scores), kcap, k_per_seq, idx, ws, st);
  return launch_select_t(s, static_cast<const int32_t*>(scores), kcap, k_per_seq, idx, ws, st);
}

}  // namespace hst
