// Block-wide building blocks of the exact top-k: scans, reductions, a radix
// threshold search over (key, index) entries in array order, and the stable
// compaction that writes the selected indices in that order.
//
// Keys are order-preserving 32-bit images of the scores (larger key = larger
// score); ties are broken toward the earlier array position, which is the
// lower key index wherever the entries are stored in index order.
#pragma once

#include "hst_common.h"

namespace hst {

__device__ __forceinline__ uint32_t order_key_f32(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks as +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint32_t order_key_i32(int32_t v) {
  return static_cast<uint32_t>(v) ^ 0x80000000u;
}

// Scratch a block needs for the helpers below (in LDS).
template <int NT>
struct BlockScratch {
  int wsum[NT / 64 + 2];
  uint32_t red[2][NT / 64];
  int found[4];
  int rank_n;  // entries collected by a rank (zeroed by the selection that uses it)
};

// Inclusive prefix sum over the 64 lanes of a wave, in DPP moves (no LDS
// crossbar): shifts by 1, 2, 4 and 8 inside each row of 16 lanes (lanes
// shifted in from outside the row add 0), then the last lane of row 0 (2) is
// added to row 1 (3), and lane 31 to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive scan of one int per thread, block wide.  All threads must call.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, BlockScratch<NT>& sc, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int x = wave_incl_scan(v);
  if (lane == 63) sc.wsum[w] = x;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int s = sc.wsum[i];
    tot += s;
    if (i < w) before += s;
  }
  total = tot;
  __syncthreads();  // sc.wsum is reused by the next call
  return before + x - v;
}

template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, BlockScratch<NT>& sc) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    mn = min(mn, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mn), o, 64)));
    mx = max(mx, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mx), o, 64)));
  }
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sc.red[0][w] = mn;
    sc.red[1][w] = mx;
  }
  __syncthreads();
  mn = sc.red[0][0];
  mx = sc.red[1][0];
  for (int i = 1; i < NT / 64; ++i) {
    mn = min(mn, sc.red[0][i]);
    mx = max(mx, sc.red[1][i]);
  }
  __syncthreads();
}

// Threshold of a selection: an entry with masked key m = key & mask is
// selected iff m > prefix, or m == prefix and fewer than krem earlier
// entries also have m == prefix.
struct SelRule {
  uint32_t prefix;
  uint32_t mask;
  int krem;
};

// Entries stored as uint2 {key, index}.
struct PairSrc {
  const uint2* p;
  __device__ __forceinline__ uint32_t key(int i) const { return p[i].x; }
  __device__ __forceinline__ int32_t idx(int i) const { return static_cast<int32_t>(p[i].y); }
};
// A dense float32 score row: key = order key of the score, index = position.
struct F32RowSrc {
  const float* p;
  __device__ __forceinline__ uint32_t key(int i) const { return order_key_f32(p[i]); }
  __device__ __forceinline__ int32_t idx(int i) const { return i; }
};
struct I32RowSrc {
  const int32_t* p;
  __device__ __forceinline__ uint32_t key(int i) const { return order_key_i32(p[i]); }
  __device__ __forceinline__ int32_t idx(int i) const { return i; }
};

// Rule selecting the k first entries of the order (key descending, array
// position ascending) among M entries.  0 <= k.  hist: 2048 words of LDS.
template <int NT, class Src>
__device__ SelRule block_select_rule(const Src& src, int M, int k, uint32_t* hist,
                                     BlockScratch<NT>& sc) {
  if (k >= M || k <= 0) return SelRule{0u, 0u, k <= 0 ? 0 : M};
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int i = threadIdx.x; i < M; i += NT) {
    const uint32_t u = src.key(i);
    mn = min(mn, u);
    mx = max(mx, u);
  }
  block_minmax<NT>(mn, mx, sc);
  if (mn == mx) return SelRule{0u, 0u, k};
  const int hb = 31 - __clz(static_cast<int>(mn ^ mx));
  uint32_t mask = hb == 31 ? 0u : ~((1u << (hb + 1)) - 1u);
  uint32_t prefix = mn & mask;
  int krem = k;
  int lo = hb + 1;
  while (lo > 0) {
    const int width = lo < 11 ? lo : 11;
    const int sh = lo - width;
    const int nb = 1 << width;
    for (int i = threadIdx.x; i < nb; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < M; i += NT) {
      const uint32_t u = src.key(i);
      if ((u & mask) == prefix) atomicAdd(&hist[(u >> sh) & (nb - 1)], 1u);
    }
    __syncthreads();
    // thread t owns ranks [t*per, (t+1)*per) counted from the top digit down
    const int per = (nb + NT - 1) / NT;
    int mine = 0;
    for (int i = 0; i < per; ++i) {
      const int r = threadIdx.x * per + i;
      if (r < nb) mine += static_cast<int>(hist[nb - 1 - r]);
    }
    int tot;
    const int above = block_excl_scan<NT>(mine, sc, tot);
    if (above < krem && krem <= above + mine) {
      int cum = above;
      for (int i = 0; i < per; ++i) {
        const int r = threadIdx.x * per + i;
        const int digit = nb - 1 - r;
        const int c = static_cast<int>(hist[digit]);
        if (cum + c >= krem) {
          sc.found[0] = digit;
          sc.found[1] = krem - cum;
          sc.found[2] = c;
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    const int digit = sc.found[0];
    krem = sc.found[1];
    const int cnt = sc.found[2];
    __syncthreads();
    prefix |= static_cast<uint32_t>(digit) << sh;
    mask |= static_cast<uint32_t>(nb - 1) << sh;
    lo = sh;
    if (cnt == krem) break;  // the whole bin is taken
  }
  return SelRule{prefix, mask, krem};
}

// Writes the indices of the selected entries, in array order, to
// out[0..cap).  Returns how many were written.
template <int NT, class Src>
__device__ int block_compact(const Src& src, int M, const SelRule& rule, int32_t* out, int cap,
                             BlockScratch<NT>& sc) {
  int out_pos = 0, eq_seen = 0;
  for (int base = 0; base < M; base += NT) {
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
    if (sel && out_pos + selx < cap) out[out_pos + selx] = src.idx(i);
    out_pos += seltot;
    eq_seen += eqtot;
  }
  return out_pos < cap ? out_pos : cap;
}

// Value of the r-th largest key (1-based) or a lower bound of it that is a
// key boundary: every entry with key >= the result is at or above rank r's
// bin.  Used for the candidate threshold of a sample.
template <int NT, class Src>
__device__ uint32_t block_rank_lower_bound(const Src& src, int M, int r, uint32_t* hist,
                                           BlockScratch<NT>& sc) {
  uint32_t mn = 0xffffffffu, mx = 0u;
  for (int i = threadIdx.x; i < M; i += NT) {
    const uint32_t u = src.key(i);
    mn = min(mn, u);
    mx = max(mx, u);
  }
  block_minmax<NT>(mn, mx, sc);
  if (r >= M || mn == mx) return mn;
  const SelRule rule = block_select_rule<NT>(src, M, r, hist, sc);
  return rule.prefix;  // unfixed low bits are zero: a lower bound of the bin
}

}  // namespace hst
