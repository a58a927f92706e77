// Prefill hashing of keys: soft-LSH bucket ids + value norms, and binary
// codes.  SOCKET overview page, "Core mechanism: soft LSH", item 1 (one
// bucket id per table from random projections, value norm cached); HATA
// explainer page, section 3 (binary codes of keys).
//
// Every output bit is the exact sign of a real dot product of stored bf16 /
// float32 values.
//
// bf16 keys with byte-sized ids (P = 8) and 128-bit codes go through the
// matrix cores: both are "pack the sign bits of the key-by-plane projection,
// little-endian" (bit p of id byte l is plane l*P + p; bit i of a code is bit
// i % 32 of word i / 32).  v_mfma_f32_32x32x16_bf16 forms the products
// exactly (8 x 8 significand bits) and accumulates in float32; the sign of
// the float32 result is taken when its magnitude clears a bound on the
// accumulation error (below), and otherwise the projection is re-summed
// exactly in float64 on the vector units.  Other shapes use one thread per
// (key, table) with the same exact float64 decision.
//
// Accumulation error bound.  One MFMA instruction adds 16 exact products to
// its accumulator; we take its result to be within 2 float32 ulps of that
// exact sum (one correctly rounded addition is within half an ulp), so over
// the d/16 instructions of a d-long projection the error is at most
// (d/16) * 2 * 2^-23 * sum_c |w_c k_c| <= d * 2^-26 * ||w|| ||k||
// (Cauchy-Schwarz).  The norms are float32 upper estimates inflated by
// 2^-8, and 2^-100 of absolute slack covers flushed subnormals.  Measured on
// gfx950 over 128-long chains with exponents spread over 2^20, the largest
// error was 7.1 * 2^-24 * sum |w_c k_c|, 4.5x inside the bound.  Signs inside
// the band (about 2e-5 of them for Gaussian data) are resolved exactly.
#include "hst_common.h"
#include "hst_launch.h"

namespace hst {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename Kern>
static hipError_t set_lds_limit(Kern kern, size_t bytes) {
  static size_t done[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev >= 0 && dev < 64 && done[dev] >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
  if (e == hipSuccess && dev >= 0 && dev < 64) done[dev] = bytes;
  return e;
}

// ---------------------------------------------------------------- generic path

// One thread per (key, table): P projections, P sign bits -> one id byte.
template <typename T>
__global__ void __launch_bounds__(256)
hash_softlsh_generic_kernel(const T* __restrict__ K, const T* __restrict__ W,
                            const int32_t* __restrict__ seq_lens, int Hkv, int Nmax,
                            int d, int L, int P, uint8_t* __restrict__ ids) {
  const int bh = blockIdx.y;
  const int b = bh / Hkv, h = bh % Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const long long t = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long long j = t / L;
  const int l = static_cast<int>(t % L);
  if (j >= n) return;
  const T* key = K + (static_cast<long long>(bh) * Nmax + j) * d;
  const T* wt = W + (static_cast<long long>(h) * L * P + static_cast<long long>(l) * P) * d;
  uint32_t id = 0;
  for (int p = 0; p < P; ++p)
    if (dot_nonneg_exact(wt + static_cast<long long>(p) * d, key, d)) id |= 1u << p;
  ids[(static_cast<long long>(bh) * Nmax + j) * L + l] = static_cast<uint8_t>(id);
}

// Binary codes: a block of 2*64 threads handles keys one at a time; thread i
// decides bit i, a wave ballot packs 64 bits into two words.
template <typename T>
__global__ void __launch_bounds__(128)
binary_codes_generic_kernel(const T* __restrict__ X, const T* __restrict__ R,
                            const int32_t* __restrict__ seq_lens, int Hkv, int Nmax,
                            int d, int keys_per_block, uint32_t* __restrict__ codes) {
  const int bh = blockIdx.y;
  const int b = bh / Hkv, h = bh % Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int i = threadIdx.x;  // bit index 0..127
  const T* rrow = R + (static_cast<long long>(h) * 128 + i) * d;
  const long long j0 = static_cast<long long>(blockIdx.x) * keys_per_block;
  for (int u = 0; u < keys_per_block; ++u) {
    const long long j = j0 + u;
    if (j >= n) break;
    const T* x = X + (static_cast<long long>(bh) * Nmax + j) * d;
    bool bit = dot_nonneg_exact(rrow, x, d);
    unsigned long long m = __ballot(bit);
    if ((i & 63) == 0) {
      uint32_t* dst = codes + (static_cast<long long>(bh) * Nmax + j) * 4 + (i >> 6) * 2;
      dst[0] = static_cast<uint32_t>(m);
      dst[1] = static_cast<uint32_t>(m >> 32);
    }
  }
}

// ---------------------------------------------------------------- matrix-core path

constexpr int kSgnWaves = 8;    // waves per workgroup (2 per SIMD)
constexpr int kSgnQueue = 64;   // projections awaiting the exact decision, per wave

template <int D, int NBG>
struct SignLds {
  static constexpr int kRowU32 = D / 2 + 4;  // plane row: D bf16 + 16 B pad (conflict-free b128 reads)
  static constexpr size_t kW = static_cast<size_t>(NBG) * kRowU32 * 4;
  static constexpr size_t kBound = (NBG / 32) * 4;
  static constexpr size_t kQueue = static_cast<size_t>(kSgnWaves) * kSgnQueue * 8;
  static constexpr size_t kBytes = kW + kBound + kQueue;
};

// Exact decisions for the queued (key, plane) pairs, one per lane, and the
// fix-up of the already stored words.
template <int D, int NBG>
__device__ __noinline__ void sign_queue_flush(const uint2* __restrict__ q, int count, int lane,
                                              const uint32_t* wl, const bf16* __restrict__ Kh,
                                              uint32_t* __restrict__ outw, int out_words,
                                              int word0) {
  // the words were written with plain stores by this wave: let them land first
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  if (lane < count) {
    const uint2 it = q[lane];
    const long long j = it.x;
    const int plane = static_cast<int>(it.y);
    const bf16* wrow = reinterpret_cast<const bf16*>(wl + plane * SignLds<D, NBG>::kRowU32);
    const bool bit = dot_nonneg_exact(wrow, Kh + j * D, D);
    uint32_t* word = outw + j * out_words + word0 + (plane >> 5);
    const uint32_t m = 1u << (plane & 31);
    if (bit)
      atomicOr(word, m);
    else
      atomicAnd(word, ~m);
  }
}

// Workgroup = 8 waves over keys [j0, j0 + kpw) of one (sequence, kv head) and
// planes [pg * NBG, (pg + 1) * NBG).  The planes live in LDS (MFMA A operand,
// 32 planes x 16 channels per step); each wave takes 64-key tiles whose
// channels sit in registers (B operand, loaded straight from HBM; the other
// waves of the SIMD compute while one waits for its tile).  Result of a 32x32 block: lane
// (j = lane % 32, half = lane / 32) holds key j, planes 8(r/4) + 4 half + r%4
// for r < 16; their sign bits are packed with alignbit and merged across the
// two halves into the 32-bit output word of that key and plane block.
template <int D, int NBG>
__global__ void __launch_bounds__(kSgnWaves * 64)
hash_signs_mfma_kernel(const bf16* __restrict__ K, const bf16* __restrict__ Wall,
                       const int32_t* __restrict__ seq_lens, int Hkv, int Nmax, int nplanes,
                       int kpw, uint32_t* __restrict__ out) {
  using LD = SignLds<D, NBG>;
  constexpr int S = D / 16;       // MFMA steps along the channels
  constexpr int RB = NBG / 32;    // 32-plane blocks
  constexpr int ROW = LD::kRowU32;
  extern __shared__ __align__(16) uint32_t sgn_lds[];
  uint32_t* wl = sgn_lds;
  float* bound = reinterpret_cast<float*>(sgn_lds + LD::kW / 4);
  uint2* queue = reinterpret_cast<uint2*>(sgn_lds + (LD::kW + LD::kBound) / 4);

  const int bh = blockIdx.x, b = bh / Hkv, h = bh % Hkv;
  const int pg = blockIdx.z;
  const int n = seq_len(seq_lens, b, Nmax);
  const long long j0 = static_cast<long long>(blockIdx.y) * kpw;
  if (j0 >= n) return;
  const long long jend = (j0 + kpw < n) ? j0 + kpw : n;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, jl = lane & 31, hf = lane >> 5;

  // planes of this group -> LDS
  {
    const uint32_t* wsrc = reinterpret_cast<const uint32_t*>(
        Wall + (static_cast<long long>(h) * nplanes + static_cast<long long>(pg) * NBG) * D);
    constexpr int CPR = D / 8;  // 16-byte pieces per plane row
    for (int p = tid; p < NBG * CPR; p += kSgnWaves * 64) {
      const int row = p / CPR, c = p % CPR;
      const u32x4 v = *reinterpret_cast<const u32x4*>(wsrc + row * (D / 2) + c * 4);
      *reinterpret_cast<u32x4*>(wl + row * ROW + c * 4) = v;
    }
  }
  __syncthreads();
  // bound factor per 32-plane block: d 2^-26 (1 + 2^-8) max ||w||
  for (int rb = wave; rb < RB; rb += kSgnWaves) {
    const uint32_t* row = wl + (rb * 32 + jl) * ROW + hf * (D / 4);
    float s2 = 0.f;
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      const float lo = bf16_lo(row[c]), hi = bf16_hi(row[c]);
      s2 = fmaf(lo, lo, s2);
      s2 = fmaf(hi, hi, s2);
    }
    s2 += __shfl_xor(s2, 32);
    for (int m = 16; m >= 1; m >>= 1) s2 = fmaxf(s2, __shfl_xor(s2, m));
    if (lane == 0) bound[rb] = sqrtf(s2) * (static_cast<float>(D) * 0x1p-26f * (1.f + 0x1p-8f));
  }
  __syncthreads();

  const bf16* Kh = K + static_cast<long long>(bh) * Nmax * D;
  const uint32_t* Kw = reinterpret_cast<const uint32_t*>(Kh);
  const int out_words = nplanes / 32;
  uint32_t* outw = out + static_cast<long long>(bh) * Nmax * out_words;
  const int word0 = pg * RB;
  uint2* q = queue + wave * kSgnQueue;
  int qn = 0;  // wave-uniform

  const int ntile = static_cast<int>((jend - j0 + 63) / 64);
  u32x4 bop[2][S];
  auto load_tile = [&](int t, u32x4(&dst)[2][S]) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      long long j = j0 + t * 64 + cb * 32 + jl;
      j = j < jend ? j : jend - 1;
      const uint32_t* src = Kw + j * (D / 2) + hf * 4;
#pragma unroll
      for (int s = 0; s < S; ++s) dst[cb][s] = *reinterpret_cast<const u32x4*>(src + s * 8);
    }
  };
  for (int t = wave; t < ntile; t += kSgnWaves) {
    load_tile(t, bop);
    // the plane rows are re-read from LDS per tile: an opaque offset keeps the
    // compiler from hoisting them into registers across the tile loop
    int aoff = (jl * ROW) + hf * 4;
    asm volatile("" : "+v"(aoff));
    // upper estimates of the key norms (both halves of the channels)
    float nk[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      float s2 = 0.f;
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2_t v = __builtin_bit_cast(bf16x2_t, bop[cb][s][e]);
          s2 = __builtin_amdgcn_fdot2_f32_bf16(v, v, s2, false);
        }
      s2 += __shfl_xor(s2, 32);
      nk[cb] = sqrtf(s2);
    }
    long long jk[2];
    jk[0] = j0 + t * 64 + jl;
    jk[1] = jk[0] + 32;
#pragma unroll 2
    for (int rb = 0; rb < RB; ++rb) {
      f32x16 acc0 = {}, acc1 = {};
      const uint32_t* arow = wl + rb * 32 * ROW + aoff;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(arow + s * 8);
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bop[0][s]),
                                                       acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8_t, bop[1][s]),
                                                       acc1, 0, 0, 0);
      }
      const float bnd = bound[rb];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const f32x16& acc = cb == 0 ? acc0 : acc1;
        const float thr = fmaf(nk[cb], bnd, 0x1p-100f);
        float mn = fabsf(acc[0]);
        uint32_t v = 0;
#pragma unroll
        for (int r = 15; r >= 0; --r) {
          v = __builtin_amdgcn_alignbit(v, __float_as_uint(acc[r]), 31);  // bit r = sign of acc[r]
          if (r > 0) mn = fminf(mn, fabsf(acc[r]));
        }
        v = ~v & 0xffffu;  // 1 = non-negative
        v = (v | (v << 8)) & 0x00ff00ffu;
        v = (v | (v << 4)) & 0x0f0f0f0fu;
        v <<= 4 * hf;
        v |= __shfl_xor(v, 32);
        const long long j = jk[cb];
        if (hf == 0 && j < jend) outw[j * out_words + word0 + rb] = v;
        // rare: some sign inside the error band
        if (__ballot(!(mn > thr) && j < jend) != 0ull) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const bool f = !(fabsf(acc[r]) > thr) && j < jend;
            const unsigned long long m = __ballot(f);
            if (m == 0ull) continue;
            const int cnt = __popcll(m);
            if (qn + cnt > kSgnQueue) {
              sign_queue_flush<D, NBG>(q, qn, lane, wl, Kh, outw, out_words, word0);
              qn = 0;
            }
            if (f) {
              const int pos = qn + __builtin_amdgcn_mbcnt_hi(
                                       static_cast<uint32_t>(m >> 32),
                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
              q[pos] = make_uint2(static_cast<uint32_t>(j),
                                  static_cast<uint32_t>(rb * 32 + 8 * (r >> 2) + 4 * hf + (r & 3)));
            }
            qn += cnt;
          }
        }
      }
    }
  }
  if (qn > 0) sign_queue_flush<D, NBG>(q, qn, lane, wl, Kh, outw, out_words, word0);
}

template <int D, int NBG>
static hipError_t launch_signs_mfma(const hst_shape& s, const void* K, const void* W, int nplanes,
                                    void* out, hipStream_t st) {
  auto kern = hash_signs_mfma_kernel<D, NBG>;
  constexpr size_t smem = SignLds<D, NBG>::kBytes;
  hipError_t e = set_lds_limit(kern, smem);
  if (e != hipSuccess) return e;
  const long long BH = static_cast<long long>(s.B) * s.Hkv;
  // about 256 workgroups (one per CU), 512..16384 keys each
  long long kpw = (BH * s.Nmax + 255) / 256;
  kpw = (kpw + 511) / 512 * 512;
  kpw = kpw < 512 ? 512 : (kpw > 16384 ? 16384 : kpw);
  while ((s.Nmax + kpw - 1) / kpw > 65535) kpw *= 2;
  const long long gy = (s.Nmax + kpw - 1) / kpw;
  // x = (sequence, kv head): workgroups are handed to the XCDs round robin in
  // linear order, so one head's workgroups (B*Hkv apart) share an XCD and its
  // L2 copy of the planes whenever B*Hkv is a multiple of 8
  dim3 grid(static_cast<unsigned>(BH), static_cast<unsigned>(gy),
            static_cast<unsigned>(nplanes / NBG));
  hipLaunchKernelGGL(kern, grid, dim3(kSgnWaves * 64), smem, st, static_cast<const bf16*>(K),
                     static_cast<const bf16*>(W), s.seq_lens, s.Hkv, s.Nmax, nplanes,
                     static_cast<int>(kpw), static_cast<uint32_t*>(out));
  return hipGetLastError();
}

// bf16 keys, 128-plane multiples, 16-byte aligned operands and 4-byte
// aligned output rows: the matrix-core path (512-plane groups when they
// divide the planes, else 128-plane groups).
static bool signs_mfma_ok(const hst_shape& s, int nplanes, const void* K, const void* W,
                          const void* out) {
  if (s.kv_dtype != HST_BF16 || (s.d != 128 && s.d != 64) || nplanes % 128 != 0) return false;
  return reinterpret_cast<uintptr_t>(K) % 16 == 0 && reinterpret_cast<uintptr_t>(W) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(out) % 4 == 0;
}

static hipError_t launch_signs(const hst_shape& s, const void* K, const void* W, int nplanes,
                               void* out, hipStream_t st) {
  if (s.d == 128)
    return nplanes % 512 == 0 ? launch_signs_mfma<128, 512>(s, K, W, nplanes, out, st)
                              : launch_signs_mfma<128, 128>(s, K, W, nplanes, out, st);
  return nplanes % 512 == 0 ? launch_signs_mfma<64, 512>(s, K, W, nplanes, out, st)
                            : launch_signs_mfma<64, 128>(s, K, W, nplanes, out, st);
}

// ---------------------------------------------------------------- value norms

// float32 values: 16 lanes per key, float64 sum of squares, one rounding.
template <bool F16OUT>
__global__ void __launch_bounds__(256)
value_norm_f32_kernel(const float* __restrict__ V, const int32_t* __restrict__ seq_lens,
                      int Hkv, int Nmax, int d, void* __restrict__ vnorm) {
  const int bh = blockIdx.y;
  const int b = bh / Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int sub = threadIdx.x & 15;
  const long long j = static_cast<long long>(blockIdx.x) * (blockDim.x / 16) + (threadIdx.x >> 4);
  double acc = 0.0;
  if (j < n) {
    const float* row = V + (static_cast<long long>(bh) * Nmax + j) * d;
    for (int c = sub; c < d; c += 16) {
      double v = row[c];
      acc += v * v;
    }
  }
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (j < n && sub == 0) {
    double r = sqrt(acc);
    long long o = static_cast<long long>(bh) * Nmax + j;
    if (F16OUT)
      static_cast<uint16_t*>(vnorm)[o] = f64_to_f16_bits(r);
    else
      static_cast<float*>(vnorm)[o] = static_cast<float>(r);
  }
}

// bf16 values: D/8 lanes per key, one 16-byte piece each (a load covers
// 512 / D consecutive rows of a wave, fully coalesced), kNormRows rows per
// thread group loaded up front; squares and their sum in float64, the square
// root rounded once to the storage type.
constexpr int kNormU = 16;

template <int D, bool F16OUT>
__global__ void __launch_bounds__(256)
value_norm_bf16_kernel(const bf16* __restrict__ V, const int32_t* __restrict__ seq_lens, int Hkv,
                       int Nmax, void* __restrict__ vnorm) {
  constexpr int LPK = D / 8;           // lanes per key
  constexpr int RPI = 256 / LPK;       // rows per load instruction of the workgroup
  const int bh = blockIdx.y;
  const int b = bh / Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const long long base = static_cast<long long>(blockIdx.x) * RPI * kNormU;
  if (base >= n) return;
  const int sub = threadIdx.x % LPK;
  const uint32_t* Vw = reinterpret_cast<const uint32_t*>(V + static_cast<long long>(bh) * Nmax * D);
  u32x4 w[kNormU];
#pragma unroll
  for (int u = 0; u < kNormU; ++u) {
    long long j = base + u * RPI + threadIdx.x / LPK;
    j = j < n ? j : n - 1;
    w[u] = *reinterpret_cast<const u32x4*>(Vw + j * (D / 2) + sub * 4);
  }
#pragma unroll
  for (int u = 0; u < kNormU; ++u) {
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double lo = bf16_lo(w[u][e]), hi = bf16_hi(w[u][e]);
      acc = fma(lo, lo, acc);
      acc = fma(hi, hi, acc);
    }
#pragma unroll
    for (int m = LPK / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, LPK);
    const long long j = base + u * RPI + threadIdx.x / LPK;
    if (j < n && sub == 0) {
      const double r = sqrt(acc);
      const long long o = static_cast<long long>(bh) * Nmax + j;
      if (F16OUT)
        static_cast<uint16_t*>(vnorm)[o] = f64_to_f16_bits(r);
      else
        static_cast<float*>(vnorm)[o] = static_cast<float>(r);
    }
  }
}

static hipError_t launch_value_norms(const hst_shape& s, const void* V, int norm_dtype,
                                     void* vnorm, hipStream_t st) {
  const int BH = s.B * s.Hkv;
  const bool f16 = norm_dtype == HST_F16;
  if (s.kv_dtype == HST_F32) {
    dim3 grid(static_cast<unsigned>((s.Nmax + 15) / 16), BH);
    if (f16)
      hipLaunchKernelGGL((value_norm_f32_kernel<true>), grid, dim3(256), 0, st,
                         static_cast<const float*>(V), s.seq_lens, s.Hkv, s.Nmax, s.d, vnorm);
    else
      hipLaunchKernelGGL((value_norm_f32_kernel<false>), grid, dim3(256), 0, st,
                         static_cast<const float*>(V), s.seq_lens, s.Hkv, s.Nmax, s.d, vnorm);
    return hipGetLastError();
  }
  if (reinterpret_cast<uintptr_t>(V) % 16 != 0) return hipErrorInvalidValue;
  const long long rpb = static_cast<long long>(256 / (s.d / 8)) * kNormU;  // rows per workgroup
  dim3 grid(static_cast<unsigned>((s.Nmax + rpb - 1) / rpb), BH);
  const bf16* v = static_cast<const bf16*>(V);
  if (s.d == 128) {
    if (f16)
      hipLaunchKernelGGL((value_norm_bf16_kernel<128, true>), grid, dim3(256), 0, st, v,
                         s.seq_lens, s.Hkv, s.Nmax, vnorm);
    else
      hipLaunchKernelGGL((value_norm_bf16_kernel<128, false>), grid, dim3(256), 0, st, v,
                         s.seq_lens, s.Hkv, s.Nmax, vnorm);
  } else {
    if (f16)
      hipLaunchKernelGGL((value_norm_bf16_kernel<64, true>), grid, dim3(256), 0, st, v,
                         s.seq_lens, s.Hkv, s.Nmax, vnorm);
    else
      hipLaunchKernelGGL((value_norm_bf16_kernel<64, false>), grid, dim3(256), 0, st, v,
                         s.seq_lens, s.Hkv, s.Nmax, vnorm);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- launchers

hipError_t launch_hash_softlsh(const hst_shape& s, const void* K, const void* V,
                               const void* W, int L, int P, int norm_dtype,
                               uint8_t* ids, void* vnorm, hipStream_t st) {
  const int BH = s.B * s.Hkv;
  hipError_t e;
  if (P == 8 && signs_mfma_ok(s, L * 8, K, W, ids)) {
    e = launch_signs(s, K, W, L * 8, ids, st);
  } else {
    long long work = static_cast<long long>(s.Nmax) * L;
    dim3 grid(static_cast<unsigned>((work + 255) / 256), BH);
    if (s.kv_dtype == HST_F32)
      hipLaunchKernelGGL(hash_softlsh_generic_kernel<float>, grid, dim3(256), 0, st,
                         static_cast<const float*>(K), static_cast<const float*>(W),
                         s.seq_lens, s.Hkv, s.Nmax, s.d, L, P, ids);
    else
      hipLaunchKernelGGL(hash_softlsh_generic_kernel<bf16>, grid, dim3(256), 0, st,
                         static_cast<const bf16*>(K), static_cast<const bf16*>(W),
                         s.seq_lens, s.Hkv, s.Nmax, s.d, L, P, ids);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  return launch_value_norms(s, V, norm_dtype, vnorm, st);
}

hipError_t launch_hash_binary(const hst_shape& s, const void* K, const void* R,
                              uint32_t* codes, hipStream_t st) {
  if (signs_mfma_ok(s, 128, K, R, codes)) return launch_signs(s, K, R, 128, codes, st);
  const int kpb = 16;
  dim3 grid(static_cast<unsigned>((s.Nmax + kpb - 1) / kpb), s.B * s.Hkv);
  if (s.kv_dtype == HST_F32)
    hipLaunchKernelGGL(binary_codes_generic_kernel<float>, grid, dim3(128), 0, st,
                       static_cast<const float*>(K), static_cast<const float*>(R),
                       s.seq_lens, s.Hkv, s.Nmax, s.d, kpb, codes);
  else
    hipLaunchKernelGGL(binary_codes_generic_kernel<bf16>, grid, dim3(128), 0, st,
                       static_cast<const bf16*>(K), static_cast<const bf16*>(R),
                       s.seq_lens, s.Hkv, s.Nmax, s.d, kpb, codes);
  return hipGetLastError();
}

}  // namespace hst
