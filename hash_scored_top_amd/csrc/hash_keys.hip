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
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename Kern>
static hipError_t set_lds_limit(Kern kern, size_t bytes) {
  return raise_lds_limit(reinterpret_cast<const void*>(kern), bytes);
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
__global__ void __launch_bounds__(256)
binary_codes_generic_kernel(const T* __restrict__ X, const T* __restrict__ R,
                            const int32_t* __restrict__ seq_lens, int Hkv, int Nmax,
                            int d, int keys_per_block, uint32_t* __restrict__ codes) {
  const int bh = blockIdx.y;
  const int b = bh / Hkv, h = bh % Hkv;
  const int n = seq_len(seq_lens, b, Nmax);
  const int nbits = blockDim.x;  // 64, 128 or 256: one thread per bit
  const int i = threadIdx.x;
  const T* rrow = R + (static_cast<long long>(h) * nbits + i) * d;
  const long long j0 = static_cast<long long>(blockIdx.x) * keys_per_block;
  for (int u = 0; u < keys_per_block; ++u) {
    const long long j = j0 + u;
    if (j >= n) break;
    const T* x = X + (static_cast<long long>(bh) * Nmax + j) * d;
    bool bit = dot_nonneg_exact(rrow, x, d);
    unsigned long long m = __ballot(bit);
    if ((i & 63) == 0) {
      uint32_t* dst = codes + (static_cast<long long>(bh) * Nmax + j) * (nbits / 32) + (i >> 6) * 2;
      dst[0] = static_cast<uint32_t>(m);
      dst[1] = static_cast<uint32_t>(m >> 32);
    }
  }
}

// ---------------------------------------------------------------- matrix-core path

constexpr int kSgnTile = 64;   // keys per tile
constexpr int kSgnExp = kExactLimbs;  // words of an exact fixed-point sum (LDS, per lane)

template <int D, int NBG>
struct SignCfg {
  static constexpr int kWaves = 8;
  static constexpr int kNT = kWaves * 64;
  static constexpr int kPS = NBG / 64;                     // 64-plane slices
  static constexpr int kKG = kWaves / kPS;                 // key groups
  static constexpr int kChunk = 256;                       // keys staged per step
  static constexpr int kSub = kChunk / kSgnTile / kKG;     // 64-key tiles per wave per step
  static constexpr int kS = D / 16;                        // MFMA steps along the channels
  static constexpr int kPPR = D / 8;                       // 16-byte pieces per key row
  static constexpr int kPieces = kChunk * kPPR / kNT;      // pieces per thread per step
  static constexpr int kRowB = 2 * D + 16;                 // padded LDS row: conflict-free b128 reads
  static constexpr size_t kBuf = static_cast<size_t>(kChunk) * kRowB + kChunk * 4;  // rows + norms
  // plus, per wave, a list of the tiles holding uncertain signs (kpw / 64 + 1 words)
  static size_t bytes(int kpw) {
    return 2 * kBuf + static_cast<size_t>(kWaves) * (kpw / kSgnTile + 1) * 4;
  }
};

// Exact sign of W[plane] . K[j] (bf16 rows of D values, 16-byte aligned):
// both rows are loaded at once, the float64 sum decides unless it lies
// within its rounding band, where the exact fixed-point sum takes over.
template <int D>
__device__ __forceinline__ bool exact_sign_rows(const bf16* __restrict__ wrow,
                                                const bf16* __restrict__ krow, uint64_t* h) {
  u32x4 wv[D / 8], kv[D / 8];
#pragma unroll
  for (int i = 0; i < D / 8; ++i) {
    wv[i] = reinterpret_cast<const u32x4*>(wrow)[i];
    kv[i] = reinterpret_cast<const u32x4*>(krow)[i];
  }
  double s = 0.0, sa = 0.0;
#pragma unroll
  for (int i = 0; i < D / 8; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double p0 = static_cast<double>(bf16_lo(wv[i][e])) * bf16_lo(kv[i][e]);
      const double p1 = static_cast<double>(bf16_hi(wv[i][e])) * bf16_hi(kv[i][e]);
      s += p0;
      s += p1;
      sa += fabs(p0) + fabs(p1);
    }
  if (fabs(s) > 2.0 * D * 0x1p-53 * sa) return s >= 0.0;
  return exact_dot_nonneg_in(wrow, krow, D, h);
}

// Workgroup = 8 waves over keys [j0, j0 + kpw) of one (sequence, kv head) and
// the planes [pg * NBG, (pg + 1) * NBG).  Wave w takes the 64-plane slice
// w % (NBG / 64), kept in registers as the MFMA A operand (plane 32 rb +
// lane % 32, channels 16 s + 8 (lane / 32) at step s), and key group
// w / (NBG / 64).  The workgroup streams 256-key steps: coalesced 16-byte
// loads of the next step run in registers during the current step's compute,
// then go to one of two padded LDS buffers (with the key norms), from which
// every wave reads the B operands of its 64-key tiles.  Result of a 32x32
// block: lane (j = lane % 32, half = lane / 32) holds key j, planes
// 8(r/4) + 4 half + r%4 for r < 16; their sign bits are packed with alignbit
// and merged across the two halves into the 32-bit output word of that key
// and plane block.
template <int D, int NBG>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2)))
hash_signs_mfma_kernel(const bf16* __restrict__ K, const bf16* __restrict__ Wall,
                       const int32_t* __restrict__ seq_lens, int Hkv, int Nmax, int nplanes,
                       int kpw, uint32_t* __restrict__ out) {
  using C = SignCfg<D, NBG>;
  constexpr int S = C::kS, NP = C::kPieces, PPR = C::kPPR, ROWB = C::kRowB;
  constexpr int NT = C::kNT, CH = C::kChunk;
  extern __shared__ __align__(16) unsigned char sgn_lds[];

  const int bh = blockIdx.x, b = bh / Hkv, h = bh % Hkv;
  const int pg = blockIdx.z;
  const int n = seq_len(seq_lens, b, Nmax);
  const long long j0 = static_cast<long long>(blockIdx.y) * kpw;
  if (j0 >= n) return;
  const long long jend = (j0 + kpw < n) ? j0 + kpw : n;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, jl = lane & 31, hf = lane >> 5;
  const int ps = wave % C::kPS, kg = wave / C::kPS;  // plane slice, key group
  const int ntile = static_cast<int>((jend - j0 + kSgnTile - 1) / kSgnTile);
  const int nchunk = static_cast<int>((jend - j0 + CH - 1) / CH);

  // this wave's planes (A operands) and the error-bound factor per 32-plane block
  const bf16* Wg = Wall + (static_cast<long long>(h) * nplanes + static_cast<long long>(pg) * NBG) * D;
  u32x4 wa[2][S];
  float bnd[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const uint32_t* src =
        reinterpret_cast<const uint32_t*>(Wg + static_cast<long long>(ps * 64 + rb * 32 + jl) * D) +
        hf * 4;
#pragma unroll
    for (int s = 0; s < S; ++s) wa[rb][s] = *reinterpret_cast<const u32x4*>(src + s * 8);
  }
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float s2 = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo(wa[rb][s][e]), hi = bf16_hi(wa[rb][s][e]);
        s2 = fmaf(lo, lo, s2);
        s2 = fmaf(hi, hi, s2);
      }
    s2 += __shfl_xor(s2, 32);
    for (int m = 16; m >= 1; m >>= 1) s2 = fmaxf(s2, __shfl_xor(s2, m));
    // (d/16) MFMA steps x 2 ulps each, norms inflated by 2^-8
    bnd[rb] = sqrtf(s2) * (static_cast<float>(D) * 0x1p-26f * (1.f + 0x1p-8f));
  }

  const bf16* Kh = K + static_cast<long long>(bh) * Nmax * D;
  const uint32_t* Kw = reinterpret_cast<const uint32_t*>(Kh);
  const int out_words = nplanes / 32;
  uint32_t* outw = out + static_cast<long long>(bh) * Nmax * out_words;
  const int word0 = pg * (NBG / 32);
  // output rows of this workgroup behind a buffer resource: a store whose
  // offset is out of range is dropped, so rows past the sequence end need no
  // branch around the store
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
      outw + j0 * out_words, 0, static_cast<int>((jend - j0) * out_words * 4), 0x00020000);
  // tiles of this wave with uncertain signs: entry = tile | block mask << 24
  uint32_t* flist = reinterpret_cast<uint32_t*>(sgn_lds + 2 * C::kBuf) + wave * (kpw / kSgnTile + 1);
  int nfl = 0;  // wave-uniform

  auto gload = [&](int ch, u32x4(&r)[NP]) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + i * NT, row = p / PPR, c = p % PPR;
      long long j = j0 + static_cast<long long>(ch) * CH + row;
      j = j < jend ? j : jend - 1;
      r[i] = *reinterpret_cast<const u32x4*>(Kw + j * (D / 2) + c * 4);
    }
  };
  // tile -> LDS buffer, with the key norms (float32 upper estimates before
  // the 2^-8 inflation folded into the bound factor)
  auto stage = [&](int buf, const u32x4(&r)[NP]) {
    unsigned char* tb = sgn_lds + buf * C::kBuf;
    float* nrm = reinterpret_cast<float*>(tb + CH * ROWB);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = tid + i * NT, row = p / PPR, c = p % PPR;
      *reinterpret_cast<u32x4*>(tb + row * ROWB + c * 16) = r[i];
      float s2 = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bf16x2_t v = __builtin_bit_cast(bf16x2_t, r[i][e]);
        s2 = __builtin_amdgcn_fdot2_f32_bf16(v, v, s2, false);
      }
      s2 = dpp_group_sum<PPR>(s2);
      if (c == 0) nrm[row] = sqrtf(s2);
    }
  };
  auto mfma_block = [&](const u32x4(&a)[S], const u32x4(&bb)[S]) {
    f32x16 acc = {};
#pragma unroll
    for (int s = 0; s < S; ++s)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[s]),
                                                    __builtin_bit_cast(bf16x8_t, bb[s]), acc, 0,
                                                    0, 0);
    return acc;
  };
  // signs of one 32x32 block -> the 32-bit word of (key, plane block), and
  // whether some sign lies inside the error band
  auto pack = [&](const f32x16& acc, float thr, uint32_t& word) {
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
    const auto sw = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    word = sw[0] | sw[1];  // both halves' planes
    return !(mn > thr);
  };
  // One step = this wave's kSub tiles of the buffer, 4 blocks (column block
  // cb, plane block rb) each, software-pipelined: the MFMAs of block k+1 are
  // issued before block k is packed, so the matrix cores and the vector units
  // work side by side.  Tiles past the end are computed and masked out.
  auto compute_step = [&](int c, int buf) {
    constexpr int NBLK = C::kSub * 4;
    const unsigned char* base = sgn_lds + buf * C::kBuf;
    const float* nrm = reinterpret_cast<const float*>(base + CH * ROWB);
    u32x4 bb[C::kSub * 2][S];
    f32x16 acc[NBLK];
    uint32_t word[2][2] = {{0u, 0u}, {0u, 0u}};
    uint32_t flags = 0;  // bit 2 rb + cb of the current tile
    auto ld = [&](int i, int cb) {
      const int row = (kg * C::kSub + i) * kSgnTile + cb * 32 + jl;
#pragma unroll
      for (int s = 0; s < S; ++s)
        bb[i * 2 + cb][s] = *reinterpret_cast<const u32x4*>(base + row * ROWB + s * 32 + hf * 16);
    };
    ld(0, 0);
    acc[0] = mfma_block(wa[0], bb[0]);
#pragma unroll
    for (int k = 0; k < NBLK; ++k) {
      const int i = k >> 2, cb = (k >> 1) & 1, rb = k & 1;
      if (k + 1 < NBLK) {
        if (((k + 1) & 1) == 0) ld((k + 1) >> 2, ((k + 1) >> 1) & 1);
        acc[k + 1] = mfma_block(wa[(k + 1) & 1], bb[(k + 1) >> 1]);
      }
      const int t = c * (CH / kSgnTile) + kg * C::kSub + i;  // tile of the workgroup
      const long long j = j0 + static_cast<long long>(t) * kSgnTile + cb * 32 + jl;
      const float nk = nrm[(kg * C::kSub + i) * kSgnTile + cb * 32 + jl];
      const bool unsure = pack(acc[k], fmaf(nk, bnd[rb], 0x1p-100f), word[rb][cb]);
      flags |= (unsure && j < jend) ? (1u << (2 * rb + cb)) : 0u;
      if (rb == 1 && cb == 1) {
        // lane (jl, hf) stores the two words of key hf * 32 + jl
        const long long jb = j0 + static_cast<long long>(t) * kSgnTile;
        const bool mine = jb + hf * 32 + jl < jend;
        const int orow = t * kSgnTile + hf * 32 + jl;
        u32x2 w2;
        w2[0] = hf ? word[0][1] : word[0][0];
        w2[1] = hf ? word[1][1] : word[1][0];
        __builtin_amdgcn_raw_buffer_store_b64(
            w2, orsrc,
            mine ? static_cast<uint32_t>((orow * out_words + word0 + ps * 2) * 4) : 0x80000000u, 0,
            0);
        // note the tile if a block holds an uncertain sign (the slot is
        // written every time and kept only then: no branch)
        const uint32_t fl = (__ballot(flags & 1u) ? 1u : 0u) | (__ballot(flags & 2u) ? 2u : 0u) |
                            (__ballot(flags & 4u) ? 4u : 0u) | (__ballot(flags & 8u) ? 8u : 0u);
        flist[nfl] = static_cast<uint32_t>(t) | (fl << 24);
        nfl += fl != 0u ? 1 : 0;
        flags = 0;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // step c: copy step c+1 (loaded during step c-1) to the other buffer, load
  // step c+2, then compute step c; one barrier per step
  u32x4 rg[NP];
  gload(0, rg);
  stage(0, rg);
  if (1 < nchunk) gload(1, rg);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    if (c + 1 < nchunk) {
      stage((c + 1) & 1, rg);
      if (c + 2 < nchunk) gload(c + 2, rg);
    }
    compute_step(c, c & 1);
    __syncthreads();
  }

  // Exact decisions for the noted tiles.  A: recompute their flagged blocks
  // from HBM and list the uncertain (key, plane) pairs in the step buffers
  // (free once every wave has left the loop); B: settle the listed pairs one
  // per lane and fix their bits.
  if (nfl == 0) return;
  // per wave: the lanes' fixed-point sums, then the listed pairs
  constexpr int kRegion = static_cast<int>(2 * C::kBuf / C::kWaves) / 8 * 8;
  constexpr int kCap = (kRegion - 64 * kSgnExp * 8) / 8;
  static_assert(kCap >= 64, "room for a wave of pairs");
  uint64_t* hx = reinterpret_cast<uint64_t*>(sgn_lds + wave * kRegion) + lane * kSgnExp;
  uint2* items = reinterpret_cast<uint2*>(sgn_lds + wave * kRegion + 64 * kSgnExp * 8);
  int nit = 0;  // wave-uniform
  // the planes again (L2-resident): the main loop's copy is dead by now,
  // which keeps this cold path clear of register spills
  u32x4 wc[2][S];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const uint32_t* src =
        reinterpret_cast<const uint32_t*>(Wg + static_cast<long long>(ps * 64 + rb * 32 + jl) * D) +
        hf * 4;
#pragma unroll
    for (int s = 0; s < S; ++s) wc[rb][s] = *reinterpret_cast<const u32x4*>(src + s * 8);
  }
  auto settle = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // the words have landed
    for (int i = lane; i < nit; i += 64) {
      const uint2 it = items[i];
      const long long j = it.x;
      const int plane = static_cast<int>(it.y);
      const bool bit = exact_sign_rows<D>(Wg + static_cast<long long>(plane) * D, Kh + j * D, hx);
      uint32_t* word = outw + j * out_words + word0 + (plane >> 5);
      const uint32_t m = 1u << (plane & 31);
      if (bit)
        atomicOr(word, m);
      else
        atomicAnd(word, ~m);
    }
    nit = 0;
  };
  for (int e = 0; e < nfl; ++e) {
    const uint32_t ent = flist[e];
    const int t = static_cast<int>(ent & 0xffffffu);
    const uint32_t fl = ent >> 24;
    const long long jb = j0 + static_cast<long long>(t) * kSgnTile;
#pragma unroll 1
    for (int cb = 0; cb < 2; ++cb) {
      if ((fl & (5u << cb)) == 0u) continue;
      const long long j = jb + cb * 32 + jl;
      const long long jc = j < jend ? j : jend - 1;
      u32x4 bk[S];
      float s2 = 0.f;
#pragma unroll
      for (int s = 0; s < S; ++s) {
        bk[s] = *reinterpret_cast<const u32x4*>(Kw + jc * (D / 2) + s * 8 + hf * 4);
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const bf16x2_t v = __builtin_bit_cast(bf16x2_t, bk[s][e2]);
          s2 = __builtin_amdgcn_fdot2_f32_bf16(v, v, s2, false);
        }
      }
      s2 += __shfl_xor(s2, 32);
      const float nk = sqrtf(s2);
      uint32_t fm = 0;  // bit 16 rb + r: uncertain (shifted in from the top bit down)
#pragma unroll
      for (int rb = 1; rb >= 0; --rb) {
        const f32x16 acc = mfma_block(wc[rb], bk);
        const float thr = fmaf(nk, bnd[rb], 0x1p-100f);
#pragma unroll
        for (int r = 15; r >= 0; --r) fm = (fm << 1) | (!(fabsf(acc[r]) > thr) ? 1u : 0u);
      }
      if (!(j < jend)) fm = 0u;
      // append this lane's pairs, one per lane and round (wave-uniform count)
      while (true) {
        const bool f = fm != 0u;
        const unsigned long long m = __ballot(f);
        if (m == 0ull) break;
        if (nit + __popcll(m) > kCap) settle();
        if (f) {
          const int i = __builtin_ctz(fm);
          fm &= fm - 1u;
          const int pos = nit + __builtin_amdgcn_mbcnt_hi(
                                    static_cast<uint32_t>(m >> 32),
                                    __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
          const int rb = i >> 4, r = i & 15;
          items[pos] = make_uint2(static_cast<uint32_t>(j),
                                  static_cast<uint32_t>(ps * 64 + rb * 32 + 8 * (r >> 2) +
                                                        4 * hf + (r & 3)));
        }
        nit += __popcll(m);
      }
    }
  }
  settle();
}

template <int D, int NBG>
static hipError_t launch_signs_mfma(const hst_shape& s, const void* K, const void* W, int nplanes,
                                    void* out, hipStream_t st) {
  using C = SignCfg<D, NBG>;
  auto kern = hash_signs_mfma_kernel<D, NBG>;
  const long long BH = static_cast<long long>(s.B) * s.Hkv;
  // one workgroup per CU at a time (the two step buffers fill most of the LDS):
  // about 256 workgroups over all keys and plane groups, whole 256-key steps
  const long long wgs = 256;
  long long kpw = (BH * s.Nmax * (nplanes / NBG) + wgs - 1) / wgs;
  kpw = (kpw + 255) / 256 * 256;
  kpw = kpw < 256 ? 256 : (kpw > 16384 ? 16384 : kpw);
  while ((s.Nmax + kpw - 1) / kpw > 65535) kpw *= 2;
  const long long gy = (s.Nmax + kpw - 1) / kpw;
  const size_t smem = C::bytes(static_cast<int>(kpw));
  if (smem > 160 * 1024) return hipErrorInvalidValue;
  hipError_t e = set_lds_limit(kern, smem);
  if (e != hipSuccess) return e;
  // x = (sequence, kv head): workgroups are handed to the XCDs round robin in
  // linear order, so one head's workgroups (B*Hkv apart) share an XCD and its
  // L2 copy of the planes whenever B*Hkv is a multiple of 8
  dim3 grid(static_cast<unsigned>(BH), static_cast<unsigned>(gy),
            static_cast<unsigned>(nplanes / NBG));
  hipLaunchKernelGGL(kern, grid, dim3(C::kNT), smem, st, static_cast<const bf16*>(K),
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
  static_assert(LPK == 8 || LPK == 16, "8 or 16 lanes per key");
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
  // lane 0 of each LPK-lane row group ends with the row's sum: row_shl moves
  // within the 16-lane DPP row give lane 0 the operands of an xor butterfly
  // (lane s adds lane s + m, whose bit m is clear on every lane lane 0 reads)
  // without the LDS crossbar.  Row u's sum then moves to lane u % LPK of the
  // group (row_shr), so that each lane takes the square root and the
  // rounding of kNormU / LPK rows instead of every lane doing all of them.
  constexpr int RPL = kNormU / LPK;  // rows per lane
  double mine[RPL];
#pragma unroll
  for (int m = 0; m < RPL; ++m) mine[m] = 0.0;
#pragma unroll
  for (int u = 0; u < kNormU; ++u) {
    double acc = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double lo = bf16_lo(w[u][e]), hi = bf16_hi(w[u][e]);
      acc = fma(lo, lo, acc);
      acc = fma(hi, hi, acc);
    }
    if constexpr (LPK == 16) acc += dpp_f64<0x108>(acc);  // row_shl 8
    acc += dpp_f64<0x104>(acc);                            // row_shl 4
    acc += dpp_f64<0x102>(acc);                            // row_shl 2
    acc += dpp_f64<0x101>(acc);                            // row_shl 1
    const double moved = u % LPK == 0 ? acc : dpp_f64_row_shr(acc, u % LPK);
    if (sub == u % LPK) mine[u / LPK] = moved;
  }
#pragma unroll
  for (int m = 0; m < RPL; ++m) {
    const long long j = base + (m * LPK + sub) * RPI + threadIdx.x / LPK;
    if (j < n) {
      const double r = sqrt(mine[m]);
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

hipError_t launch_hash_ids_softlsh(const hst_shape& s, const void* K, const void* W, int L, int P,
                                   uint8_t* ids, hipStream_t st) {
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
  return e;
}

hipError_t launch_hash_softlsh(const hst_shape& s, const void* K, const void* V,
                               const void* W, int L, int P, int norm_dtype,
                               uint8_t* ids, void* vnorm, hipStream_t st) {
  const hipError_t e = launch_hash_ids_softlsh(s, K, W, L, P, ids, st);
  if (e != hipSuccess) return e;
  return launch_value_norms(s, V, norm_dtype, vnorm, st);
}

hipError_t launch_hash_binary(const hst_shape& s, const void* K, const void* R, int code_bits,
                              uint32_t* codes, hipStream_t st) {
  if (signs_mfma_ok(s, code_bits, K, R, codes)) return launch_signs(s, K, R, code_bits, codes, st);
  const int kpb = 16;
  dim3 grid(static_cast<unsigned>((s.Nmax + kpb - 1) / kpb), s.B * s.Hkv);
  if (s.kv_dtype == HST_F32)
    hipLaunchKernelGGL(binary_codes_generic_kernel<float>, grid, dim3(code_bits), 0, st,
                       static_cast<const float*>(K), static_cast<const float*>(R),
                       s.seq_lens, s.Hkv, s.Nmax, s.d, kpb, codes);
  else
    hipLaunchKernelGGL(binary_codes_generic_kernel<bf16>, grid, dim3(code_bits), 0, st,
                       static_cast<const bf16*>(K), static_cast<const bf16*>(R),
                       s.seq_lens, s.Hkv, s.Nmax, s.d, kpb, codes);
  return hipGetLastError();
}

}  // namespace hst
