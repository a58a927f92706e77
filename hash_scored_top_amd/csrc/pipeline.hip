// Host-side composition of the decode path: workspace layout and the launch
// sequence of every C-ABI operation.
//
//   decode step (soft-LSH or binary codes):
//     prep  (several workgroups per kv head: query tables / codes, and the
//            key sample scored on each workgroup's part of the hash)
//     scan  (score every key once; one extra workgroup per kv head derives
//            the candidate threshold from the sample meanwhile; keys scoring
//            >= threshold go to the chunk candidate slots)
//     attend (each split derives the exact top-k from the candidates and
//             attends over its part of the selected rows)
//     combine (merge the splits through their log-sum-exp)
#include "hst_fused.h"
#include "hst_launch.h"

namespace hst {

FusedLayout fused_layout(const hst_shape& s, int op, int L, int P, int kcap) {
  FusedLayout f{};
  const long long BH = static_cast<long long>(s.B) * s.Hkv;
  const bool soft = op == HST_OP_SCORE_SOFTLSH || op == HST_OP_DECODE_SOFTLSH;
  const bool ham = op == HST_OP_SCORE_HAMMING || op == HST_OP_DECODE_HAMMING;
  const bool decode = op == HST_OP_DECODE_SOFTLSH || op == HST_OP_DECODE_HAMMING;
  const bool select = op == HST_OP_SELECT_TOPK || decode;
  const bool attn = op == HST_OP_SPARSE_ATTENTION || decode;
  f.kind = soft ? ((L == 16 || L == 32 || L == 64 || L == 128) ? kScanSoftFast : kScanSoftAny)
               : (ham ? kScanHamming : kScanGivenF32);
  const int dchunk = soft ? scan_chunk(L) : scan_chunk(0);
  f.chunk = soft ? scan_cap(L) : scan_cap(0);
  f.nchunks = select ? static_cast<int>((s.Nmax + dchunk - 1) / dchunk) : 0;
  f.sample = select ? kSample : 0;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t r = o;
    o += (bytes + 255) / 256 * 256;
    return r;
  };
  f.off_heads = take(BH * sizeof(HeadState));  // first: the head states start the workspace
  if (soft) f.off_tables = take(BH * (static_cast<size_t>(L) << P) * sizeof(float));
  if (ham) f.off_qcodes = take(static_cast<size_t>(s.B) * s.Hq * 16);
  if (select) {
    f.xparts = prep_parts(f.kind, L);
    f.off_spart = take(BH * static_cast<size_t>(f.xparts) * kSample * 4);
  }
  if (select) {
    f.off_counts = take(BH * f.nchunks * 4);
    f.off_slots = take(BH * f.nchunks * static_cast<size_t>(f.chunk) * 8);
  }
  if (attn) {
    const long long rows = static_cast<long long>(kcap) * BH;
    // about one split per CU: a selecting split spends a fixed time on the
    // head's selection before its gather, so a second round of splits would
    // pay it again on the critical path; up to 4096 rows per split keep one
    // round (given rows: up to 1024)
    long long r = (rows + 255) / 256;
    r = (r + 63) / 64 * 64;
    if (r < 64) r = 64;
    if (r > (select ? 4096 : 1024)) r = select ? 4096 : 1024;
    if ((kcap + r - 1) / r > kMaxSplits) r = (kcap + kMaxSplits - 1) / kMaxSplits;
    f.rps = static_cast<int>(r);
    f.nsplit = static_cast<int>((kcap + r - 1) / r);
    const size_t parts = static_cast<size_t>(s.B) * s.Hq * f.nsplit;
    f.off_part_o = take(parts * s.d * 4);
    f.off_part_ml = take(parts * 2 * 4);
  }
  f.bytes = o;
  return f;
}

static FusedArgs make_args(const hst_shape& s, const FusedLayout& f, void* ws, int L, int P,
                           double tau, int kcap) {
  FusedArgs a{};
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.nbh = s.B * s.Hkv;
  a.d = s.d;
  a.Nmax = s.Nmax;
  a.L = L;
  a.P = P;
  a.inv_tau = tau > 0.0 ? 1.0 / tau : 0.0;
  a.kcap = kcap;
  a.sample = f.sample;
  a.nchunks = f.nchunks;
  a.rps = f.rps;
  a.nsplit = f.nsplit;
  a.xparts = f.xparts;
  a.region_bytes = 65536;
  a.meta_kind = -1;
  const int dchunk = f.kind == kScanSoftFast ? scan_chunk(L) : scan_chunk(0);
  a.span = f.nchunks > 0 ? scan_span(s, dchunk, f.chunk, true) : dchunk;
  char* p = static_cast<char*>(ws);
  if (p != nullptr) {
    a.heads = reinterpret_cast<HeadState*>(p + f.off_heads);
    a.tables = reinterpret_cast<float*>(p + f.off_tables);
    a.qcodes = reinterpret_cast<uint32_t*>(p + f.off_qcodes);
    a.spart = reinterpret_cast<float*>(p + f.off_spart);
    a.counts = reinterpret_cast<uint32_t*>(p + f.off_counts);
    a.slots = reinterpret_cast<uint2*>(p + f.off_slots);
    a.part_o = reinterpret_cast<float*>(p + f.off_part_o);
    a.part_ml = reinterpret_cast<float*>(p + f.off_part_ml);
  }
  return a;
}

#define HST_CHECK(x)                   \
  do {                                 \
    hipError_t _e = (x);               \
    if (_e != hipSuccess) return _e;   \
  } while (0)

hipError_t fused_decode_softlsh(const hst_shape& s, const void* q, const void* K, const void* V,
                                const void* W, int L, int P, double tau, const uint8_t* ids,
                                const void* vnorm, int norm_dtype, int kcap, const int32_t* kps,
                                float scale, int32_t* idx, float* out, float* lse, void* ws,
                                hipStream_t st) {
  HST_CHECK(decode_prepare_softlsh(s, q, W, L, P, tau, ids, vnorm, norm_dtype, kcap, kps, ws, st));
  HST_CHECK(decode_filter_softlsh(s, L, P, ids, vnorm, norm_dtype, kcap, kps, ws, st));
  return decode_finish_softlsh(s, q, K, V, L, P, ids, vnorm, norm_dtype, kcap, scale, idx, out, lse, ws, st);
}

// The three stages of the soft-LSH decode step over one workspace.
static FusedArgs soft_args(const hst_shape& s, void* ws, int L, int P, double tau, int kcap,
                           const uint8_t* ids, const void* vnorm, int norm_dtype, FusedLayout* fo) {
  const FusedLayout f = fused_layout(s, HST_OP_DECODE_SOFTLSH, L, P, kcap);
  FusedArgs a = make_args(s, f, ws, L, P, tau, kcap);
  a.meta = ids;
  a.meta_vn = vnorm;
  a.meta_f16 = norm_dtype == HST_F16;
  a.meta_kind = f.kind;
  if (fo != nullptr) *fo = f;
  return a;
}

hipError_t decode_prepare_softlsh(const hst_shape& s, const void* q, const void* W, int L, int P,
                                  double tau, const uint8_t* ids, const void* vnorm, int norm_dtype,
                                  int kcap, const int32_t* kps, void* ws, hipStream_t st) {
  const FusedArgs a = soft_args(s, ws, L, P, tau, kcap, ids, vnorm, norm_dtype, nullptr);
  return launch_prep_soft(s, a, q, W, ids, kps, st);
}

hipError_t decode_filter_softlsh(const hst_shape& s, int L, int P, const uint8_t* ids,
                                 const void* vnorm, int norm_dtype, int kcap, const int32_t* kps,
                                 void* ws, hipStream_t st) {
  FusedLayout f;
  const FusedArgs a = soft_args(s, ws, L, P, 0.0, kcap, ids, vnorm, norm_dtype, &f);
  return launch_scan(s, a, f.kind, ids, vnorm, norm_dtype == HST_F16, nullptr, 1, kps, st);
}

hipError_t decode_finish_softlsh(const hst_shape& s, const void* q, const void* K, const void* V,
                                 int L, int P, const uint8_t* ids, const void* vnorm,
                                 int norm_dtype, int kcap, float scale, int32_t* idx, float* out,
                                 float* lse, void* ws, hipStream_t st) {
  FusedLayout f;
  const FusedArgs a = soft_args(s, ws, L, P, 0.0, kcap, ids, vnorm, norm_dtype, &f);
  return launch_attend(s, a, q, K, V, idx, true, nullptr, 0, f.chunk, scale, out, lse, st);
}

// Workspace of the mass decode step: the decode layout, then the candidate
// list [B*Hkv][kcap] and the logits [B*Hq][kcap] (float64).
static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t decode_mass_bytes(const hst_shape& s, int L, int P, int kcap) {
  const FusedLayout f = fused_layout(s, HST_OP_DECODE_SOFTLSH, L, P, kcap);
  const size_t cand = static_cast<size_t>(s.B) * s.Hkv * static_cast<size_t>(kcap) * 4;
  return align256(f.bytes) + align256(cand) + align256(mass_logits_bytes(s, kcap));
}

hipError_t fused_decode_softlsh_mass(const hst_shape& s, const void* q, const void* K,
                                     const void* V, const void* W, int L, int P, double tau,
                                     const uint8_t* ids, const void* vnorm, int norm_dtype,
                                     int kcap, const int32_t* kps, double p, float scale,
                                     int32_t* idx, int32_t* counts, float* out, float* lse,
                                     void* ws, hipStream_t st) {
  FusedLayout f;
  const FusedArgs a = soft_args(s, ws, L, P, tau, kcap, ids, vnorm, norm_dtype, &f);
  const int f16 = norm_dtype == HST_F16;
  char* base = static_cast<char*>(ws);
  int32_t* cand = reinterpret_cast<int32_t*>(base + align256(f.bytes));
  const size_t ncand = static_cast<size_t>(s.B) * s.Hkv * static_cast<size_t>(kcap) * 4;
  double* logits = reinterpret_cast<double*>(base + align256(f.bytes) + align256(ncand));
  HST_CHECK(launch_prep_soft(s, a, q, W, ids, kps, st));
  HST_CHECK(launch_scan(s, a, f.kind, ids, vnorm, f16, nullptr, 1, kps, st));
  HST_CHECK(launch_select_only(s, a, cand, nullptr, 0, f.chunk, st));
  HST_CHECK(launch_select_mass(s, q, K, cand, kcap, p, scale, idx, counts, logits, st));
  return launch_attend(s, a, q, K, V, idx, false, nullptr, 0, f.chunk, scale, out, lse, st);
}

hipError_t build_cards_softlsh(const hst_shape& s, const void* K, const void* vnorm, int norm_dtype,
                               const void* W, int L, int P, void* ckeys, uint8_t* cids, void* cw,
                               int32_t* clens, hipStream_t st) {
  HST_CHECK(launch_card_sums(s, K, vnorm, norm_dtype == HST_F16, ckeys, cw, clens, st));
  hst_shape sc = s;
  sc.Nmax = route_chunks(s.Nmax);
  sc.seq_lens = clens;
  return launch_hash_ids_softlsh(sc, ckeys, W, L, P, cids, st);
}

// Workspace of the routed step: tables, the attention partials, the kept
// chunks and the scores of their keys.
struct RouteLayout {
  size_t tables, cpart, attn, chunks, tscore, bytes;
};

static RouteLayout route_layout(const hst_shape& s, int L, int P, int kcap) {
  RouteLayout r{};
  const size_t BH = static_cast<size_t>(s.B) * s.Hkv;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  r.tables = take(BH * (static_cast<size_t>(L) << P) * 4);
  r.cpart = take(BH * prep_parts(kScanSoftFast, L) * static_cast<size_t>(route_chunks(s.Nmax)) * 4);
  r.attn = take(fused_layout(s, HST_OP_SPARSE_ATTENTION, 0, 0, kcap).bytes);
  r.chunks = take(BH * kRouteMaxChunks * 4);
  r.tscore = take(BH * kRouteMaxChunks * 64 * 4);
  r.bytes = o;
  return r;
}

size_t route_ws_bytes(const hst_shape& s, int L, int P, int kcap) {
  return route_layout(s, L, P, kcap).bytes;
}

hipError_t fused_decode_softlsh_routed(const hst_shape& s, const void* q, const void* K,
                                       const void* V, const void* W, int L, int P, double tau,
                                       const uint8_t* ids, const void* vnorm, int norm_dtype,
                                       const uint8_t* cids, const void* cw, int C, int kcap,
                                       const int32_t* kps, float scale, int32_t* idx, float* out,
                                       float* lse, void* ws, hipStream_t st) {
  const RouteLayout r = route_layout(s, L, P, kcap);
  char* base = static_cast<char*>(ws);
  float* tables = reinterpret_cast<float*>(base + r.tables);
  int32_t* chunks = reinterpret_cast<int32_t*>(base + r.chunks);
  float* tscore = reinterpret_cast<float*>(base + r.tscore);
  const int f16 = norm_dtype == HST_F16;
  // query tables, and every card scored on each prep workgroup's tables
  const FusedLayout fs = fused_layout(s, HST_OP_SCORE_SOFTLSH, L, P, 1);
  FusedArgs as = make_args(s, fs, nullptr, L, P, tau, 1);
  as.tables = tables;
  as.xparts = prep_parts(kScanSoftFast, L);
  as.cids = cids;
  as.cpart = reinterpret_cast<float*>(base + r.cpart);
  as.ncards = route_chunks(s.Nmax);
  HST_CHECK(launch_prep_soft(s, as, q, W, nullptr, nullptr, st));
  // the C best chunks kept; then the k best keys inside
  HST_CHECK(launch_card_route(s, as.cpart, as.xparts, cw, f16, C, chunks, st));
  HST_CHECK(launch_route_scan(s, tables, chunks, C, ids, vnorm, f16, L, P, C * 64, tscore, st));
  HST_CHECK(launch_token_route(s, tscore, C * 64, chunks, C, kcap, kps, idx, st));
  // exact attention over the original rows
  const FusedLayout fa = fused_layout(s, HST_OP_SPARSE_ATTENTION, 0, 0, kcap);
  const FusedArgs aa = make_args(s, fa, base + r.attn, 0, 0, 0.0, kcap);
  return launch_attend(s, aa, q, K, V, idx, false, nullptr, 0, fa.chunk, scale, out, lse, st);
}

// Workspace of the shared-prefix step: tables, the context lengths, the
// scores of every context key, the selection's workspace, the attention
// partials.
struct SharedLayout {
  size_t tables, vlens, scores, select, attn, bytes;
};

static hst_shape shared_context_shape(const hst_shape& s, int Np, const int32_t* vlens) {
  hst_shape v = s;
  v.Nmax = Np + s.Nmax;
  v.seq_lens = s.seq_lens != nullptr ? vlens : nullptr;
  return v;
}

static SharedLayout shared_layout(const hst_shape& s, int Np, int L, int P, int kcap) {
  SharedLayout r{};
  const size_t BH = static_cast<size_t>(s.B) * s.Hkv;
  const hst_shape v = shared_context_shape(s, Np, nullptr);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  r.tables = take(BH * (static_cast<size_t>(L) << P) * 4);
  r.vlens = take(static_cast<size_t>(s.B) * 4);
  r.scores = take(BH * static_cast<size_t>(v.Nmax) * 4);
  r.select = take(fused_layout(v, HST_OP_SELECT_TOPK, 0, 0, kcap).bytes);
  r.attn = take(fused_layout(s, HST_OP_SPARSE_ATTENTION, 0, 0, kcap).bytes);
  r.bytes = o;
  return r;
}

size_t shared_ws_bytes(const hst_shape& s, int Np, int L, int P, int kcap) {
  return shared_layout(s, Np, L, P, kcap).bytes;
}

hipError_t fused_decode_softlsh_shared(const hst_shape& s, int Np, const void* q, const void* Kp,
                                       const void* Vp, const uint8_t* ids_p, const void* vn_p,
                                       const void* Ks, const void* Vs, const uint8_t* ids_s,
                                       const void* vn_s, const void* W, int L, int P, double tau,
                                       int norm_dtype, int kcap, const int32_t* kps, float scale,
                                       int32_t* idx, float* out, float* lse, void* ws,
                                       hipStream_t st) {
  const SharedLayout r = shared_layout(s, Np, L, P, kcap);
  char* base = static_cast<char*>(ws);
  float* tables = reinterpret_cast<float*>(base + r.tables);
  int32_t* vlens = reinterpret_cast<int32_t*>(base + r.vlens);
  float* scores = reinterpret_cast<float*>(base + r.scores);
  const hst_shape v = shared_context_shape(s, Np, vlens);
  // query tables, context lengths, the scores of every context key
  const FusedLayout fs = fused_layout(s, HST_OP_SCORE_SOFTLSH, L, P, 1);
  FusedArgs as = make_args(s, fs, nullptr, L, P, tau, 1);
  as.tables = tables;
  HST_CHECK(launch_prep_soft(s, as, q, W, nullptr, nullptr, st));
  if (s.seq_lens != nullptr) HST_CHECK(launch_shared_lens(s, Np, vlens, st));
  HST_CHECK(launch_scan_shared(s, as, Np, ids_p, vn_p, ids_s, vn_s, norm_dtype == HST_F16, scores,
                               st));
  // exact top-k over the whole context
  HST_CHECK(fused_select(v, HST_F32, scores, kcap, kps, idx, base + r.select, st));
  // attention: rows below Np from the prefix cache
  const FusedLayout fa = fused_layout(s, HST_OP_SPARSE_ATTENTION, 0, 0, kcap);
  FusedArgs aa = make_args(s, fa, base + r.attn, 0, 0, 0.0, kcap);
  aa.pk = Kp;
  aa.pv = Vp;
  aa.np = Np;
  return launch_attend(s, aa, q, Ks, Vs, idx, false, nullptr, 0, fa.chunk, scale, out, lse, st);
}

// Workspace of the binary-code path for 64 / 256-bit codes: query codes,
// then (decode) the scores, the selection's workspace and the attention
// partials.
struct CodesLayout {
  size_t qcodes, scores, select, attn, bytes;
};

static CodesLayout codes_layout(const hst_shape& s, int code_bits, int kcap, bool decode) {
  CodesLayout r{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += align256(bytes);
    return at;
  };
  r.qcodes = take(static_cast<size_t>(s.B) * s.Hq * (code_bits / 32) * 4);
  if (decode) {
    r.scores = take(static_cast<size_t>(s.B) * s.Hkv * s.Nmax * 4);
    r.select = take(fused_layout(s, HST_OP_SELECT_TOPK, 0, 0, kcap).bytes);
    r.attn = take(fused_layout(s, HST_OP_SPARSE_ATTENTION, 0, 0, kcap).bytes);
  }
  r.bytes = o;
  return r;
}

size_t codes_ws_bytes(const hst_shape& s, int code_bits, int kcap, bool decode) {
  return codes_layout(s, code_bits, kcap, decode).bytes;
}

hipError_t codes_score(const hst_shape& s, const void* q, const void* R, int code_bits,
                       const uint32_t* codes, int32_t* scores, void* ws, hipStream_t st) {
  const CodesLayout r = codes_layout(s, code_bits, 1, false);
  uint32_t* qc = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + r.qcodes);
  HST_CHECK(launch_query_codes(s, q, R, code_bits, qc, st));
  return launch_hamming_scan(s, code_bits, qc, codes, scores, st);
}

hipError_t codes_decode(const hst_shape& s, const void* q, const void* K, const void* V,
                        const void* R, int code_bits, const uint32_t* codes, int kcap,
                        const int32_t* kps, float scale, int32_t* idx, float* out, float* lse,
                        void* ws, hipStream_t st) {
  const CodesLayout r = codes_layout(s, code_bits, kcap, true);
  char* base = static_cast<char*>(ws);
  uint32_t* qc = reinterpret_cast<uint32_t*>(base + r.qcodes);
  int32_t* scores = reinterpret_cast<int32_t*>(base + r.scores);
  HST_CHECK(launch_query_codes(s, q, R, code_bits, qc, st));
  HST_CHECK(launch_hamming_scan(s, code_bits, qc, codes, scores, st));
  HST_CHECK(fused_select(s, HST_I32, scores, kcap, kps, idx, base + r.select, st));
  const FusedLayout fa = fused_layout(s, HST_OP_SPARSE_ATTENTION, 0, 0, kcap);
  const FusedArgs aa = make_args(s, fa, base + r.attn, 0, 0, 0.0, kcap);
  return launch_attend(s, aa, q, K, V, idx, false, nullptr, 0, fa.chunk, scale, out, lse, st);
}

hipError_t fused_decode_hamming(const hst_shape& s, const void* q, const void* K, const void* V,
                                const void* R, const uint32_t* codes, int kcap, const int32_t* kps,
                                float scale, int32_t* idx, float* out, float* lse, void* ws,
                                hipStream_t st) {
  HST_CHECK(decode_prepare_hamming(s, q, R, codes, kcap, kps, ws, st));
  HST_CHECK(decode_filter_hamming(s, codes, kcap, kps, ws, st));
  return decode_finish_hamming(s, q, K, V, codes, kcap, scale, idx, out, lse, ws, st);
}

static FusedArgs ham_args(const hst_shape& s, void* ws, int kcap, const uint32_t* codes, FusedLayout* fo) {
  const FusedLayout f = fused_layout(s, HST_OP_DECODE_HAMMING, 0, 0, kcap);
  FusedArgs a = make_args(s, f, ws, 0, 0, 0.0, kcap);
  a.meta = codes;
  a.meta_kind = kScanHamming;
  if (fo != nullptr) *fo = f;
  return a;
}

hipError_t decode_prepare_hamming(const hst_shape& s, const void* q, const void* R,
                                  const uint32_t* codes, int kcap, const int32_t* kps, void* ws,
                                  hipStream_t st) {
  const FusedArgs a = ham_args(s, ws, kcap, codes, nullptr);
  return launch_prep_hamming(s, a, q, R, codes, kps, st);
}

hipError_t decode_filter_hamming(const hst_shape& s, const uint32_t* codes, int kcap,
                                 const int32_t* kps, void* ws, hipStream_t st) {
  const FusedArgs a = ham_args(s, ws, kcap, codes, nullptr);
  return launch_scan(s, a, kScanHamming, codes, nullptr, 0, nullptr, 1, kps, st);
}

hipError_t decode_finish_hamming(const hst_shape& s, const void* q, const void* K, const void* V,
                                 const uint32_t* codes, int kcap, float scale, int32_t* idx,
                                 float* out, float* lse, void* ws, hipStream_t st) {
  FusedLayout f;
  const FusedArgs a = ham_args(s, ws, kcap, codes, &f);
  return launch_attend(s, a, q, K, V, idx, true, nullptr, 1, f.chunk, scale, out, lse, st);
}

hipError_t decode_candidates(const hst_shape& s, int op, int L, int P, int kcap, void* ws,
                             uint32_t* keys, int32_t* index, int32_t* count, uint32_t* theta,
                             int cap, hipStream_t st) {
  const bool soft = op == HST_OP_DECODE_SOFTLSH;
  const FusedLayout f = fused_layout(s, soft ? HST_OP_DECODE_SOFTLSH : HST_OP_DECODE_HAMMING,
                                     soft ? L : 0, soft ? P : 0, kcap);
  const FusedArgs a = make_args(s, f, ws, soft ? L : 0, soft ? P : 0, 0.0, kcap);
  return launch_candidates(s, a, f.chunk, keys, index, count, theta, cap, st);
}

hipError_t fused_score_softlsh(const hst_shape& s, const void* q, const void* W, int L, int P,
                               double tau, const uint8_t* ids, const void* vnorm, int norm_dtype,
                               float* scores, void* ws, hipStream_t st) {
  const FusedLayout f = fused_layout(s, HST_OP_SCORE_SOFTLSH, L, P, 1);
  const FusedArgs a = make_args(s, f, ws, L, P, tau, 1);
  HST_CHECK(launch_prep_soft(s, a, q, W, nullptr, nullptr, st));
  return launch_scan(s, a, f.kind, ids, vnorm, norm_dtype == HST_F16, scores, 0, nullptr, st);
}

hipError_t fused_score_hamming(const hst_shape& s, const void* q, const void* R,
                               const uint32_t* codes, int32_t* scores, void* ws, hipStream_t st) {
  const FusedLayout f = fused_layout(s, HST_OP_SCORE_HAMMING, 0, 0, 1);
  const FusedArgs a = make_args(s, f, ws, 0, 0, 0.0, 1);
  HST_CHECK(launch_prep_hamming(s, a, q, R, codes, nullptr, st));
  return launch_scan(s, a, kScanHamming, codes, nullptr, 0, scores, 0, nullptr, st);
}

hipError_t fused_tables_softlsh(const hst_shape& s, const void* q, const void* W, int L, int P,
                                double tau, float* tables, hipStream_t st) {
  const FusedLayout f = fused_layout(s, HST_OP_SCORE_SOFTLSH, L, P, 1);
  FusedArgs a = make_args(s, f, nullptr, L, P, tau, 1);
  a.tables = tables;
  return launch_prep_soft(s, a, q, W, nullptr, nullptr, st);
}

hipError_t fused_scan_softlsh(const hst_shape& s, const float* tables, int L, int P,
                              const uint8_t* ids, const void* vnorm, int norm_dtype, float* scores,
                              hipStream_t st) {
  const FusedLayout f = fused_layout(s, HST_OP_SCORE_SOFTLSH, L, P, 1);
  FusedArgs a = make_args(s, f, nullptr, L, P, 0.0, 1);
  a.tables = const_cast<float*>(tables);
  return launch_scan(s, a, f.kind, ids, vnorm, norm_dtype == HST_F16, scores, 0, nullptr, st);
}

hipError_t fused_select(const hst_shape& s, int score_dtype, const void* scores, int kcap,
                        const int32_t* kps, int32_t* idx, void* ws, hipStream_t st) {
  const FusedLayout f = fused_layout(s, HST_OP_SELECT_TOPK, 0, 0, kcap);
  const FusedArgs a = make_args(s, f, ws, 0, 0, 0.0, kcap);
  const int is_int = score_dtype == HST_I32;
  HST_CHECK(launch_prep_given(s, a, score_dtype, scores, kps, st));
  HST_CHECK(launch_scan(s, a, is_int ? kScanGivenI32 : kScanGivenF32, scores, nullptr, 0, nullptr, 1, kps, st));
  return launch_select_only(s, a, idx, scores, is_int, f.chunk, st);
}

hipError_t fused_attention(const hst_shape& s, const void* q, const void* K, const void* V,
                           const int32_t* idx, int kcap, float scale, float* out, float* lse,
                           void* ws, hipStream_t st) {
  const FusedLayout f = fused_layout(s, HST_OP_SPARSE_ATTENTION, 0, 0, kcap);
  const FusedArgs a = make_args(s, f, ws, 0, 0, 0.0, kcap);
  return launch_attend(s, a, q, K, V, const_cast<int32_t*>(idx), false, nullptr, 0, f.chunk, scale,
                       out, lse, st);
}

}  // namespace hst
