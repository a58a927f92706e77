// C ABI of libhst: argument validation, workspace layout and launch order.
// Validation is pure host logic and finishes before anything is enqueued.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "hst.h"
#include "hst_fused.h"
#include "hst_launch.h"

#ifdef HST_DEBUG
namespace hst {
__device__ uint32_t hst_debug_word = 0u;  // first failed check of the debug build (see hst_common.h)
}
#endif

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool ptr_ok(const void* p) { return p != nullptr && aligned16(p); }

hst_status hip_status(hipError_t e) {
  if (e == hipSuccess) return HST_OK;
  g_last_hip_error = static_cast<int>(e);
  return HST_ERR_HIP;
}

hst_status check_shape(const hst_shape* s) {
  if (s == nullptr) return HST_ERR_INVALID_ARG;
  if (s->B < 1 || s->Hkv < 1 || s->Hq < 1 || s->Nmax < 1 || s->d < 1) return HST_ERR_INVALID_ARG;
  if (s->Hq % s->Hkv != 0) return HST_ERR_INVALID_ARG;
  if (s->kv_dtype != HST_F32 && s->kv_dtype != HST_BF16) return HST_ERR_UNSUPPORTED;
  if (s->d != 64 && s->d != 128) return HST_ERR_UNSUPPORTED;
  if (static_cast<long long>(s->B) * s->Hkv > 65535) return HST_ERR_UNSUPPORTED;
  if (static_cast<long long>(s->B) * s->Hq > 0x7fffffffLL) return HST_ERR_UNSUPPORTED;
  if (s->Nmax > (1 << 30)) return HST_ERR_UNSUPPORTED;
  if (s->seq_lens != nullptr && !aligned16(s->seq_lens)) return HST_ERR_INVALID_ARG;
  return HST_OK;
}

hst_status check_lp(int L, int P) {
  if (L < 1 || P < 1) return HST_ERR_INVALID_ARG;
  if (P > 8 || L > 128 || (static_cast<long long>(L) << P) > 16384) return HST_ERR_UNSUPPORTED;
  return HST_OK;
}

hst_status check_norm_dtype(int nd) {
  if (nd != HST_F16 && nd != HST_F32) return HST_ERR_UNSUPPORTED;
  return HST_OK;
}

int group(const hst_shape* s) { return s->Hq / s->Hkv; }

// Limits of the per-head query preprocessing (its LDS holds G*L*P float64
// projections and G*d float64 query components).
hst_status check_soft_prep(const hst_shape* s, int L, int P) {
  if (static_cast<long long>(group(s)) * L * P > 4096) return HST_ERR_UNSUPPORTED;
  if (static_cast<long long>(group(s)) * s->d > 1024) return HST_ERR_UNSUPPORTED;
  return HST_OK;
}

#define HST_TRY(x)                       \
  do {                                   \
    hst_status _st = (x);                \
    if (_st != HST_OK) return _st;       \
  } while (0)

// the routed step: fast table scan shapes, tables that fit the scan LDS,
// at most 16384 cards per head
hst_status check_route(const hst_shape* s, int L, int P) {
  HST_TRY(check_lp(L, P));
  if (L != 16 && L != 32 && L != 64 && L != 128) return HST_ERR_UNSUPPORTED;
  if ((static_cast<long long>(L) << P) * 4 > 131072) return HST_ERR_UNSUPPORTED;
  if (hst::route_chunks(s->Nmax) > hst::kRouteMaxCards) return HST_ERR_UNSUPPORTED;
  if (hst::card_route_smem(hst::route_chunks(s->Nmax)) > 160 * 1024 - 2048)
    return HST_ERR_UNSUPPORTED;  // the card cut holds keys, candidates and histogram in LDS
  return HST_OK;
}


}  // namespace

extern "C" {

int hst_version(void) { return 100; }

const char* hst_status_string(int status) {
  switch (status) {
    case HST_OK: return "HST_OK";
    case HST_ERR_INVALID_ARG: return "HST_ERR_INVALID_ARG: invalid argument";
    case HST_ERR_UNSUPPORTED: return "HST_ERR_UNSUPPORTED: unsupported shape or dtype";
    case HST_ERR_WORKSPACE: return "HST_ERR_WORKSPACE: workspace too small";
    case HST_ERR_HIP: return "HST_ERR_HIP: HIP launch failed";
    default: return "unknown hst_status";
  }
}

int hst_last_hip_error(void) { return g_last_hip_error; }

hst_status hst_debug_status(uint32_t* code) {
  if (code == nullptr) return HST_ERR_INVALID_ARG;
#ifdef HST_DEBUG
  uint32_t v = 0u;
  hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(hst::hst_debug_word), sizeof(v), 0, hipMemcpyDeviceToHost);
  if (e == hipSuccess) {
    const uint32_t zero = 0u;
    e = hipMemcpyToSymbol(HIP_SYMBOL(hst::hst_debug_word), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
  }
  if (e != hipSuccess) {
    g_last_hip_error = static_cast<int>(e);
    return HST_ERR_HIP;
  }
  *code = v;
  return HST_OK;
#else
  *code = 0u;
  return HST_ERR_UNSUPPORTED;
#endif
}

hst_status hst_workspace_size(int op, const hst_shape* shape, int L, int P, int code_bits, int k,
                              size_t* bytes) {
  if (bytes == nullptr) return HST_ERR_INVALID_ARG;
  HST_TRY(check_shape(shape));
  const bool soft = op == HST_OP_SCORE_SOFTLSH || op == HST_OP_DECODE_SOFTLSH ||
                    op == HST_OP_HASH_SOFTLSH;
  const bool bin = op == HST_OP_SCORE_HAMMING || op == HST_OP_DECODE_HAMMING ||
                   op == HST_OP_HASH_BINARY;
  if (soft) HST_TRY(check_lp(L, P));
  if (bin && code_bits != 64 && code_bits != 128 && code_bits != 256) return HST_ERR_UNSUPPORTED;
  const bool mass = op == HST_OP_SELECT_MASS || op == HST_OP_DECODE_SOFTLSH_MASS;
  const bool needk = op == HST_OP_SELECT_TOPK || op == HST_OP_SPARSE_ATTENTION ||
                     op == HST_OP_DECODE_SOFTLSH || op == HST_OP_DECODE_HAMMING || mass;
  if (needk && k < 1) return HST_ERR_INVALID_ARG;
  if (needk && k > hst::kMaxSplits * 1024) return HST_ERR_UNSUPPORTED;
  if (mass && k > hst::kMassCap) return HST_ERR_UNSUPPORTED;
  const bool routed = op == HST_OP_DECODE_SOFTLSH_ROUTED;
  if (routed) {
    if (k < 1) return HST_ERR_INVALID_ARG;
    HST_TRY(check_route(shape, L, P));
  }
  if (op == HST_OP_DECODE_SOFTLSH_MASS) {
    HST_TRY(check_lp(L, P));
    HST_TRY(check_soft_prep(shape, L, P));
  }
  if (soft && op != HST_OP_HASH_SOFTLSH) HST_TRY(check_soft_prep(shape, L, P));
  size_t b = 0;
  switch (op) {
    case HST_OP_HASH_SOFTLSH:
    case HST_OP_HASH_BINARY: b = 0; break;
    case HST_OP_SCORE_HAMMING:
    case HST_OP_DECODE_HAMMING:
      if (code_bits != 128) {  // 64 / 256 bits: query codes, scan, selection, attention
        if (op == HST_OP_DECODE_HAMMING &&
            hst::fused_layout(*shape, HST_OP_SELECT_TOPK, 0, 0, k).nchunks > hst::kMaxChunks)
          return HST_ERR_UNSUPPORTED;
        b = align_up(hst::codes_ws_bytes(*shape, code_bits, needk ? k : 1,
                                         op == HST_OP_DECODE_HAMMING));
        break;
      }
      [[fallthrough]];
    case HST_OP_SCORE_SOFTLSH:
    case HST_OP_SELECT_TOPK:
    case HST_OP_SPARSE_ATTENTION:
    case HST_OP_DECODE_SOFTLSH: {
      const hst::FusedLayout f = hst::fused_layout(*shape, op, L, P, needk ? k : 1);
      if (f.nchunks > hst::kMaxChunks) return HST_ERR_UNSUPPORTED;
      b = align_up(f.bytes);
      break;
    }
    case HST_OP_SELECT_MASS: b = align_up(hst::mass_logits_bytes(*shape, k)); break;
    case HST_OP_DECODE_SOFTLSH_ROUTED: b = align_up(hst::route_ws_bytes(*shape, L, P, k)); break;
    case HST_OP_DECODE_SOFTLSH_MASS: {
      const hst::FusedLayout f = hst::fused_layout(*shape, HST_OP_DECODE_SOFTLSH, L, P, k);
      if (f.nchunks > hst::kMaxChunks) return HST_ERR_UNSUPPORTED;
      b = align_up(hst::decode_mass_bytes(*shape, L, P, k));
      break;
    }
    default: return HST_ERR_INVALID_ARG;
  }
  *bytes = b;
  return HST_OK;
}

hst_status hst_hash_keys_softlsh(const hst_shape* shape, const void* K, const void* V,
                                 const void* W, int L, int P, int norm_dtype, uint8_t* ids,
                                 void* vnorm, void* stream) {
  HST_TRY(check_shape(shape));
  // hashing alone has no table-size limit: ids are bytes (P <= 8), at most 1024 tables
  if (L < 1 || P < 1) return HST_ERR_INVALID_ARG;
  if (P > 8 || L > 1024) return HST_ERR_UNSUPPORTED;
  HST_TRY(check_norm_dtype(norm_dtype));
  if (!ptr_ok(K) || !ptr_ok(V) || !ptr_ok(W) || !ptr_ok(ids) || !ptr_ok(vnorm))
    return HST_ERR_INVALID_ARG;
  return hip_status(hst::launch_hash_softlsh(*shape, K, V, W, L, P, norm_dtype, ids, vnorm,
                                             static_cast<hipStream_t>(stream)));
}

hst_status hst_hash_keys_binary(const hst_shape* shape, const void* K, const void* R,
                                int code_bits, uint32_t* codes, void* stream) {
  HST_TRY(check_shape(shape));
  if (code_bits != 64 && code_bits != 128 && code_bits != 256) return HST_ERR_UNSUPPORTED;
  if (!ptr_ok(K) || !ptr_ok(R) || !ptr_ok(codes)) return HST_ERR_INVALID_ARG;
  return hip_status(
      hst::launch_hash_binary(*shape, K, R, code_bits, codes, static_cast<hipStream_t>(stream)));
}

hst_status hst_append_kv_softlsh(const hst_shape* shape, const void* k_new, const void* v_new,
                                 const void* W, int L, int P, int norm_dtype, void* K, void* V,
                                 uint8_t* ids, void* vnorm, void* stream) {
  HST_TRY(check_shape(shape));
  if (L < 1 || P < 1) return HST_ERR_INVALID_ARG;
  if (P > 8 || L > 1024) return HST_ERR_UNSUPPORTED;
  HST_TRY(check_norm_dtype(norm_dtype));
  if (shape->seq_lens == nullptr) return HST_ERR_INVALID_ARG;  // the lengths advance in place
  if (!ptr_ok(k_new) || !ptr_ok(v_new) || !ptr_ok(W) || !ptr_ok(K) || !ptr_ok(V) || !ptr_ok(ids) ||
      !ptr_ok(vnorm))
    return HST_ERR_INVALID_ARG;
  return hip_status(hst::launch_append_softlsh(*shape, k_new, v_new, W, L, P, norm_dtype, K, V, ids,
                                               vnorm, static_cast<hipStream_t>(stream)));
}

hst_status hst_append_kv_binary(const hst_shape* shape, const void* k_new, const void* v_new,
                                const void* R, int code_bits, void* K, void* V, uint32_t* codes,
                                void* stream) {
  HST_TRY(check_shape(shape));
  if (code_bits != 128) return HST_ERR_UNSUPPORTED;
  if (shape->seq_lens == nullptr) return HST_ERR_INVALID_ARG;  // the lengths advance in place
  if (!ptr_ok(k_new) || !ptr_ok(v_new) || !ptr_ok(R) || !ptr_ok(K) || !ptr_ok(V) || !ptr_ok(codes))
    return HST_ERR_INVALID_ARG;
  return hip_status(hst::launch_append_binary(*shape, k_new, v_new, R, K, V, codes,
                                              static_cast<hipStream_t>(stream)));
}

static hst_status score_softlsh_checks(const hst_shape* shape, const void* q, const void* W, int L,
                                       int P, double tau, const uint8_t* ids, const void* vnorm,
                                       int norm_dtype) {
  HST_TRY(check_shape(shape));
  HST_TRY(check_lp(L, P));
  HST_TRY(check_norm_dtype(norm_dtype));
  if (!(tau > 0.0) || !isfinite(tau)) return HST_ERR_INVALID_ARG;
  HST_TRY(check_soft_prep(shape, L, P));
  if (!ptr_ok(q) || !ptr_ok(W) || !ptr_ok(ids) || !ptr_ok(vnorm)) return HST_ERR_INVALID_ARG;
  return HST_OK;
}

static hst_status score_hamming_checks(const hst_shape* shape, const void* q, const void* R,
                                       int code_bits, const uint32_t* codes) {
  HST_TRY(check_shape(shape));
  if (code_bits != 64 && code_bits != 128 && code_bits != 256) return HST_ERR_UNSUPPORTED;
  if (group(shape) > (code_bits == 128 ? 64 : 8)) return HST_ERR_UNSUPPORTED;
  if (!ptr_ok(q) || !ptr_ok(R) || !ptr_ok(codes)) return HST_ERR_INVALID_ARG;
  return HST_OK;
}

static hst_status attention_checks(const hst_shape* shape, const void* q, const void* K,
                                   const void* V, int k, float scale, float* out, float* lse) {
  HST_TRY(check_shape(shape));
  if (group(shape) > 8) return HST_ERR_UNSUPPORTED;
  if (k < 1 || !isfinite(scale)) return HST_ERR_INVALID_ARG;
  if (!ptr_ok(q) || !ptr_ok(K) || !ptr_ok(V) || !ptr_ok(out)) return HST_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned16(lse)) return HST_ERR_INVALID_ARG;
  return HST_OK;
}

static hst_status workspace_check(int op, const hst_shape* shape, int L, int P, int k, void* ws,
                                  size_t ws_bytes, int code_bits = 128) {
  size_t need = 0;
  HST_TRY(hst_workspace_size(op, shape, L, P, code_bits, k, &need));
  if (ws_bytes < need) return HST_ERR_WORKSPACE;
  if (need > 0 && (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0))
    return HST_ERR_INVALID_ARG;
  return HST_OK;
}

hst_status hst_score_keys_softlsh(const hst_shape* shape, const void* q, const void* W, int L,
                                  int P, double tau, const uint8_t* ids, const void* vnorm,
                                  int norm_dtype, float* scores, void* ws, size_t ws_bytes,
                                  void* stream) {
  HST_TRY(score_softlsh_checks(shape, q, W, L, P, tau, ids, vnorm, norm_dtype));
  if (!ptr_ok(scores)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_SCORE_SOFTLSH, shape, L, P, 1, ws, ws_bytes));
  return hip_status(hst::fused_score_softlsh(*shape, q, W, L, P, tau, ids, vnorm, norm_dtype,
                                             scores, ws, static_cast<hipStream_t>(stream)));
}

hst_status hst_query_tables_softlsh(const hst_shape* shape, const void* q, const void* W, int L,
                                    int P, double tau, float* tables, void* stream) {
  HST_TRY(check_shape(shape));
  HST_TRY(check_lp(L, P));
  if (!(tau > 0.0) || !isfinite(tau)) return HST_ERR_INVALID_ARG;
  HST_TRY(check_soft_prep(shape, L, P));
  if (!ptr_ok(q) || !ptr_ok(W) || !ptr_ok(tables)) return HST_ERR_INVALID_ARG;
  return hip_status(hst::fused_tables_softlsh(*shape, q, W, L, P, tau, tables,
                                              static_cast<hipStream_t>(stream)));
}

hst_status hst_score_scan_softlsh(const hst_shape* shape, const float* tables, int L, int P,
                                  const uint8_t* ids, const void* vnorm, int norm_dtype,
                                  float* scores, void* stream) {
  HST_TRY(check_shape(shape));
  HST_TRY(check_lp(L, P));
  HST_TRY(check_norm_dtype(norm_dtype));
  if (!ptr_ok(tables) || !ptr_ok(ids) || !ptr_ok(vnorm) || !ptr_ok(scores))
    return HST_ERR_INVALID_ARG;
  return hip_status(hst::fused_scan_softlsh(*shape, tables, L, P, ids, vnorm, norm_dtype, scores,
                                            static_cast<hipStream_t>(stream)));
}

hst_status hst_score_keys_hamming(const hst_shape* shape, const void* q, const void* R,
                                  int code_bits, const uint32_t* codes, int32_t* scores, void* ws,
                                  size_t ws_bytes, void* stream) {
  HST_TRY(score_hamming_checks(shape, q, R, code_bits, codes));
  if (!ptr_ok(scores)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_SCORE_HAMMING, shape, 0, 0, 1, ws, ws_bytes, code_bits));
  if (code_bits != 128)
    return hip_status(hst::codes_score(*shape, q, R, code_bits, codes, scores, ws,
                                       static_cast<hipStream_t>(stream)));
  return hip_status(hst::fused_score_hamming(*shape, q, R, codes, scores, ws,
                                             static_cast<hipStream_t>(stream)));
}

hst_status hst_select_topk(const hst_shape* shape, int score_dtype, const void* scores, int k,
                           const int32_t* k_per_seq, int32_t* idx, void* ws, size_t ws_bytes,
                           void* stream) {
  HST_TRY(check_shape(shape));
  if (score_dtype != HST_F32 && score_dtype != HST_I32) return HST_ERR_UNSUPPORTED;
  if (k < 1) return HST_ERR_INVALID_ARG;
  if (!ptr_ok(scores) || !ptr_ok(idx)) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_SELECT_TOPK, shape, 0, 0, k, ws, ws_bytes));
  return hip_status(hst::fused_select(*shape, score_dtype, scores, k, k_per_seq, idx, ws,
                                      static_cast<hipStream_t>(stream)));
}

hst_status hst_sparse_decode_attention(const hst_shape* shape, const void* q, const void* K,
                                       const void* V, const int32_t* idx, int k, float scale,
                                       float* out, float* lse, void* ws, size_t ws_bytes,
                                       void* stream) {
  HST_TRY(attention_checks(shape, q, K, V, k, scale, out, lse));
  if (!ptr_ok(idx)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_SPARSE_ATTENTION, shape, 0, 0, k, ws, ws_bytes));
  return hip_status(hst::fused_attention(*shape, q, K, V, idx, k, scale, out, lse, ws,
                                         static_cast<hipStream_t>(stream)));
}

hst_status hst_build_cards_softlsh(const hst_shape* shape, const void* K, const void* vnorm,
                                   int norm_dtype, const void* W, int L, int P, void* card_keys,
                                   uint8_t* card_ids, void* card_w, int32_t* card_lens,
                                   void* stream) {
  HST_TRY(check_shape(shape));
  if (L < 1 || P < 1) return HST_ERR_INVALID_ARG;
  if (P > 8 || L > 1024) return HST_ERR_UNSUPPORTED;
  HST_TRY(check_norm_dtype(norm_dtype));
  if (!ptr_ok(K) || !ptr_ok(vnorm) || !ptr_ok(W) || !ptr_ok(card_keys) || !ptr_ok(card_ids) ||
      !ptr_ok(card_w) || !ptr_ok(card_lens))
    return HST_ERR_INVALID_ARG;
  return hip_status(hst::build_cards_softlsh(*shape, K, vnorm, norm_dtype, W, L, P, card_keys,
                                             card_ids, card_w, card_lens,
                                             static_cast<hipStream_t>(stream)));
}

hst_status hst_decode_step_softlsh_routed(const hst_shape* shape, const void* q, const void* K,
                                          const void* V, const void* W, int L, int P, double tau,
                                          const uint8_t* ids, const void* vnorm, int norm_dtype,
                                          const uint8_t* card_ids, const void* card_w, int C,
                                          int k, const int32_t* k_per_seq, float scale,
                                          int32_t* idx, float* out, float* lse, void* ws,
                                          size_t ws_bytes, void* stream) {
  HST_TRY(score_softlsh_checks(shape, q, W, L, P, tau, ids, vnorm, norm_dtype));
  HST_TRY(attention_checks(shape, q, K, V, k, scale, out, lse));
  HST_TRY(check_route(shape, L, P));
  if (C < 1) return HST_ERR_INVALID_ARG;
  if (C > hst::kRouteMaxChunks) return HST_ERR_UNSUPPORTED;
  if (!ptr_ok(idx) || !ptr_ok(card_ids) || !ptr_ok(card_w)) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_DECODE_SOFTLSH_ROUTED, shape, L, P, k, ws, ws_bytes));
  return hip_status(hst::fused_decode_softlsh_routed(*shape, q, K, V, W, L, P, tau, ids, vnorm,
                                                     norm_dtype, card_ids, card_w, C, k,
                                                     k_per_seq, scale, idx, out, lse, ws,
                                                     static_cast<hipStream_t>(stream)));
}

static hst_status shared_checks(const hst_shape* shape, int Np, int L, int P, int k,
                                size_t* need) {
  HST_TRY(check_shape(shape));
  if (Np < 0 || k < 1) return HST_ERR_INVALID_ARG;
  if (static_cast<long long>(Np) + shape->Nmax > (1 << 30)) return HST_ERR_UNSUPPORTED;
  HST_TRY(check_lp(L, P));
  if (L != 16 && L != 32 && L != 64 && L != 128) return HST_ERR_UNSUPPORTED;
  if ((static_cast<long long>(L) * ((1 << P) + 1)) * 4 > 160 * 1024 - 1024) return HST_ERR_UNSUPPORTED;
  HST_TRY(check_soft_prep(shape, L, P));
  // the selection runs over the whole context
  hst_shape v = *shape;
  v.Nmax = Np + shape->Nmax;
  v.seq_lens = nullptr;
  size_t sel = 0;
  HST_TRY(hst_workspace_size(HST_OP_SELECT_TOPK, &v, 0, 0, 128, k, &sel));
  size_t att = 0;
  HST_TRY(hst_workspace_size(HST_OP_SPARSE_ATTENTION, shape, 0, 0, 128, k, &att));
  *need = align_up(hst::shared_ws_bytes(*shape, Np, L, P, k));
  return HST_OK;
}

hst_status hst_workspace_size_shared(const hst_shape* shape, int Np, int L, int P, int k,
                                     size_t* bytes) {
  if (bytes == nullptr) return HST_ERR_INVALID_ARG;
  size_t need = 0;
  HST_TRY(shared_checks(shape, Np, L, P, k, &need));
  *bytes = need;
  return HST_OK;
}

hst_status hst_decode_step_softlsh_shared(const hst_shape* shape, int Np, const void* q,
                                          const void* Kp, const void* Vp, const uint8_t* ids_p,
                                          const void* vnorm_p, const void* Ks, const void* Vs,
                                          const uint8_t* ids_s, const void* vnorm_s,
                                          const void* W, int L, int P, double tau,
                                          int norm_dtype, int k, const int32_t* k_per_seq,
                                          float scale, int32_t* idx, float* out, float* lse,
                                          void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  HST_TRY(shared_checks(shape, Np, L, P, k, &need));
  HST_TRY(score_softlsh_checks(shape, q, W, L, P, tau, ids_s, vnorm_s, norm_dtype));
  HST_TRY(attention_checks(shape, q, Ks, Vs, k, scale, out, lse));
  if (Np > 0 && (!ptr_ok(Kp) || !ptr_ok(Vp) || !ptr_ok(ids_p) || !ptr_ok(vnorm_p)))
    return HST_ERR_INVALID_ARG;
  if (!ptr_ok(idx)) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  if (ws_bytes < need) return HST_ERR_WORKSPACE;
  if (ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return HST_ERR_INVALID_ARG;
  return hip_status(hst::fused_decode_softlsh_shared(
      *shape, Np, q, Kp, Vp, ids_p, vnorm_p, Ks, Vs, ids_s, vnorm_s, W, L, P, tau, norm_dtype, k,
      k_per_seq, scale, idx, out, lse, ws, static_cast<hipStream_t>(stream)));
}

static hst_status mass_p_check(double p) {
  return (p > 0.0 && p <= 1.0) ? HST_OK : HST_ERR_INVALID_ARG;  // NaN fails both
}

hst_status hst_select_mass(const hst_shape* shape, const void* q, const void* K,
                           const int32_t* cand, int k, double p, float scale, int32_t* idx,
                           int32_t* counts, void* ws, size_t ws_bytes, void* stream) {
  HST_TRY(check_shape(shape));
  if (group(shape) > 8) return HST_ERR_UNSUPPORTED;
  if (k < 1 || !isfinite(scale)) return HST_ERR_INVALID_ARG;
  HST_TRY(mass_p_check(p));
  if (!ptr_ok(q) || !ptr_ok(K) || !ptr_ok(cand) || !ptr_ok(idx) || !ptr_ok(counts))
    return HST_ERR_INVALID_ARG;
  if (cand == idx) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_SELECT_MASS, shape, 0, 0, k, ws, ws_bytes));
  return hip_status(hst::launch_select_mass(*shape, q, K, cand, k, p, scale, idx, counts,
                                            static_cast<double*>(ws),
                                            static_cast<hipStream_t>(stream)));
}

hst_status hst_decode_step_softlsh_mass(const hst_shape* shape, const void* q, const void* K,
                                        const void* V, const void* W, int L, int P, double tau,
                                        const uint8_t* ids, const void* vnorm, int norm_dtype,
                                        int k, const int32_t* k_per_seq, double p, float scale,
                                        int32_t* idx, int32_t* counts, float* out, float* lse,
                                        void* ws, size_t ws_bytes, void* stream) {
  HST_TRY(score_softlsh_checks(shape, q, W, L, P, tau, ids, vnorm, norm_dtype));
  HST_TRY(attention_checks(shape, q, K, V, k, scale, out, lse));
  HST_TRY(mass_p_check(p));
  if (!ptr_ok(idx) || !ptr_ok(counts)) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_DECODE_SOFTLSH_MASS, shape, L, P, k, ws, ws_bytes));
  return hip_status(hst::fused_decode_softlsh_mass(*shape, q, K, V, W, L, P, tau, ids, vnorm,
                                                   norm_dtype, k, k_per_seq, p, scale, idx,
                                                   counts, out, lse, ws,
                                                   static_cast<hipStream_t>(stream)));
}

hst_status hst_decode_step_softlsh(const hst_shape* shape, const void* q, const void* K,
                                   const void* V, const void* W, int L, int P, double tau,
                                   const uint8_t* ids, const void* vnorm, int norm_dtype, int k,
                                   const int32_t* k_per_seq, float scale, int32_t* idx,
                                   float* out, float* lse, void* ws, size_t ws_bytes,
                                   void* stream) {
  HST_TRY(score_softlsh_checks(shape, q, W, L, P, tau, ids, vnorm, norm_dtype));
  HST_TRY(attention_checks(shape, q, K, V, k, scale, out, lse));
  if (!ptr_ok(idx)) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_DECODE_SOFTLSH, shape, L, P, k, ws, ws_bytes));
  return hip_status(hst::fused_decode_softlsh(*shape, q, K, V, W, L, P, tau, ids, vnorm, norm_dtype,
                                              k, k_per_seq, scale, idx, out, lse, ws,
                                              static_cast<hipStream_t>(stream)));
}

hst_status hst_decode_step_hamming(const hst_shape* shape, const void* q, const void* K,
                                   const void* V, const void* R, int code_bits,
                                   const uint32_t* codes, int k, const int32_t* k_per_seq,
                                   float scale, int32_t* idx, float* out, float* lse, void* ws,
                                   size_t ws_bytes, void* stream) {
  HST_TRY(score_hamming_checks(shape, q, R, code_bits, codes));
  HST_TRY(attention_checks(shape, q, K, V, k, scale, out, lse));
  if (!ptr_ok(idx)) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_DECODE_HAMMING, shape, 0, 0, k, ws, ws_bytes, code_bits));
  if (code_bits != 128)
    return hip_status(hst::codes_decode(*shape, q, K, V, R, code_bits, codes, k, k_per_seq, scale,
                                        idx, out, lse, ws, static_cast<hipStream_t>(stream)));
  return hip_status(hst::fused_decode_hamming(*shape, q, K, V, R, codes, k, k_per_seq, scale, idx,
                                              out, lse, ws, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The decode step in three stages over one workspace.

extern "C" {

hst_status hst_decode_prepare_softlsh(const hst_shape* shape, const void* q, const void* W, int L,
                                      int P, double tau, const uint8_t* ids, const void* vnorm,
                                      int norm_dtype, int k, const int32_t* k_per_seq, void* ws,
                                      size_t ws_bytes, void* stream) {
  HST_TRY(score_softlsh_checks(shape, q, W, L, P, tau, ids, vnorm, norm_dtype));
  if (k < 1) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_DECODE_SOFTLSH, shape, L, P, k, ws, ws_bytes));
  return hip_status(hst::decode_prepare_softlsh(*shape, q, W, L, P, tau, ids, vnorm, norm_dtype, k,
                                                k_per_seq, ws, static_cast<hipStream_t>(stream)));
}

hst_status hst_decode_filter_softlsh(const hst_shape* shape, int L, int P, const uint8_t* ids,
                                     const void* vnorm, int norm_dtype, int k,
                                     const int32_t* k_per_seq, void* ws, size_t ws_bytes,
                                     void* stream) {
  HST_TRY(check_shape(shape));
  HST_TRY(check_lp(L, P));
  HST_TRY(check_norm_dtype(norm_dtype));
  HST_TRY(check_soft_prep(shape, L, P));
  if (k < 1) return HST_ERR_INVALID_ARG;
  if (!ptr_ok(ids) || !ptr_ok(vnorm)) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_DECODE_SOFTLSH, shape, L, P, k, ws, ws_bytes));
  return hip_status(hst::decode_filter_softlsh(*shape, L, P, ids, vnorm, norm_dtype, k, k_per_seq,
                                               ws, static_cast<hipStream_t>(stream)));
}

hst_status hst_decode_finish_softlsh(const hst_shape* shape, const void* q, const void* K,
                                     const void* V, int L, int P, const uint8_t* ids,
                                     const void* vnorm, int norm_dtype, int k, float scale,
                                     int32_t* idx, float* out, float* lse, void* ws,
                                     size_t ws_bytes, void* stream) {
  HST_TRY(check_lp(L, P));
  HST_TRY(check_norm_dtype(norm_dtype));
  HST_TRY(attention_checks(shape, q, K, V, k, scale, out, lse));
  HST_TRY(check_soft_prep(shape, L, P));
  if (!ptr_ok(idx) || !ptr_ok(ids) || !ptr_ok(vnorm)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_DECODE_SOFTLSH, shape, L, P, k, ws, ws_bytes));
  return hip_status(hst::decode_finish_softlsh(*shape, q, K, V, L, P, ids, vnorm, norm_dtype, k,
                                               scale, idx, out, lse, ws,
                                               static_cast<hipStream_t>(stream)));
}

hst_status hst_decode_prepare_hamming(const hst_shape* shape, const void* q, const void* R,
                                      const uint32_t* codes, int k, const int32_t* k_per_seq,
                                      void* ws, size_t ws_bytes, void* stream) {
  HST_TRY(score_hamming_checks(shape, q, R, 128, codes));
  if (k < 1) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_DECODE_HAMMING, shape, 0, 0, k, ws, ws_bytes));
  return hip_status(hst::decode_prepare_hamming(*shape, q, R, codes, k, k_per_seq, ws,
                                                static_cast<hipStream_t>(stream)));
}

hst_status hst_decode_filter_hamming(const hst_shape* shape, const uint32_t* codes, int k,
                                     const int32_t* k_per_seq, void* ws, size_t ws_bytes,
                                     void* stream) {
  HST_TRY(check_shape(shape));
  if (group(shape) > 64) return HST_ERR_UNSUPPORTED;
  if (k < 1) return HST_ERR_INVALID_ARG;
  if (!ptr_ok(codes)) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_DECODE_HAMMING, shape, 0, 0, k, ws, ws_bytes));
  return hip_status(hst::decode_filter_hamming(*shape, codes, k, k_per_seq, ws,
                                               static_cast<hipStream_t>(stream)));
}

hst_status hst_decode_finish_hamming(const hst_shape* shape, const void* q, const void* K,
                                     const void* V, const uint32_t* codes, int k, float scale,
                                     int32_t* idx, float* out, float* lse, void* ws,
                                     size_t ws_bytes, void* stream) {
  HST_TRY(attention_checks(shape, q, K, V, k, scale, out, lse));
  if (!ptr_ok(idx) || !ptr_ok(codes)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(HST_OP_DECODE_HAMMING, shape, 0, 0, k, ws, ws_bytes));
  return hip_status(hst::decode_finish_hamming(*shape, q, K, V, codes, k, scale, idx, out, lse, ws,
                                               static_cast<hipStream_t>(stream)));
}

hst_status hst_decode_candidates(const hst_shape* shape, int op, int L, int P, int k,
                                 void* ws, size_t ws_bytes, int cap, uint32_t* keys,
                                 int32_t* index, int32_t* count, uint32_t* theta, void* stream) {
  HST_TRY(check_shape(shape));
  if (op != HST_OP_DECODE_SOFTLSH && op != HST_OP_DECODE_HAMMING) return HST_ERR_INVALID_ARG;
  if (op == HST_OP_DECODE_SOFTLSH) HST_TRY(check_lp(L, P));
  if (k < 1 || cap < 1) return HST_ERR_INVALID_ARG;
  if (!ptr_ok(keys) || !ptr_ok(index) || !ptr_ok(count) || !ptr_ok(theta)) return HST_ERR_INVALID_ARG;
  HST_TRY(workspace_check(op, shape, L, P, k, ws, ws_bytes));
  return hip_status(hst::decode_candidates(*shape, op, L, P, k, ws, keys, index, count, theta, cap,
                                           static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The soft-LSH decode step without allocation, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops,
// harnesses that forbid it).  Its workspace is a file-scope device array,
// one copy per GPU, held from module load until the process ends.  Host code
// never uses the array's name as an address: the first call on a device
// looks its address up with hipGetSymbolAddress (with that device current)
// and keeps it per device.

namespace {

constexpr size_t kScratchBytes = size_t{64} << 20;  // 64 MiB per GPU
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};  // device address of `scratch`, per device ordinal

hst_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= 64) return HST_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return HST_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return HST_OK;
}

}  // namespace

extern "C" {

size_t hst_noalloc_scratch_bytes(void) { return kScratchBytes; }

hst_status hst_decode_step_softlsh_noalloc(const hst_shape* shape, const void* q, const void* K,
                                           const void* V, const void* W, int L, int P, double tau,
                                           const uint8_t* ids, const void* vnorm, int norm_dtype,
                                           int k, const int32_t* k_per_seq, float scale,
                                           int32_t* idx, float* out, float* lse, void* stream) {
  HST_TRY(score_softlsh_checks(shape, q, W, L, P, tau, ids, vnorm, norm_dtype));
  HST_TRY(attention_checks(shape, q, K, V, k, scale, out, lse));
  if (!ptr_ok(idx)) return HST_ERR_INVALID_ARG;
  if (k_per_seq != nullptr && !aligned16(k_per_seq)) return HST_ERR_INVALID_ARG;
  size_t need = 0;
  HST_TRY(hst_workspace_size(HST_OP_DECODE_SOFTLSH, shape, L, P, 128, k, &need));
  if (need > kScratchBytes) return HST_ERR_WORKSPACE;  // the shape needs more than the array
  void* ws = nullptr;
  HST_TRY(scratch_address(&ws));
  // the step needs no initial workspace contents: whatever the previous call
  // on this GPU left there is reset or overwritten before it is read
  return hip_status(hst::fused_decode_softlsh(*shape, q, K, V, W, L, P, tau, ids, vnorm, norm_dtype,
                                              k, k_per_seq, scale, idx, out, lse, ws,
                                              static_cast<hipStream_t>(stream)));
}

}  // extern "C"
