// Workspace layout and kernel arguments of the fused decode path (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hst.h"

namespace hst {

constexpr int kSample = 2048;      // keys sampled per head for the candidate threshold
constexpr int kSelCap = 8192;      // candidates a workgroup selects from in LDS
constexpr int kHistBins = 2048;    // bins of a selection's histogram of candidate keys
constexpr int kRunLen = 8;         // the sample is kSample / kRunLen runs of consecutive keys
constexpr int kMaxChunks = 4096;   // scan chunks per head (bounds Nmax)
constexpr int kMaxSplits = 256;    // attention splits per kv head (bounds the merge LDS)
constexpr int kCardKeys = 64;     // keys one index card of the routed step summarises
constexpr int kPrepBlocks = 8;     // prep workgroups per head (at least): each gathers 1/8 of the sample

enum ScanKind { kScanSoftFast = 0, kScanSoftAny = 1, kScanHamming = 2, kScanGivenF32 = 3, kScanGivenI32 = 4 };

// Per (sequence, kv head) state in the workspace header.
struct HeadState {
  uint32_t theta;       // candidate threshold (order key)
  int32_t k_eff;        // keys to select
  int32_t n;            // context length
  uint32_t cand_total;  // candidates the scan found (diagnostic)
  uint32_t path;        // selection path: 0 LDS, 1 HBM, 2 every key rescored or read (diagnostic)
  uint32_t shift;       // bin width of the selection's candidate histogram: key c >= theta
                        //   falls in bin min(kHistBins - 1, (c - theta) >> shift)
  uint64_t thr_word;    // (1 << 32) | theta once the scan has published it, else 0
  uint32_t arrive;      // attention splits of the head that have written their state
  uint32_t pad[7];
};
static_assert(sizeof(HeadState) == 64, "head state stride");

struct FusedLayout {
  size_t off_heads, off_tables, off_qcodes, off_spart, off_counts, off_slots, off_part_o,
      off_part_ml, bytes;
  int chunk;    // candidate slots per scan chunk (the stride of the slot array)
  int nchunks;  // scan chunks per head at the default chunk length (the most there can be)
  int sample, xparts, rps, nsplit, kind;
};

struct FusedArgs {
  int Hq, Hkv, d, Nmax, L, P;
  int nbh;  // B * Hkv: the (sequence, kv head) pairs
  double inv_tau;
  int kcap, sample, xparts, nchunks, rps, nsplit, region_bytes;
  int span;  // keys per scan chunk (at most the slot stride; see scan_span)
  HeadState* heads;
  float* tables;     // [B*Hkv][2^P][L] bucket-major
  uint32_t* qcodes;  // [B*Hkv][G][4]
  float* spart;      // [B*Hkv][xparts][kSample]: partial sample scores, one part per prep workgroup
                     //   (soft-LSH: tables of the workgroup; binary codes: its 16 code bits;
                     //   given scores: part 0 holds the order keys' bits)
  uint32_t* counts;  // [B*Hkv][nchunks]
  uint2* slots;      // [B*Hkv][nchunks][chunk] (order key, index), chunk c holding keys [c*span, (c+1)*span)
  float* part_o;     // [B*Hq][nsplit][d]
  float* part_ml;    // [B*Hq][nsplit][2]
  // the key metadata, for rescoring every key when fewer than k keys passed
  // the threshold (meta_kind: kScanSoftFast / kScanSoftAny: ids [.][Nmax][L]
  // with value norms meta_vn; kScanHamming: 128-bit codes; -1: none)
  const void* meta;
  const void* meta_vn;
  int meta_f16, meta_kind;
  // shared prefix (attention over given rows only): rows j < np come from
  // pk / pv [Hkv][np][d], rows np + j from K / V row j of the sequence
  const void* pk;
  const void* pv;
  int np;
  // index cards of the routed step (soft-LSH prep only): when cpart is set,
  // each prep workgroup also scores the first ceil(n_b / kCardKeys) cards of
  // its head on its own tables, cpart[B*Hkv][xparts][ncards] (no weight)
  const uint8_t* cids;  // [B*Hkv][ncards][L] card bucket ids
  float* cpart;
  int ncards;
};
__host__ __device__ inline int a_nsplit(const FusedArgs& a) { return a.nsplit; }

// The dispatcher places workgroup i of a 1-D grid on XCD i % kXcds (each XCD
// has its own L2).  xcd_item maps workgroup lid of a grid of `total` to a
// work item so that the workgroups of one XCD take consecutive items: XCD x
// takes [x*q + min(x, r), ... + q + (x < r)), q = total / kXcds,
// r = total % kXcds (a bijection of [0, total)).  Items laid out head-major
// then keep one head's workgroups, and the data they share, on one XCD.
constexpr int kXcds = 8;
__host__ __device__ inline int xcd_item(int lid, int total) {
  const int q = total / kXcds, r = total % kXcds, x = lid % kXcds;
  return x * q + (x < r ? x : r) + lid / kXcds;
}
// Threshold workgroups of a filtering scan, padded to whole XCD rounds so
// that the chunk workgroups after them start on XCD 0.
__host__ __device__ inline long long theta_groups(long long nbh) { return (nbh + kXcds - 1) / kXcds * kXcds; }
__host__ __device__ inline size_t hst_align16(size_t x) { return (x + 15) / 16 * 16; }

FusedLayout fused_layout(const hst_shape& s, int op, int L, int P, int kcap);

// kernel launchers (prep.hip, scan.hip, attend.hip)
hipError_t launch_prep_soft(const hst_shape& s, const FusedArgs& a, const void* q, const void* W,
                            const uint8_t* ids, const int32_t* kps, hipStream_t st);
hipError_t launch_prep_hamming(const hst_shape& s, const FusedArgs& a, const void* q, const void* R,
                               const uint32_t* codes, const int32_t* kps, hipStream_t st);
hipError_t launch_prep_given(const hst_shape& s, const FusedArgs& a, int score_dtype,
                             const void* scores, const int32_t* kps, hipStream_t st);
int prep_parts(int kind, int L);  // partial sample scores per head (prep workgroups)
int scan_chunk(int L);  // default keys per scan chunk
int scan_cap(int L);    // candidate slots per chunk: the longest chunk a scan workgroup takes
// keys per chunk of a filtering scan over s (slot stride cap, default length
// chunk): lengthened (up to cap) when the threshold workgroups would
// otherwise add a round of resident workgroups
int scan_span(const hst_shape& s, int chunk, int cap, bool filter);
// filter != 0: the scan also derives each head's candidate threshold from the
// partial sample scores (prep with sampling must precede it) and fills the
// candidate slots
hipError_t launch_scan(const hst_shape& s, const FusedArgs& a, int kind, const void* src,
                       const void* vnorm, int norm_f16, void* scores_out, int filter,
                       const int32_t* kps, hipStream_t st);
hipError_t launch_attend(const hst_shape& s, const FusedArgs& a, const void* q, const void* K,
                         const void* V, int32_t* idx, bool select, const void* scores, int scores_int,
                         int chunk, float scale, float* out, float* lse, hipStream_t st);
hipError_t launch_select_only(const hst_shape& s, const FusedArgs& a, int32_t* idx, const void* scores,
                              int scores_int, int chunk, hipStream_t st);
hipError_t launch_candidates(const hst_shape& s, const FusedArgs& a, int chunk, uint32_t* keys, int32_t* index,
                             int32_t* count, uint32_t* theta, int cap, hipStream_t st);

// cumulative-mass selection (mass.hip): float64 logits of the candidates in
// `logits` ([B*Hq][kcap] doubles), then the cut and the compaction
constexpr int kMassCap = 8192;
size_t mass_logits_bytes(const hst_shape& s, int kcap);
hipError_t launch_select_mass(const hst_shape& s, const void* q, const void* K,
                              const int32_t* cand, int kcap, double p, float scale, int32_t* idx,
                              int32_t* counts, double* logits, hipStream_t st);
hipError_t fused_decode_softlsh_mass(const hst_shape& s, const void* q, const void* K,
                                     const void* V, const void* W, int L, int P, double tau,
                                     const uint8_t* ids, const void* vnorm, int norm_dtype,
                                     int kcap, const int32_t* kps, double p, float scale,
                                     int32_t* idx, int32_t* counts, float* out, float* lse,
                                     void* ws, hipStream_t st);
size_t decode_mass_bytes(const hst_shape& s, int L, int P, int kcap);

// two-level chunk routing (route.hip)
constexpr int kRouteMaxChunks = 256;      // chunks one routed step keeps per head
constexpr int kRouteMaxCards = 16384;     // cards per head (Nmax <= 1M)
int route_chunks(int Nmax);
hipError_t launch_card_sums(const hst_shape& s, const void* K, const void* vnorm, int norm_f16,
                            void* ckeys, void* cw, int32_t* clens, hipStream_t st);
hipError_t launch_route_scan(const hst_shape& s, const float* tables, const int32_t* chunks, int C,
                             const uint8_t* ids, const void* vnorm, int norm_f16, int L, int P,
                             int out_stride, float* out, hipStream_t st);
size_t card_route_smem(int Nc);
// cpart: the prep workgroups' partial card scores, xparts parts per head
hipError_t launch_card_route(const hst_shape& s, const float* cpart, int xparts, const void* cw,
                             int norm_f16, int C, int32_t* chunks, hipStream_t st);
hipError_t launch_token_route(const hst_shape& s, const float* scores, int nitems,
                              const int32_t* chunks, int C, int k, const int32_t* kps,
                              int32_t* out, hipStream_t st);
hipError_t build_cards_softlsh(const hst_shape& s, const void* K, const void* vnorm, int norm_dtype,
                               const void* W, int L, int P, void* ckeys, uint8_t* cids, void* cw,
                               int32_t* clens, hipStream_t st);
size_t route_ws_bytes(const hst_shape& s, int L, int P, int kcap);
hipError_t fused_decode_softlsh_routed(const hst_shape& s, const void* q, const void* K,
                                       const void* V, const void* W, int L, int P, double tau,
                                       const uint8_t* ids, const void* vnorm, int norm_dtype,
                                       const uint8_t* cids, const void* cw, int C, int kcap,
                                       const int32_t* kps, float scale, int32_t* idx, float* out,
                                       float* lse, void* ws, hipStream_t st);

// shared-prefix decode (shared.hip)
hipError_t launch_shared_lens(const hst_shape& s, int Np, int32_t* v_lens, hipStream_t st);
hipError_t launch_scan_shared(const hst_shape& s, const FusedArgs& a, int Np,
                              const uint8_t* ids_p, const void* vn_p, const uint8_t* ids_s,
                              const void* vn_s, int norm_f16, float* scores_out, hipStream_t st);
size_t shared_ws_bytes(const hst_shape& s, int Np, int L, int P, int kcap);
hipError_t fused_decode_softlsh_shared(const hst_shape& s, int Np, const void* q, const void* Kp,
                                       const void* Vp, const uint8_t* ids_p, const void* vn_p,
                                       const void* Ks, const void* Vs, const uint8_t* ids_s,
                                       const void* vn_s, const void* W, int L, int P, double tau,
                                       int norm_dtype, int kcap, const int32_t* kps, float scale,
                                       int32_t* idx, float* out, float* lse, void* ws,
                                       hipStream_t st);

// binary codes of 64 or 256 bits (codes.hip, pipeline.hip)
hipError_t launch_hamming_scan(const hst_shape& s, int code_bits, const uint32_t* qcodes,
                               const uint32_t* kcodes, int32_t* scores, hipStream_t st);
hipError_t launch_query_codes(const hst_shape& s, const void* q, const void* R, int code_bits,
                              uint32_t* qcodes, hipStream_t st);
size_t codes_ws_bytes(const hst_shape& s, int code_bits, int kcap, bool decode);
hipError_t codes_score(const hst_shape& s, const void* q, const void* R, int code_bits,
                       const uint32_t* codes, int32_t* scores, void* ws, hipStream_t st);
hipError_t codes_decode(const hst_shape& s, const void* q, const void* K, const void* V,
                        const void* R, int code_bits, const uint32_t* codes, int kcap,
                        const int32_t* kps, float scale, int32_t* idx, float* out, float* lse,
                        void* ws, hipStream_t st);

hipError_t fused_decode_softlsh(const hst_shape& s, const void* q, const void* K, const void* V,
                                const void* W, int L, int P, double tau, const uint8_t* ids,
                                const void* vnorm, int norm_dtype, int kcap, const int32_t* kps,
                                float scale, int32_t* idx, float* out, float* lse, void* ws,
                                hipStream_t st);
// The decode step's three stages over one workspace (the full step runs
// them in this order): query tables or codes with the key sample; the
// filtering scan (scores, threshold, candidates and their histogram); the
// selection and the attention.
hipError_t decode_prepare_softlsh(const hst_shape& s, const void* q, const void* W, int L, int P,
                                  double tau, const uint8_t* ids, const void* vnorm, int norm_dtype,
                                  int kcap, const int32_t* kps, void* ws, hipStream_t st);
hipError_t decode_filter_softlsh(const hst_shape& s, int L, int P, const uint8_t* ids,
                                 const void* vnorm, int norm_dtype, int kcap, const int32_t* kps,
                                 void* ws, hipStream_t st);
hipError_t decode_finish_softlsh(const hst_shape& s, const void* q, const void* K, const void* V,
                                 int L, int P, const uint8_t* ids, const void* vnorm,
                                 int norm_dtype, int kcap, float scale, int32_t* idx, float* out,
                                 float* lse, void* ws, hipStream_t st);
hipError_t decode_prepare_hamming(const hst_shape& s, const void* q, const void* R,
                                  const uint32_t* codes, int kcap, const int32_t* kps, void* ws,
                                  hipStream_t st);
hipError_t decode_filter_hamming(const hst_shape& s, const uint32_t* codes, int kcap,
                                 const int32_t* kps, void* ws, hipStream_t st);
hipError_t decode_finish_hamming(const hst_shape& s, const void* q, const void* K, const void* V,
                                 const uint32_t* codes, int kcap, float scale, int32_t* idx,
                                 float* out, float* lse, void* ws, hipStream_t st);
// candidates of every head after the filtering scan, in index order:
// (order key, index) pairs, up to cap per head, their count and threshold
hipError_t decode_candidates(const hst_shape& s, int op, int L, int P, int kcap, void* ws,
                             uint32_t* keys, int32_t* index, int32_t* count, uint32_t* theta,
                             int cap, hipStream_t st);
hipError_t fused_decode_hamming(const hst_shape& s, const void* q, const void* K, const void* V,
                                const void* R, const uint32_t* codes, int kcap, const int32_t* kps,
                                float scale, int32_t* idx, float* out, float* lse, void* ws,
                                hipStream_t st);
hipError_t fused_score_softlsh(const hst_shape& s, const void* q, const void* W, int L, int P,
                               double tau, const uint8_t* ids, const void* vnorm, int norm_dtype,
                               float* scores, void* ws, hipStream_t st);
hipError_t fused_score_hamming(const hst_shape& s, const void* q, const void* R,
                               const uint32_t* codes, int32_t* scores, void* ws, hipStream_t st);
hipError_t fused_tables_softlsh(const hst_shape& s, const void* q, const void* W, int L, int P,
                                double tau, float* tables, hipStream_t st);
hipError_t fused_scan_softlsh(const hst_shape& s, const float* tables, int L, int P,
                              const uint8_t* ids, const void* vnorm, int norm_dtype, float* scores,
                              hipStream_t st);
hipError_t fused_select(const hst_shape& s, int score_dtype, const void* scores, int kcap,
                        const int32_t* kps, int32_t* idx, void* ws, hipStream_t st);
hipError_t fused_attention(const hst_shape& s, const void* q, const void* K, const void* V,
                           const int32_t* idx, int kcap, float scale, float* out, float* lse,
                           void* ws, hipStream_t st);

}  // namespace hst
