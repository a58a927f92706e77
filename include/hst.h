/*
 * hst.h - C ABI of the hash-scored top-k sparse decode attention library
 * (libhst.so, MI355X / gfx950).
 *
 * One decode step of one attention layer: every cached key is scored cheaply
 * against the query from metadata computed once at prefill, the top-k keys of
 * each kv head are selected, and exact softmax attention runs over the
 * gathered K/V rows of that subset only.
 *
 * Method sources (web pages, cited by title and section):
 *   [SOCKET] "SOCKET - SOft Collision Kernel EsTimator" technical overview
 *            (gist.science), section "Core mechanism: soft LSH", items 1-4,
 *            and section "Experimental results" (metadata = bucket ids plus
 *            value norms, about 15% over the KV cache).
 *   [HATA]   "HATA: Hash-Aware Top-k Attention" explainer (aibr.jp),
 *            section 3 "core technical elements": binary codes for queries
 *            and keys, ranking by code comparison.  The learned hash is
 *            replaced by the sign of a caller-supplied projection.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates, frees or keeps them.  Memory needed beyond
 *     inputs and outputs is a caller-owned workspace whose size
 *     hst_workspace_size() reports.
 *   - Layouts are dense row-major C arrays:
 *       K, V     [B][Hkv][Nmax][d]   element type shape->kv_dtype
 *       q        [B][Hq][d]          element type shape->kv_dtype
 *       W        [Hkv][L*P][d]       soft-LSH hyperplanes, row l*P + p
 *       R        [Hkv][code_bits][d] binary-code projections
 *       ids      [B][Hkv][Nmax][L]   uint8 bucket ids (bit p = hyperplane p)
 *       vnorm    [B][Hkv][Nmax]      value norms, norm_dtype (F16 or F32)
 *       codes    [B][Hkv][Nmax][code_bits/32] uint32 (bit i in word i/32,
 *                                    position i%32)
 *       scores   [B][Hkv][Nmax]      F32 (soft) or I32 (binary)
 *       idx      [B][Hkv][k]         int32, ascending, -1 after the count
 *       out      [B][Hq][d]          float32
 *       lse      [B][Hq]             float32 (natural log), nullable
 *     Query head hq reads kv head hq / (Hq / Hkv) (grouped-query attention).
 *   - shape->seq_lens is an optional DEVICE array [B] of context lengths
 *     N_b in [0, Nmax]; NULL means every N_b = Nmax.  Rows j >= N_b are
 *     never read or written by any call, except that the append calls write
 *     row N_b and then advance N_b.
 *   - Pointers must be 16-byte aligned.
 *   - Workspaces: a caller-owned device buffer of at least
 *     hst_workspace_size() bytes, 256-byte aligned, with no required initial
 *     contents.  Calls that share a workspace must not overlap in time (use
 *     one stream per workspace).
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the
 *     null stream) and never synchronizes.  Arguments are validated on the
 *     host before anything is enqueued; on error nothing is launched.
 *   - Calls are reentrant and may be made from several host threads at once.
 *     The only process-wide state is host-side and set once per device: the
 *     raised dynamic-LDS limit of each kernel (a table under a mutex) and the
 *     device's compute-unit count (an atomic cache); plus the thread-local
 *     last HIP error.
 */
#ifndef HST_H_
#define HST_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  HST_OK = 0,
  HST_ERR_INVALID_ARG = -1, /* null pointer, bad size, misalignment        */
  HST_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype, d, P ...)  */
  HST_ERR_WORKSPACE = -3,   /* workspace smaller than hst_workspace_size() */
  HST_ERR_HIP = -4          /* a HIP launch failed: see hst_last_hip_error */
} hst_status;

typedef enum { HST_F32 = 0, HST_BF16 = 1, HST_F16 = 2, HST_I32 = 3 } hst_dtype;

typedef struct {
  int32_t B;                /* sequences in the batch, >= 1                */
  int32_t Hq;               /* query heads, multiple of Hkv                */
  int32_t Hkv;              /* kv heads, >= 1                              */
  int32_t d;                /* head dim: 64 or 128                         */
  int32_t Nmax;             /* cache capacity per sequence, >= 1           */
  int32_t kv_dtype;         /* hst_dtype of K, V, q, W, R: F32 or BF16     */
  const int32_t* seq_lens;  /* device [B] or NULL                          */
} hst_shape;

typedef enum {
  HST_OP_HASH_SOFTLSH = 0,
  HST_OP_HASH_BINARY = 1,
  HST_OP_SCORE_SOFTLSH = 2,
  HST_OP_SCORE_HAMMING = 3,
  HST_OP_SELECT_TOPK = 4,
  HST_OP_SPARSE_ATTENTION = 5,
  HST_OP_DECODE_SOFTLSH = 6,
  HST_OP_DECODE_HAMMING = 7,
  HST_OP_SELECT_MASS = 8,
  HST_OP_DECODE_SOFTLSH_MASS = 9,
  HST_OP_DECODE_SOFTLSH_ROUTED = 10
} hst_op;

/* Library version as major*10000 + minor*100 + patch. */
int hst_version(void);

/* Static, human-readable text for a status code. */
const char* hst_status_string(int status);

/* hipError_t of the last HST_ERR_HIP on the calling thread (0 if none). */
int hst_last_hip_error(void);

/*
 * Debug builds only (libhst_debug.so, compiled with HST_DEBUG): the code of
 * the first failed bounds check of any kernel since the last call (0 if
 * none; the codes are listed in csrc/hst_common.h), which the call then
 * clears.  A failed check clamps the value it guards, so kernels always
 * complete; their results are then not to be trusted.  This call
 * synchronises the device (a blocking copy), unlike every other entry point.
 * The release library sets *code = 0 and returns HST_ERR_UNSUPPORTED.
 * code: host pointer, must not be NULL (HST_ERR_INVALID_ARG).
 */
hst_status hst_debug_status(uint32_t* code);

/*
 * Workspace bytes the given op needs for this shape.  L, P describe the
 * soft-LSH tables (ignored otherwise), code_bits the binary codes (ignored
 * otherwise), k the idx row capacity (select, attention, decode).
 * Returns HST_ERR_INVALID_ARG / HST_ERR_UNSUPPORTED for shapes the op rejects.
 */
hst_status hst_workspace_size(int op, const hst_shape* shape, int L, int P,
                              int code_bits, int k, size_t* bytes);

/*
 * Prefill hashing of keys into soft-LSH bucket ids and cached value norms
 * [SOCKET, core mechanism item 1].
 *   ids[b][h][j][l] = sum_p [ W[h][l*P+p] . K[b][h][j] >= 0 ] << p
 * The sign is that of the exact real dot product of the stored values (a
 * zero projection sets the bit).  vnorm[b][h][j] = ||V[b][h][j]||_2 rounded
 * to nearest-even in norm_dtype (F16 or F32).
 * Requires 1 <= P <= 8, 1 <= L <= 1024.  No workspace.  Rows j >= N_b are
 * not written.  Inputs must be finite.
 */
hst_status hst_hash_keys_softlsh(const hst_shape* shape, const void* K,
                                 const void* V, const void* W, int L, int P,
                                 int norm_dtype, uint8_t* ids, void* vnorm,
                                 void* stream);

/*
 * Prefill binary codes of keys [HATA, section 3; random-projection stand-in
 * for the learned hash]:
 *   bit i of codes[b][h][j] = [ R[h][i] . K[b][h][j] >= 0 ]  (exact sign)
 * code_bits is 64, 128 or 256 (R holds that many rows per kv head).  No
 * workspace.  Errors: HST_ERR_UNSUPPORTED for any other code_bits.
 */
hst_status hst_hash_keys_binary(const hst_shape* shape, const void* K,
                                const void* R, int code_bits, uint32_t* codes,
                                void* stream);

/*
 * Decode-time append of one token per sequence, with incremental hashing
 * [SOCKET, core mechanism item 1: the per-key hash and value norm are
 * computed once per key; a decode step adds one key per sequence].
 * For every b with N_b < Nmax and every kv head h:
 *   K[b][h][N_b] = k_new[b][h], V[b][h][N_b] = v_new[b][h]   ([B][Hkv][d])
 *   ids[b][h][N_b], vnorm[b][h][N_b] as hst_hash_keys_softlsh computes them
 *   (codes[b][h][N_b] as hst_hash_keys_binary, for the binary variant),
 * then N_b += 1 in shape->seq_lens, which is required (device array, read
 * and written).  A sequence whose cache is full (N_b == Nmax) is left
 * unchanged.  The rows are written before the lengths advance (two kernels
 * on the stream), so a decode step enqueued after the call sees the new
 * token.  A negative N_b counts as 0.  Same requirements as the prefill
 * calls (1 <= P <= 8, 1 <= L <= 1024, code_bits == 128); no workspace.
 * Errors: HST_ERR_INVALID_ARG for a NULL shape->seq_lens or a NULL or
 * misaligned pointer, HST_ERR_UNSUPPORTED for limits outside those.
 */
hst_status hst_append_kv_softlsh(const hst_shape* shape, const void* k_new,
                                 const void* v_new, const void* W, int L, int P,
                                 int norm_dtype, void* K, void* V, uint8_t* ids,
                                 void* vnorm, void* stream);
hst_status hst_append_kv_binary(const hst_shape* shape, const void* k_new,
                                const void* v_new, const void* R, int code_bits,
                                void* K, void* V, uint32_t* codes, void* stream);

/*
 * Soft-collision scores of all keys [SOCKET, core mechanism items 2-3].
 * For each query head: q_hat = q/||q||, z_{l,p} = W[h][l*P+p] . q_hat; the
 * probability of bucket c in table l is the softmax over all 2^P buckets of
 * sum_p s_p(c) z_{l,p} / tau with s_p(c) = +1 if bit p of c is set, else -1
 * (a zero query gives uniform probabilities).  Summing the probabilities
 * of the G = Hq/Hkv query heads of kv head h gives a table T[b][h][l][c],
 * and
 *   scores[b][h][j] = vnorm[b][h][j] * sum_l T[b][h][l][ ids[b][h][j][l] ]
 * in float32 for j < N_b.  tau > 0.  Workspace holds the tables.
 */
hst_status hst_score_keys_softlsh(const hst_shape* shape, const void* q,
                                  const void* W, int L, int P, double tau,
                                  const uint8_t* ids, const void* vnorm,
                                  int norm_dtype, float* scores, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * The two steps of hst_score_keys_softlsh as separate calls.
 * hst_query_tables_softlsh writes the per-(sequence, kv head) bucket
 * probability tables, bucket-major: T[b][h][c][l] float32, shape
 * [B][Hkv][2^P][L] (the soft assignment of the query, summed over the G
 * query heads of the kv head).
 * hst_score_scan_softlsh streams the bucket ids and value norms of every key
 * once and writes scores[b][h][j] = vnorm * sum_l T[b][h][ids[b][h][j][l]][l]
 * for j < N_b.  No workspace.  Both require shape->Hq / shape->Hkv query
 * heads per kv head as for hst_score_keys_softlsh.
 */
hst_status hst_query_tables_softlsh(const hst_shape* shape, const void* q,
                                    const void* W, int L, int P, double tau,
                                    float* tables, void* stream);
hst_status hst_score_scan_softlsh(const hst_shape* shape, const float* tables,
                                  int L, int P, const uint8_t* ids,
                                  const void* vnorm, int norm_dtype,
                                  float* scores, void* stream);

/*
 * Binary-code similarity scores [HATA, section 3]:
 *   scores[b][h][j] = sum over query heads hq of kv head h of
 *                     (code_bits - popcount(qcode_hq XOR codes[b][h][j]))
 * with qcode_hq the code of q[b][hq] under R[h] (exact sign, as above).
 * int32, range [0, code_bits * G].  Workspace holds the query codes.
 */
hst_status hst_score_keys_hamming(const hst_shape* shape, const void* q,
                                  const void* R, int code_bits,
                                  const uint32_t* codes, int32_t* scores,
                                  void* ws, size_t ws_bytes, void* stream);

/*
 * Deterministic top-k per (sequence, kv head) [SOCKET, core mechanism
 * item 4]: among j < N_b, the keys first in the order (score descending,
 * index ascending), count k_b = min(k, N_b) or, with k_per_seq (device [B]),
 * min(max(k_per_seq[b], 0), k, N_b).  idx rows have capacity k; the k_b
 * selected indices are written in ascending order and the rest of the row
 * is -1.  score_dtype is F32 (-0 equals +0; NaN unsupported) or I32.
 * k >= 1.
 */
hst_status hst_select_topk(const hst_shape* shape, int score_dtype,
                           const void* scores, int k,
                           const int32_t* k_per_seq, int32_t* idx, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * Exact softmax attention over selected keys [SOCKET, core mechanism
 * item 4]: for query head hq of kv head h and S = { idx[b][h][i] : i < k,
 * 0 <= idx[b][h][i] < N_b } (other entries are padding and are skipped),
 *   a_j = scale * q[b][hq] . K[b][h][j],
 *   out[b][hq] = sum_{j in S} softmax(a)_j V[b][h][j],
 *   lse[b][hq] = log sum_{j in S} exp(a_j)
 * accumulated in float32.  An empty S gives out = 0, lse = -inf.
 * Repeated indices count once per occurrence.
 */
hst_status hst_sparse_decode_attention(const hst_shape* shape, const void* q,
                                       const void* K, const void* V,
                                       const int32_t* idx, int k, float scale,
                                       float* out, float* lse, void* ws,
                                       size_t ws_bytes, void* stream);

/*
 * Cumulative-mass selection over candidates [Tactic, sections 1 and 3:
 * tokens are added until the summed normalised attention score of the set
 * reaches a target, so the count adapts per head and query].  For kv head
 * h of sequence b, the candidates are C = { cand[b][h][i] : i < k,
 * 0 <= cand[b][h][i] < N_b } (other entries are padding).  With the G query
 * heads of h,
 *   a_gj = scale * q[b][h*G+g] . K[b][h][j]             (float64, j in C)
 *   m_j  = (1/G) sum_g exp(a_gj) / sum_{i in C} exp(a_gi)
 * the keys are taken in the order (m_j descending, j ascending) until the
 * running sum of m reaches p * sum_{j in C} m_j (at least one key when C is
 * not empty).  counts[b][h] receives the number taken; idx[b][h][0..k)
 * receives them in candidate order (ascending when cand is, as
 * hst_select_topk writes it), then -1.  0 < p <= 1; 1 <= k <= 8192.
 * idx must not overlap cand.  The decisions are taken in float64; a
 * running sum within a few units in the last place of the target may land
 * on either side.
 */
hst_status hst_select_mass(const hst_shape* shape, const void* q, const void* K,
                           const int32_t* cand, int k, double p, float scale,
                           int32_t* idx, int32_t* counts, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * One soft-LSH decode step: the scores of hst_score_keys_softlsh, the
 * selection of hst_select_topk over them and hst_sparse_decode_attention
 * over that selection, on the same stream (the three stage calls below).
 * Only the candidate keys' scores are kept (in the workspace), not the
 * whole score row.  idx (the selection, as hst_select_topk writes it) is an
 * output.  lse nullable.
 */
hst_status hst_decode_step_softlsh(const hst_shape* shape, const void* q,
                                   const void* K, const void* V,
                                   const void* W, int L, int P, double tau,
                                   const uint8_t* ids, const void* vnorm,
                                   int norm_dtype, int k,
                                   const int32_t* k_per_seq, float scale,
                                   int32_t* idx, float* out, float* lse,
                                   void* ws, size_t ws_bytes, void* stream);

/* One binary-code decode step: score (Hamming), select, attend. */
hst_status hst_decode_step_hamming(const hst_shape* shape, const void* q,
                                   const void* K, const void* V,
                                   const void* R, int code_bits,
                                   const uint32_t* codes, int k,
                                   const int32_t* k_per_seq, float scale,
                                   int32_t* idx, float* out, float* lse,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * Soft-LSH decode step with a cumulative-mass budget [Tactic, section 3]:
 * as hst_decode_step_softlsh up to the selection of the k (or
 * k_per_seq[b]) keys of highest hash score, which become the candidates of
 * hst_select_mass; attention then runs over the keys it keeps.  idx and
 * counts are as hst_select_mass writes them; lse nullable.
 * 1 <= k <= 8192, 0 < p <= 1.
 */
hst_status hst_decode_step_softlsh_mass(const hst_shape* shape, const void* q,
                                        const void* K, const void* V,
                                        const void* W, int L, int P,
                                        double tau, const uint8_t* ids,
                                        const void* vnorm, int norm_dtype,
                                        int k, const int32_t* k_per_seq,
                                        double p, float scale, int32_t* idx,
                                        int32_t* counts, float* out,
                                        float* lse, void* ws, size_t ws_bytes,
                                        void* stream);

/*
 * Index cards of 64-token chunks [HGA, section 2, step 1: the context is
 * cut into 64-token chunks, each summarised on a small card that the query
 * scans first].  For chunk c of (b, h) (keys 64c .. min(64c+64, N_b) - 1):
 *   card_keys[b][h][c] = sum of the chunk's keys, accumulated in float64 in
 *                        index order and rounded to the KV type (bf16: to
 *                        float32, then to bf16, both to nearest even)
 *   card_ids[b][h][c]  = bucket ids of that card key, as
 *                        hst_hash_keys_softlsh computes them for a key
 *   card_w[b][h][c]    = the largest stored value norm of the chunk
 *                        (norm_dtype, as vnorm)
 *   card_lens[b]       = ceil(N_b / 64)
 * Arrays have Nc = ceil(Nmax / 64) cards per head; cards c >= card_lens[b]
 * are not written.  vnorm is the output of hst_hash_keys_softlsh.  Same
 * requirements as hst_hash_keys_softlsh; no workspace.
 */
hst_status hst_build_cards_softlsh(const hst_shape* shape, const void* K,
                                   const void* vnorm, int norm_dtype,
                                   const void* W, int L, int P, void* card_keys,
                                   uint8_t* card_ids, void* card_w,
                                   int32_t* card_lens, void* stream);

/*
 * Soft-LSH decode step with two-level routing [HGA, section 2: chunk
 * routing on the cards, token routing inside the chosen chunks, exact
 * attention over the original tokens].  The query tables of
 * hst_score_keys_softlsh score every card (card_w times the table mass of
 * its buckets); the C cards first in the order (score descending, chunk
 * ascending) are kept; every key of those chunks is scored as in
 * hst_score_keys_softlsh; the k (or k_per_seq[b]) keys first in the order
 * (score descending, index ascending) among them are attended as in
 * hst_sparse_decode_attention.  idx [B][Hkv][k] receives them ascending,
 * then -1.  1 <= C <= 256; L in {16, 32, 64, 128}; Nmax <= 1048576.
 */
hst_status hst_decode_step_softlsh_routed(const hst_shape* shape, const void* q,
                                          const void* K, const void* V,
                                          const void* W, int L, int P,
                                          double tau, const uint8_t* ids,
                                          const void* vnorm, int norm_dtype,
                                          const uint8_t* card_ids,
                                          const void* card_w, int C, int k,
                                          const int32_t* k_per_seq, float scale,
                                          int32_t* idx, float* out, float* lse,
                                          void* ws, size_t ws_bytes,
                                          void* stream);

/*
 * Soft-LSH decode step for a batch that shares a prefix [bifurcated
 * attention, sections 1 and 3: the shared context is kept apart from each
 * sample's own part and read once for the whole batch].  shape describes
 * the suffix caches (Nmax = suffix capacity, seq_lens = suffix lengths).
 * The context of sequence b is the Np prefix keys followed by its own
 * N_b suffix keys; key j < Np is prefix key j, key Np + j is suffix key j.
 *   Kp, Vp  [Hkv][Np][d], ids_p [Hkv][Np][L], vnorm_p [Hkv][Np] (the
 *           prefix cache and its metadata, as hst_hash_keys_softlsh writes
 *           them for a batch of one)
 *   Ks, Vs, ids_s, vnorm_s: the suffix caches, [B][Hkv][Nmax]...
 * The result is hst_decode_step_softlsh's over the concatenated context:
 * idx [B][Hkv][k] holds context indices, ascending, then -1.  The prefix
 * metadata is scanned once per kv head for the whole batch.  L in {16, 32,
 * 64, 128}; Np >= 0; Np + Nmax <= 2^30.  Workspace from
 * hst_workspace_size_shared.
 */
hst_status hst_decode_step_softlsh_shared(const hst_shape* shape, int Np,
                                          const void* q, const void* Kp,
                                          const void* Vp, const uint8_t* ids_p,
                                          const void* vnorm_p, const void* Ks,
                                          const void* Vs, const uint8_t* ids_s,
                                          const void* vnorm_s, const void* W,
                                          int L, int P, double tau,
                                          int norm_dtype, int k,
                                          const int32_t* k_per_seq, float scale,
                                          int32_t* idx, float* out, float* lse,
                                          void* ws, size_t ws_bytes,
                                          void* stream);

/* Workspace bytes of hst_decode_step_softlsh_shared. */
hst_status hst_workspace_size_shared(const hst_shape* shape, int Np, int L,
                                     int P, int k, size_t* bytes);

/*
 * The decode step in three stages over one workspace (the same workspace
 * hst_workspace_size reports for HST_OP_DECODE_SOFTLSH / _HAMMING).  Run in
 * this order on one stream, they compute exactly what hst_decode_step_softlsh
 * (hst_decode_step_hamming, 128-bit codes) computes; the step itself is
 * these three calls.  Each stage reads what the previous one left in the
 * workspace, so a caller may put other work between them but must not reuse
 * the workspace in between.
 *   prepare: the query tables [SOCKET, core mechanism item 2] (or the query
 *            codes [HATA, section 3]) and, per table group (code slice),
 *            the parts of the scores of a fixed sample of 2048 keys per
 *            (sequence, kv head);
 *   filter:  the sample's scores (the parts added up, times the sampled
 *            keys' value norms for soft-LSH) give a threshold below the
 *            k-th score; every key is scored once [SOCKET, item 3; HATA,
 *            section 3]; the keys scoring at or above the threshold are kept
 *            as candidates, in index order (the exactness of the selection
 *            never depends on the threshold);
 *   finish:  the exact top-k of the candidates (or of every key, rescored,
 *            when fewer than k_b keys passed the threshold) and exact
 *            attention over them [SOCKET, item 4]; idx, out, lse as for the
 *            full step.
 * k_per_seq (optional) is read by prepare and filter; finish uses what
 * filter recorded.  Arguments are those of the full step.
 */
hst_status hst_decode_prepare_softlsh(const hst_shape* shape, const void* q,
                                      const void* W, int L, int P, double tau,
                                      const uint8_t* ids, const void* vnorm,
                                      int norm_dtype, int k,
                                      const int32_t* k_per_seq, void* ws,
                                      size_t ws_bytes, void* stream);
hst_status hst_decode_filter_softlsh(const hst_shape* shape, int L, int P,
                                     const uint8_t* ids, const void* vnorm,
                                     int norm_dtype, int k,
                                     const int32_t* k_per_seq, void* ws,
                                     size_t ws_bytes, void* stream);
hst_status hst_decode_finish_softlsh(const hst_shape* shape, const void* q,
                                     const void* K, const void* V, int L, int P,
                                     const uint8_t* ids, const void* vnorm,
                                     int norm_dtype, int k, float scale,
                                     int32_t* idx, float* out, float* lse,
                                     void* ws, size_t ws_bytes, void* stream);
hst_status hst_decode_prepare_hamming(const hst_shape* shape, const void* q,
                                      const void* R, const uint32_t* codes,
                                      int k, const int32_t* k_per_seq, void* ws,
                                      size_t ws_bytes, void* stream);
hst_status hst_decode_filter_hamming(const hst_shape* shape,
                                     const uint32_t* codes, int k,
                                     const int32_t* k_per_seq, void* ws,
                                     size_t ws_bytes, void* stream);
hst_status hst_decode_finish_hamming(const hst_shape* shape, const void* q,
                                     const void* K, const void* V,
                                     const uint32_t* codes, int k, float scale,
                                     int32_t* idx, float* out, float* lse,
                                     void* ws, size_t ws_bytes, void* stream);

/*
 * Inspection of the filter stage: for every (sequence b, kv head h), row
 * bh = b*Hkv + h of the outputs receives the candidates the filter stage
 * left in the workspace, in index order, as (order key, index) pairs in
 * keys[bh][0..cap) / index[bh][0..cap) (at most cap of them), their number
 * in count[bh] (which may exceed cap) and the threshold in theta[bh].  The
 * order key of a float32 score s >= 0 is bits(s) | 0x80000000 (of an int32
 * score v: v ^ 0x80000000).  op is HST_OP_DECODE_SOFTLSH (L, P as for the
 * step) or HST_OP_DECODE_HAMMING; ws must come from a filter stage of the
 * same shape and k.
 */
hst_status hst_decode_candidates(const hst_shape* shape, int op, int L, int P,
                                 int k, void* ws, size_t ws_bytes, int cap,
                                 uint32_t* keys, int32_t* index, int32_t* count,
                                 uint32_t* theta, void* stream);

/*
 * For callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the soft-LSH decode
 * step of hst_decode_step_softlsh, same arguments and results, without the
 * caller's workspace.  Its workspace is a fixed device array inside the
 * library, hst_noalloc_scratch_bytes() bytes (64 MiB) per GPU, held from the
 * library's load on that GPU until the process ends; the call allocates
 * nothing.  The first call on a device looks up that device's copy of the
 * array (once, under a lock).
 *   - Shapes whose workspace (hst_workspace_size of HST_OP_DECODE_SOFTLSH)
 *     exceeds the array are rejected with HST_ERR_WORKSPACE before anything
 *     is enqueued.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (different streams, or host threads) race and must not
 *     be made.  Calls in sequence on one stream are safe; the array keeps the
 *     last call's contents, and the step needs none of them.
 */
size_t hst_noalloc_scratch_bytes(void);
hst_status hst_decode_step_softlsh_noalloc(const hst_shape* shape, const void* q,
                                           const void* K, const void* V,
                                           const void* W, int L, int P,
                                           double tau, const uint8_t* ids,
                                           const void* vnorm, int norm_dtype,
                                           int k, const int32_t* k_per_seq,
                                           float scale, int32_t* idx, float* out,
                                           float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HST_H_ */
