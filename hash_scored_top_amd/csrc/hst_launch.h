// Host-side launchers of the HIP kernels (internal to libhst).  Each enqueues
// on the given stream and returns the launch status; arguments are already
// validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hst.h"

namespace hst {

hipError_t launch_hash_softlsh(const hst_shape& s, const void* K, const void* V, const void* W,
                               int L, int P, int norm_dtype, uint8_t* ids, void* vnorm,
                               hipStream_t st);
hipError_t launch_hash_binary(const hst_shape& s, const void* K, const void* R, uint32_t* codes,
                              hipStream_t st);

hipError_t launch_query_tables(const hst_shape& s, const void* q, const void* W, int L, int P,
                               float tau, float* tables, hipStream_t st);
hipError_t launch_query_codes(const hst_shape& s, const void* q, const void* R, uint32_t* qcodes,
                              hipStream_t st);

hipError_t launch_score_softlsh(const hst_shape& s, const float* tables, int L, int P,
                                const uint8_t* ids, const void* vnorm, int norm_dtype,
                                float* scores, hipStream_t st);
hipError_t launch_score_hamming(const hst_shape& s, const uint32_t* qcodes,
                                const uint32_t* codes, int32_t* scores, hipStream_t st);

size_t select_ws_bytes(const hst_shape& s);
hipError_t launch_select(const hst_shape& s, int score_dtype, const void* scores, int kcap,
                         const int32_t* k_per_seq, int32_t* idx, void* ws, hipStream_t st);

size_t attention_ws_bytes(const hst_shape& s, int kcap);
hipError_t launch_attention(const hst_shape& s, const void* q, const void* K, const void* V,
                            const int32_t* idx, int kcap, float scale, float* out, float* lse,
                            void* ws, hipStream_t st);

}  // namespace hst
