// Host-side launchers of the HIP kernels (internal to libhst).  Each enqueues
// on the given stream and returns the launch status; arguments are already
// validated by the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hst.h"

namespace hst {

// Raises the dynamic LDS limit of kernel `kern` on the current device to at
// least `bytes` (each kernel and device keeps the largest size asked so far).
hipError_t raise_lds_limit(const void* kern, size_t bytes);

hipError_t launch_hash_softlsh(const hst_shape& s, const void* K, const void* V, const void* W,
                               int L, int P, int norm_dtype, uint8_t* ids, void* vnorm,
                               hipStream_t st);
hipError_t launch_hash_binary(const hst_shape& s, const void* K, const void* R, int code_bits,
                              uint32_t* codes, hipStream_t st);
// bucket ids only (no value norms)
hipError_t launch_hash_ids_softlsh(const hst_shape& s, const void* K, const void* W, int L, int P,
                                   uint8_t* ids, hipStream_t st);
hipError_t launch_append_softlsh(const hst_shape& s, const void* k_new, const void* v_new,
                                 const void* W, int L, int P, int norm_dtype, void* K, void* V,
                                 uint8_t* ids, void* vnorm, hipStream_t st);
hipError_t launch_append_binary(const hst_shape& s, const void* k_new, const void* v_new,
                                const void* R, void* K, void* V, uint32_t* codes, hipStream_t st);

}  // namespace hst
