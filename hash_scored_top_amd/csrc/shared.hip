// Shared-prefix decode: a batch whose sequences share one prefix.
// Bifurcated-attention page, sections 1 and 3: the shared context and each
// sample's own incremental part are handled apart, so that the shared part
// is read once for the whole batch instead of once per sample.
//
// The context of sequence b is prefix (Np keys, one copy per kv head)
// followed by its own suffix (N_b keys); key j < Np is prefix key j, key
// Np + j suffix key j.  Every sequence's scores over that context are the
// plain step's; what changes is where the bytes come from.  The scan
// (scan_shared_kernel, with the plain scan's scorer) lays its prefix chunks
// out so that the B workgroups of one (kv head, chunk) have block ids
// congruent modulo 8, hence run on one XCD (blocks are dealt to the 8 XCDs
// round robin), and within 8*B consecutive ids, hence at about the same
// time: the prefix metadata leaves HBM once and the other B - 1 reads hit
// that XCD's L2.  The selection runs on the scores of the whole context;
// the attention kernel takes rows below Np from the prefix K/V.  Here: the
// context lengths.
#include "hst_common.h"
#include "hst_fused.h"
#include "hst_launch.h"

namespace hst {

__global__ void shared_lens_kernel(const int32_t* __restrict__ s_lens, int B, int Ns, int Np,
                                   int32_t* __restrict__ v_lens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B) v_lens[b] = Np + seq_len(s_lens, b, Ns);
}

hipError_t launch_shared_lens(const hst_shape& s, int Np, int32_t* v_lens, hipStream_t st) {
  hipLaunchKernelGGL(shared_lens_kernel, dim3((s.B + 255) / 256), dim3(256), 0, st, s.seq_lens,
                     s.B, s.Nmax, Np, v_lens);
  return hipGetLastError();
}

}  // namespace hst
