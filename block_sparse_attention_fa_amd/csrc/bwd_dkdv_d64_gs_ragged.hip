// The stored-G_S G_K/G_V pass for head dimension 64 on the ragged last key tile of a
// non-causal problem (n not a multiple of 128): the one instance whose loop masks keys >= n.
#include "bwd_dkdv.h"

namespace backlite {

hipError_t launch_dkdv_d64_gs_ragged(const BwdArgs& a, hipStream_t st) {
  // one workgroup per (b, g) and possible chunk of its last key tile
  const dim3 grid(a.B * a.Hk * ragged_chunks_max(a)), block(256);
  hipLaunchKernelGGL((dkdv_kernel<64, false, true, true>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace backlite
