// The stored-G_S G_K/G_V pass for head dimension 128 on the ragged last key tile of a
// non-causal problem (n not a multiple of 128): the one instance whose loop masks keys >= n.
#include "bwd_dkdv.h"

namespace backlite {

hipError_t launch_dkdv_d128_gs_ragged(const BwdArgs& a, hipStream_t st) {
  const dim3 grid(2 * a.B * a.Hk * a.T), block(256);  // chunks of other key tiles return at once
  hipLaunchKernelGGL((dkdv_kernel<128, false, true, true>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace backlite
