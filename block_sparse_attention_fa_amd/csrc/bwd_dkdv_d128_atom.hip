// Instances of the G_K/G_V pass for head dimension 128 with the fp32-atomic G_Q product
// (the fused single-pass backward variant; one translation unit per head dimension).
#include "bwd_dkdv.h"

namespace backlite {

hipError_t launch_dkdv_d128_atom(const BwdArgs& a, bool causal, hipStream_t st) {
  const dim3 grid(2 * a.B * a.Hk * a.T), block(256);  // at most 2 chunks per key tile on average
  if (causal) hipLaunchKernelGGL((dkdv_kernel<128, true, false, false, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((dkdv_kernel<128, false, false, false, true>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace backlite
