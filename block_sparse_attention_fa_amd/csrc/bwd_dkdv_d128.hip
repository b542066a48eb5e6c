// Instances of the G_K/G_V pass for head dimension 128, plain variant (one translation
// unit per head dimension and variant, so the kernels compile in parallel).
#include "bwd_dkdv.h"

namespace backlite {

hipError_t launch_dkdv_d128(const BwdArgs& a, bool causal, hipStream_t st) {
  const dim3 grid(2 * a.B * a.Hk * a.T), block(256);  // at most 2 chunks per key tile on average
  if (causal) hipLaunchKernelGGL((dkdv_kernel<128, true, false, false>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((dkdv_kernel<128, false, false, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace backlite
