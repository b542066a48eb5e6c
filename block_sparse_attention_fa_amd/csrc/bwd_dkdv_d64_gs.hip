// Instances of the G_K/G_V pass for head dimension 64, stored-G_S variant (one translation
// unit per head dimension and variant, so the kernels compile in parallel).
#include "bwd_dkdv.h"

namespace backlite {

hipError_t launch_dkdv_d64_gs_ragged(const BwdArgs& a, hipStream_t st);

hipError_t launch_dkdv_d64_gs(const BwdArgs& a, bool causal, hipStream_t st) {
  const dim3 grid(2 * a.B * a.Hk * a.T), block(256);  // at most 2 chunks per key tile on average
  if (causal) {
    hipLaunchKernelGGL((dkdv_kernel<64, true, true, false>), grid, block, 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((dkdv_kernel<64, false, true, false>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  // the ragged last key tile (n not a multiple of 128) has an instance of its own
  if (e == hipSuccess && a.T * TILE != a.n) e = launch_dkdv_d64_gs_ragged(a, st);
  return e;
}

}  // namespace backlite
