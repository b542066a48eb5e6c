// Sums behind the gradient-similarity metrics of the negl_prob calibration:
// for two bf16 tensors a, b of m elements, S = (sum a*b, sum a*a, sum b*b,
// sum (a-b)^2) in fp64, from which cosine = S0 / sqrt(S1 S2) and relative L2 =
// sqrt(S3 / S2) ("Introducing BackLite", "Experiments": BackLite's gradients
// are compared with exact attention's by cosine similarity and relative L2).
//
// Two launches, deterministic: SIM_NB workgroups each reduce a strided share
// of the elements (fp32 per element product, fp64 accumulation) to one partial
// per sum, then one workgroup adds the partials in index order.  HBM-bound:
// 4 bytes read per element pair.
#include "bl_device.h"

namespace backlite {

constexpr int SIM_NB = 512, SIM_NT = 256;

__device__ __forceinline__ double block_sum(double v, double* red) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double s = 0.0;
  if (tid == 0)
    for (int w = 0; w < SIM_NT / 64; ++w) s += red[w];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(SIM_NT) void similarity_partial_kernel(const uint16_t* a, const uint16_t* b, long m,
                                                                    double* part) {
  __shared__ double red[SIM_NT / 64];
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  const long m8 = m / 8;
  const long stride = (long)SIM_NB * SIM_NT;
  // 16-byte loads over the multiple-of-8 prefix, then the tail element-wise
  for (long i = (long)blockIdx.x * SIM_NT + threadIdx.x; i < m8; i += stride) {
    const bf16x8 x = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a + 8 * i));
    const bf16x8 y = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(b + 8 * i));
    float t[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float xa = (float)x[u], yb = (float)y[u], df = xa - yb;
      t[0] = fmaf(xa, yb, t[0]);
      t[1] = fmaf(xa, xa, t[1]);
      t[2] = fmaf(yb, yb, t[2]);
      t[3] = fmaf(df, df, t[3]);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] += (double)t[j];
  }
  for (long i = 8 * m8 + (long)blockIdx.x * SIM_NT + threadIdx.x; i < m; i += stride) {
    const float xa = (float)__builtin_bit_cast(bf16, a[i]), yb = (float)__builtin_bit_cast(bf16, b[i]);
    s[0] += (double)(xa * yb);
    s[1] += (double)(xa * xa);
    s[2] += (double)(yb * yb);
    s[3] += (double)((xa - yb) * (xa - yb));
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double t = block_sum(s[j], red);
    if (threadIdx.x == 0) part[j * SIM_NB + blockIdx.x] = t;
  }
}

__global__ __launch_bounds__(SIM_NT) void similarity_final_kernel(const double* part, double* out) {
  __shared__ double red[SIM_NT / 64];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    double v = 0.0;
    for (int i = threadIdx.x; i < SIM_NB; i += SIM_NT) v += part[j * SIM_NB + i];
    const double t = block_sum(v, red);
    if (threadIdx.x == 0) out[j] = t;
  }
}

size_t similarity_elems() { return 4 + 4 * (size_t)SIM_NB; }

hipError_t launch_similarity(const uint16_t* a, const uint16_t* b, long m, double* out, hipStream_t st) {
  double* part = out + 4;
  hipLaunchKernelGGL(similarity_partial_kernel, dim3(SIM_NB), dim3(SIM_NT), 0, st, a, b, m, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(similarity_final_kernel, dim3(1), dim3(SIM_NT), 0, st, part, out);
  return hipGetLastError();
}

}  // namespace backlite
