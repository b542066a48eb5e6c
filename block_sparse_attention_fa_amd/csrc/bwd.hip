// Block-sparse attention backward: D preprocess, G_K/G_V pass, G_Q pass.
//
// What it computes ("Introducing BackLite", backward equations and "Using
// Sparsity"; BackLite README, "How It Works"): with P rebuilt from Q, K and the
// stored row LSE (FlashAttention tutorial, "Flash Attention Backward Pass"),
//   D = rowsum(G_O * O)                 (full row, once, before the tiles)
//   G_V += P^T G_O,  G_P = G_O V^T,  G_S = P * (G_P - D),
//   G_K += scale * G_S^T Q,  G_Q += scale * G_S K
// over the kept tile pairs only; skipped tiles are never loaded.
//
// dkdv_kernel: one workgroup per (b, kv head g, key tile kt) walks, for every
//   query head of the group, that head's list of kept query tiles.  Per query
//   tile, Q and G_O sit row-major in LDS; S = Q K^T and G_P = G_O V^T read them
//   as row operands, G_V and G_K read them through the LDS transpose read.
// dq_kernel (bwd_dq.hip): one workgroup per (b, h, query tile qt) walks the
//   tile's list of kept key tiles with K, V row-major in LDS.
// Stored-G_S path (bwd_gs.hip), taken when the workspace has a slot for every
//   kept tile: the G_K/G_V pass also writes each tile's bf16 G_S, and the G_Q
//   pass multiplies the stored G_S by K instead of rebuilding P and G_S.
// Every pass is free of atomics, so results are bit-reproducible.
#include "bl_device.h"
#include "bwd_common.h"
#include "prof.h"

namespace backlite {

hipError_t launch_dq(const BwdArgs& a, int d, bool causal, hipStream_t st);
// G_K/G_V pass instances (bwd_dkdv_d*.hip; the _gs variants also store G_S)
hipError_t launch_dkdv_d64(const BwdArgs& a, bool causal, hipStream_t st);
hipError_t launch_dkdv_d128(const BwdArgs& a, bool causal, hipStream_t st);
hipError_t launch_dkdv_d64_gs(const BwdArgs& a, bool causal, hipStream_t st);
hipError_t launch_dkdv_d128_gs(const BwdArgs& a, bool causal, hipStream_t st);
// stored-G_S path (bwd_gs.hip): slot assignment, G_Q from stored G_S
hipError_t launch_gs_slots(const BwdArgs& a, hipStream_t st);
hipError_t launch_dq_gs(const BwdArgs& a, int d, hipStream_t st);

// ---------------------------------------------------------------------------
// D[b,h,i] = sum_c G_O[b,i,h,c] * O[b,i,h,c]; 16 lanes per (i, h) row of d = 128
// (8 lanes for d = 64), one 16-byte load of each operand per lane.  With the
// forward's residual, O is taken as O + O_lo (about 16 significant bits): an
// error in D shifts a whole row of G_S, whose row sum should vanish, and G_Q
// then picks up that shift times the mean key vector.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row
  const long rows = (long)a.B * a.n * a.H;
  const long row = (long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 ov = *reinterpret_cast<const u32x4*>(a.o + row * D + sub * 8);
    const u32x4 gv = *reinterpret_cast<const u32x4*>(a.dout + row * D + sub * 8);
    const bf16x8 o8 = __builtin_bit_cast(bf16x8, ov);
    const bf16x8 g8 = __builtin_bit_cast(bf16x8, gv);
    float of[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) of[u] = (float)o8[u];
    if (a.olo) {
      const bf16x8 r8 = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(a.olo + row * D + sub * 8));
#pragma unroll
      for (int u = 0; u < 8; ++u) of[u] += (float)r8[u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc = fmaf(of[u], (float)g8[u], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (row < rows && sub == 0) {
    // row = (b*n + i)*H + h  ->  D[(b*H + h)*n + i]
    const int h = (int)(row % a.H);
    const long bi = row / a.H;
    const int i = (int)(bi % a.n);
    const int b = (int)(bi / a.n);
    const long ri = ((long)b * a.H + h) * a.n + i;
    a.dbuf[ri] = acc;
    a.lse2[ri] = a.lse[ri] * LOG2E;
  }
}

// ---------------------------------------------------------------------------
// kbar[b,g,kt,:] = mean of K over the valid keys of tile kt (fp32).  Used by the
// G_Q pass to compensate the bf16 rounding of G_S (see dq_kernel).  One
// workgroup per (b, g, kt); thread t sums rows t/(D/8) + 256/(D/8)*i of the
// 8-column chunk t%(D/8), then the partial sums meet in LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void kmean_kernel(BwdArgs a) {
  constexpr int CH = D / 8;
  constexpr int RSTEP = 256 / CH;
  __shared__ float part[RSTEP][D];
  const int T = a.T, n = a.n;
  const int kt = blockIdx.x % T;
  const int bg = blockIdx.x / T;
  const int g = bg % a.Hk, b = bg / a.Hk;
  const int tid = threadIdx.x, ch = tid % CH, r0 = tid / CH;
  const long stride = (long)a.Hk * D;
  const uint16_t* kp = a.k + ((long)b * n + (long)kt * TILE) * stride + (long)g * D + ch * 8;
  const int nv = min(TILE, n - kt * TILE);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = r0; r < nv; r += RSTEP) {
    const bf16x8 v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kp + (long)r * stride));
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += (float)v[u];
  }
#pragma unroll
  for (int u = 0; u < 8; ++u) part[r0][ch * 8 + u] = acc[u];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < RSTEP; ++i) s += part[i][tid];
    a.kbar[((long)bg * T + kt) * D + tid] = s / (float)nv;
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  {
    const long rows = (long)a.B * a.n * a.H;
    const long rpb = 256 / (D / 8);
    ProfScope ps(PK_DELTA, st);
    hipLaunchKernelGGL((delta_kernel<D>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps(PK_KMEAN, st);
    hipLaunchKernelGGL((kmean_kernel<D>), dim3(a.B * a.Hk * a.T), dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // With slots in the workspace, the slot pass decides on the device whether
  // every kept tile fits; the variant of each pass that does not apply returns
  // at once.
  if (a.gsinfo) {
    e = launch_gs_slots(a, st);
    if (e != hipSuccess) return e;
    ProfScope ps(PK_DKDV, st);
    e = D == 64 ? launch_dkdv_d64_gs(a, CAUSAL, st) : launch_dkdv_d128_gs(a, CAUSAL, st);
    if (e != hipSuccess) return e;
  }
  {
    ProfScope ps(PK_DKDV, st);
    e = D == 64 ? launch_dkdv_d64(a, CAUSAL, st) : launch_dkdv_d128(a, CAUSAL, st);
  }
  if (e != hipSuccess) return e;
  e = launch_dq(a, D, CAUSAL, st);
  if (e != hipSuccess || !a.gsinfo) return e;
  return launch_dq_gs(a, D, st);
}

hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                      const uint16_t* olo, const uint16_t* dout, const float* lse, const int32_t* qcnt,
                      const uint16_t* qidx, const int32_t* kcnt, const uint16_t* kidx, int B, int n,
                      int H, int Hk, int d, float scale, int causal, uint16_t* dq, uint16_t* dk,
                      uint16_t* dv, float* dbuf, float* lse2, float* kbar, int32_t* gsinfo, uint32_t* qbase,
                      uint32_t* kslot, uint16_t* gs, float* gsl, long long gs_cap, hipStream_t st) {
  BwdArgs a{q,    k,      v,     o,     olo, dout, lse,    qcnt, qidx, kcnt, kidx, dq,
            dk,   dv,     dbuf,  lse2,  kbar, gsinfo, qbase, kslot, gs, gsl, gs_cap, B,
            n,    H,      Hk,    (n + TILE - 1) / TILE, scale, scale * LOG2E};
  if (d == 64) return causal ? launch_bwd_t<64, true>(a, st) : launch_bwd_t<64, false>(a, st);
  return causal ? launch_bwd_t<128, true>(a, st) : launch_bwd_t<128, false>(a, st);
}

}  // namespace backlite
