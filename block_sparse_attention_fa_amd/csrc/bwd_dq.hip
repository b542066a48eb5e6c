// Block-sparse attention backward, G_Q pass: for each query tile, over its
// kept key tiles, G_Q += scale * G_S K with P and G_S rebuilt from Q, K, V, G_O,
// the row LSE and D ("Introducing BackLite", backward equations and "Using
// Sparsity").  Built with MFMA results in arithmetic registers (the S / G_P
// accumulators feed VALU work directly); see build.py.
#include "bl_device.h"
#include "bwd_common.h"
#include "prof.h"

namespace backlite {

// ---------------------------------------------------------------------------
// G_Q
// ---------------------------------------------------------------------------
// Stage K, V and the key mean of key tile kt into LDS.
template <int D, int NT>
__device__ __forceinline__ void stage_kvb(bf16* Kd, bf16* Vd, float* Bd, const BwdArgs& a, const DmaOffsets<D, NT>& dmo,
                                          const uint16_t* kbase, const uint16_t* vbase, const float* kbar, int kt,
                                          int tid) {
  const int n = a.n;
  const long stride = (long)a.Hk * D;
  const int key0 = kt * TILE;
  if (key0 + TILE <= n) {
    dma_tile<D, NT, false>(Kd, kbase + (long)key0 * stride, dmo, tid);
    dma_tile<D, NT, false>(Vd, vbase + (long)key0 * stride, dmo, tid);
  } else {
    load_tile<D, NT>(Kd, kbase + (long)key0 * stride, stride, n - key0, tid);
    load_tile<D, NT>(Vd, vbase + (long)key0 * stride, stride, n - key0, tid);
  }
  if ((tid >> 6) == 0) dma_words<false>(Bd, kbar + (long)kt * D, D, tid & 63);
}

// One workgroup of 4 waves (one per SIMD) per (b, h, query tile qt).  Wave w
// owns query rows 32w .. +31: their Q, G_O fragments and the G_Q^T accumulator
// stay in registers.  The next listed key tile is copied into the other LDS
// stage while the current one is consumed.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void dq_kernel(BwdArgs a) {
  constexpr int NT = 256;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 Ks0[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs0[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Ks1[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs1[TILE * D];
  __shared__ __attribute__((aligned(16))) float Kb0[D];
  __shared__ __attribute__((aligned(16))) float Kb1[D];

  const int T = a.T, n = a.n;
  const int L = work_index(blockIdx.x);
  const int qt = L % T;
  const int bh = L / T;
  const int h = bh % a.H, b = bh / a.H;
  const int g = h / (a.H / a.Hk);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int lrow = wave * 32 + l32;
  const int qrow = qt * TILE + lrow;

  const long qstride = (long)a.H * D;
  bf16x8 qf[NKS], gf[NKS];
  {
    const long base = ((long)b * n) * qstride + (long)h * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 qv = {0u, 0u, 0u, 0u}, gv = {0u, 0u, 0u, 0u};
      if (qrow < n) {
        qv = *reinterpret_cast<const u32x4*>(a.q + base + (long)qrow * qstride + ks * 16 + h32 * 8);
        gv = *reinterpret_cast<const u32x4*>(a.dout + base + (long)qrow * qstride + ks * 16 + h32 * 8);
      }
      qf[ks] = __builtin_bit_cast(bf16x8, qv);
      gf[ks] = __builtin_bit_cast(bf16x8, gv);
    }
  }
  const float lse2 = (qrow < n) ? a.lse[(long)bh * n + qrow] * LOG2E : INFINITY;
  const float dl = (qrow < n) ? a.dbuf[(long)bh * n + qrow] : 0.f;
  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};
  const float c = a.scale_log2;
  const long kvstride = (long)a.Hk * D;
  const uint16_t* kbase = a.k + ((long)b * n) * kvstride + (long)g * D;
  const uint16_t* vbase = a.v + ((long)b * n) * kvstride + (long)g * D;
  const float* kbar = a.kbar + (long)(b * a.Hk + g) * T * D;
  const int cnt = a.qcnt[(long)bh * T + qt];
  const uint16_t* list = a.qidx + ((long)bh * T + qt) * T;
  LdsOffsets<D> lo;
  lo.init(lane);
  DmaOffsets<D, NT> dmo;
  dmo.init(kvstride, tid);

  auto visit = [&](int it, const bf16* Kc, const bf16* Vc, const float* Bc, bf16* Kn, bf16* Vn, float* Bn) {
    const int kt = list[it];
    wait_vmem();
    __syncthreads();  // key tile kt staged in (Kc, Vc, Bc); stage n is free
    if (it + 1 < cnt) stage_kvb<D, NT>(Kn, Vn, Bn, a, dmo, kbase, vbase, kbar, list[it + 1], tid);
    const int key0 = kt * TILE;
    const bool diag = CAUSAL && (qt == kt);
    const bool edge = key0 + TILE > n;
    float losum = 0.f;  // sum over this tile's keys of (G_S - bf16(G_S)) for this row
    // Per 32-key block kb: [S^T, G_P^T MFMAs] -> [G_S on the VALU] -> [G_Q MFMAs],
    // software-pipelined over kb like the G_K/G_V pass.
    auto mm_sdp = [&](int kb, f32x16& sv, f32x16& gv) {
      bf16x8 kfr[NKS], vfr[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        kfr[ks] = rd_row<D>(Kc, lo, kb, ks);
        vfr[ks] = rd_row<D>(Vc, lo, kb, ks);
      }
      sv = f32x16{};
      gv = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        sv = mfma32(kfr[ks], qf[ks], sv);
        gv = mfma32(vfr[ks], gf[ks], gv);
      }
      sched_interleave<6, NKS - 3, 2, 2, 6>();
    };
    auto soft = [&](int kb, const f32x16& sv, f32x16& gv) {
      // register r holds key key0 + 32kb + 4*h32 + (8(r/4) + r%4); a key is
      // dropped when it is padding (>= n) or, on the diagonal, after the row
      const int base = key0 + kb * 32 + 4 * h32;
      const int lim = (diag ? min(n - 1, qrow) : n - 1) - base;  // keep offsets <= lim
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = fast_exp2(fmaf(sv[r], c, -lse2));
        if (diag || edge) pv = (8 * (r >> 2) + (r & 3) <= lim) ? pv : 0.f;
        gv[r] = pv * (gv[r] - dl);
      }
    };
    // G_Q^T += K^T G_S^T; step st covers keys 32kb + 16st + 4*h32 + 0..3 and +8
    auto mm_dq = [&](int kb, const f32x16& gv) {
      bf16x8 ka[2][NDB];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < NDB; ++db) ka[st][db] = rd_tr<D>(Kc, lo, kb, st, db);
      bf16x8 sb[2];
      sb[0] = pack8_lo(gv, 0, losum);
      sb[1] = pack8_lo(gv, 1, losum);
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < NDB; ++db) dq[db] = mfma32(ka[st][db], sb[st], dq[db]);
      sched_interleave<6, 2 * NDB - 3, 1, 2, 3>();
    };
    f32x16 sA, gA, sB, gB;
    mm_sdp(0, sA, gA);
    mm_sdp(1, sB, gB);
    soft(0, sA, gA);
    mm_dq(0, gA);
    mm_sdp(2, sA, gA);
    soft(1, sB, gB);
    mm_dq(1, gB);
    mm_sdp(3, sB, gB);
    soft(2, sA, gA);
    mm_dq(2, gA);
    soft(3, sB, gB);
    mm_dq(3, gB);
    // Rounding compensation.  The MFMA used bf16(G_S); the residual
    // lo = G_S - bf16(G_S) contributes sum_j lo_ij K_j, whose dominant part when
    // the tile's keys share a large common vector is (sum_j lo_ij) * kbar.  Rows
    // of G_S nearly sum to zero, so without this term that common vector would
    // multiply the rounding error.  Exact algebra: the leftover error is
    // sum_j lo_ij (K_j - kbar).  The rank-1 update kbar (x) losum is one MFMA per
    // 32-dim block whose A and B operands are zero except for contraction slot 0
    // (bf16 operands: the term is already a rounding-sized correction).
    losum += __shfl_xor(losum, 32);
    {
      bf16x8 bl = {};
      if (h32 == 0) bl[0] = (bf16)losum;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        bf16x8 al = {};
        if (h32 == 0) al[0] = (bf16)Bc[db * 32 + l32];
        dq[db] = mfma32(al, bl, dq[db]);
      }
    }
  };

  if (cnt > 0) stage_kvb<D, NT>(Ks0, Vs0, Kb0, a, dmo, kbase, vbase, kbar, list[0], tid);
  for (int it = 0; it < cnt; it += 2) {
    visit(it, Ks0, Vs0, Kb0, Ks1, Vs1, Kb1);
    if (it + 1 < cnt) visit(it + 1, Ks1, Vs1, Kb1, Ks0, Vs0, Kb0);
  }

  // epilogue: dq C layout is [dim = 32db + 8(r/4) + 4*h32 + r%4][query l32]
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int dim = db * 32 + 8 * j + 4 * h32;
      bf16x4 w4 = {(bf16)(dq[db][4 * j] * a.scale), (bf16)(dq[db][4 * j + 1] * a.scale),
                   (bf16)(dq[db][4 * j + 2] * a.scale), (bf16)(dq[db][4 * j + 3] * a.scale)};
      *reinterpret_cast<bf16x4*>(Vs0 + tile_off<D>(lrow, dim >> 3) + (dim & 7)) = w4;
    }
  __syncthreads();
  {
    constexpr int CH = D / 8;
    uint16_t* op = a.dq + ((long)b * n + (long)qt * TILE) * qstride + (long)h * D;
#pragma unroll
    for (int it = 0; it < TILE * CH / NT; ++it) {
      const int cc = tid + it * NT;
      const int row = cc / CH, ch = cc % CH;
      if (qt * TILE + row < n)
        *reinterpret_cast<u32x4*>(op + (long)row * qstride + ch * 8) =
            *reinterpret_cast<const u32x4*>(Vs0 + tile_off<D>(row, ch));
    }
  }
}

hipError_t launch_dq(const BwdArgs& a, int d, bool causal, hipStream_t st) {
  ProfScope ps(PK_DQ, st);
  const dim3 grid(a.B * a.H * a.T), block(256);
  if (d == 64) {
    if (causal) hipLaunchKernelGGL((dq_kernel<64, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((dq_kernel<64, false>), grid, block, 0, st, a);
  } else {
    if (causal) hipLaunchKernelGGL((dq_kernel<128, true>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((dq_kernel<128, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace backlite
