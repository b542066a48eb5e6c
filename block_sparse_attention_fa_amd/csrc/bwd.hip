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
// Both passes are free of atomics, so results are bit-reproducible.
#include "bl_device.h"
#include "bwd_common.h"
#include "prof.h"

namespace backlite {

hipError_t launch_dq(const BwdArgs& a, int d, bool causal, hipStream_t st);

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
    a.dbuf[((long)b * a.H + h) * a.n + i] = acc;
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

// ---------------------------------------------------------------------------
// G_K, G_V
// ---------------------------------------------------------------------------
// Work items of a (b, g, kt) workgroup: for each query head h of the group, the
// kept query tiles of key tile kt in that head's k-list.
struct KItems {
  int hh, it, cnt;  // current head of the group, position in its list, list length
};

// Stage Q, G_O, LSE and D of query tile qt of head bh into LDS; asynchronously
// for full tiles, synchronously (zero / +inf padding) for the ragged last one.
template <int D, int NT>
__device__ __forceinline__ void stage_qg(bf16* Qd, bf16* Gd, float* Ld, float* Dd, const BwdArgs& a,
                                         const DmaOffsets<D, NT>& dmo, long bh, int b, int h, int qt, int tid) {
  const int n = a.n;
  const long qstride = (long)a.H * D;
  const int q0 = qt * TILE;
  const uint16_t* qsrc = a.q + ((long)b * n + q0) * qstride + (long)h * D;
  const uint16_t* gsrc = a.dout + ((long)b * n + q0) * qstride + (long)h * D;
  if (q0 + TILE <= n) {
    dma_tile<D, NT>(Qd, qsrc, dmo, tid);
    dma_tile<D, NT>(Gd, gsrc, dmo, tid);
    const int wave = tid >> 6, lane = tid & 63;
    if (wave == 0) dma_words(Ld, a.lse + bh * n + q0, TILE, lane);
    if (wave == 1) dma_words(Dd, a.dbuf + bh * n + q0, TILE, lane);
  } else {
    load_tile<D, NT>(Qd, qsrc, qstride, n - q0, tid);
    load_tile<D, NT>(Gd, gsrc, qstride, n - q0, tid);
    if (tid < TILE) {
      const int i = q0 + tid;
      Ld[tid] = (i < n) ? a.lse[bh * n + i] : INFINITY;
      Dd[tid] = (i < n) ? a.dbuf[bh * n + i] : 0.f;
    }
  }
}

// One workgroup of 4 waves (one per SIMD, so each wave may hold up to 512
// registers) per (b, kv head g, key tile kt).  Wave w owns keys 32w .. +31 of
// the tile; their K, V fragments and G_K, G_V accumulators stay in registers.
// The next listed query tile is copied into the other LDS stage while the
// current one is consumed.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs a) {
  constexpr int NT = 256;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 Qs0[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Gs0[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Qs1[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Gs1[TILE * D];
  __shared__ __attribute__((aligned(16))) float Ls0[TILE];  // natural-log row LSE
  __shared__ __attribute__((aligned(16))) float Ds0[TILE];
  __shared__ __attribute__((aligned(16))) float Ls1[TILE];
  __shared__ __attribute__((aligned(16))) float Ds1[TILE];

  const int T = a.T, n = a.n;
  const int L = work_index(blockIdx.x);
  const int kt = L % T;
  const int bg = L / T;
  const int g = bg % a.Hk, b = bg / a.Hk;
  const int G = a.H / a.Hk;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h32 = lane >> 5;
  const int kw = wave;
  const int key = kt * TILE + kw * 32 + l32;  // this lane's key (B-operand column)

  const long kvstride = (long)a.Hk * D;
  bf16x8 kf[NKS], vf[NKS];
  {
    const long base = ((long)b * n) * kvstride + (long)g * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (key < n) {
        kv = *reinterpret_cast<const u32x4*>(a.k + base + (long)key * kvstride + ks * 16 + h32 * 8);
        vv = *reinterpret_cast<const u32x4*>(a.v + base + (long)key * kvstride + ks * 16 + h32 * 8);
      }
      kf[ks] = __builtin_bit_cast(bf16x8, kv);
      vf[ks] = __builtin_bit_cast(bf16x8, vv);
    }
  }
  f32x16 dk[NDB], dv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  const float c = a.scale_log2;
  LdsOffsets<D> lo;
  lo.init(lane);
  DmaOffsets<D, NT> dmo;
  dmo.init((long)a.H * D, tid);

  // flattened work list over the group's heads
  const long bh0 = (long)b * a.H + (long)g * G;
  int nitems = 0;
  for (int hh = 0; hh < G; ++hh) nitems += a.kcnt[(bh0 + hh) * T + kt];
  KItems cur{0, 0, a.kcnt[bh0 * T + kt]};
  auto skip_empty = [&](KItems& s) {
    while (s.it >= s.cnt && s.hh + 1 < G) {
      ++s.hh;
      s.it = 0;
      s.cnt = a.kcnt[(bh0 + s.hh) * T + kt];
    }
  };
  skip_empty(cur);
  KItems nxt = cur;
  auto qt_of = [&](const KItems& s) { return (int)a.kidx[((bh0 + s.hh) * T + kt) * T + s.it]; };
  auto advance = [&](KItems& s) {
    ++s.it;
    skip_empty(s);
  };

  auto visit = [&](int j, const bf16* Qc, const bf16* Gc, const float* Lc, const float* Dc, bf16* Qn,
                   bf16* Gn, float* Ln, float* Dn) {
    const int qt = qt_of(cur);
    wait_vmem();
    __syncthreads();  // item j staged in (Qc, Gc, Lc, Dc); stage n is free
    if (j + 1 < nitems) {
      advance(nxt);
      stage_qg<D, NT>(Qn, Gn, Ln, Dn, a, dmo, bh0 + nxt.hh, b, (int)(g * G + nxt.hh), qt_of(nxt), tid);
    }
    const int q0 = qt * TILE;
    const bool diag = CAUSAL && (qt == kt);
    // Per 32-query chunk qc: [S, G_P MFMAs] -> [P, G_S on the VALU] -> [G_V, G_K
    // MFMAs].  The chunks are software-pipelined: chunk qc+1's S and G_P MFMAs
    // are issued before chunk qc's VALU work, so the matrix pipe stays busy
    // while the wave computes exponentials.
    auto mm_sdp = [&](int qc, f32x16& sv, f32x16& gv) {
      bf16x8 qfr[NKS], gfr[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        qfr[ks] = rd_row<D>(Qc, lo, qc, ks);
        gfr[ks] = rd_row<D>(Gc, lo, qc, ks);
      }
      sv = f32x16{};
      gv = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        sv = mfma32(qfr[ks], kf[ks], sv);
        gv = mfma32(gfr[ks], vf[ks], gv);
      }
      sched_interleave<6, NKS - 3, 2, 2, 6>();
    };
    auto soft = [&](int qc, f32x16& sv, f32x16& gv) {
      // register r holds query q0 + 32qc + 4*h32 + (8(r/4) + r%4); on the
      // diagonal tile a key after the query is dropped
      const int lim = key - (q0 + qc * 32 + 4 * h32);  // drop offsets < lim
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const int qr = qc * 32 + 8 * j4 + 4 * h32;  // local query row of registers 4j4..4j4+3
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lc + qr);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(Dc + qr);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 4 * j4 + t;
          float pv = fast_exp2(fmaf(sv[r], c, -l4[t] * LOG2E));
          if (diag) pv = (8 * j4 + t >= lim) ? pv : 0.f;
          sv[r] = pv;
          gv[r] = pv * (gv[r] - d4[t]);
        }
      }
    };
    // G_V += P^T G_O and G_K += G_S^T Q; step st covers queries
    // 32qc + 16st + 4*h32 + 0..3 and 32qc + 16st + 8 + 4*h32 + 0..3
    auto mm_dvdk = [&](int qc, const f32x16& pv, const f32x16& sv) {
      bf16x8 gb[2][NDB], qb[2][NDB];
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          gb[st][db] = rd_tr<D>(Gc, lo, qc, st, db);
          qb[st][db] = rd_tr<D>(Qc, lo, qc, st, db);
        }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8 pa = pack8(pv, st);
        const bf16x8 sa = pack8(sv, st);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dv[db] = mfma32(pa, gb[st][db], dv[db]);
          dk[db] = mfma32(sa, qb[st][db], dk[db]);
        }
      }
      sched_interleave<8, 4 * NDB - 4, 1, 2, 4>();
    };
    f32x16 sA, gA, sB, gB;
    mm_sdp(0, sA, gA);
    mm_sdp(1, sB, gB);
    soft(0, sA, gA);
    mm_dvdk(0, sA, gA);
    mm_sdp(2, sA, gA);
    soft(1, sB, gB);
    mm_dvdk(1, sB, gB);
    mm_sdp(3, sB, gB);
    soft(2, sA, gA);
    mm_dvdk(2, sA, gA);
    soft(3, sB, gB);
    mm_dvdk(3, sB, gB);
    advance(cur);
  };

  if (nitems > 0)
    stage_qg<D, NT>(Qs0, Gs0, Ls0, Ds0, a, dmo, bh0 + cur.hh, b, (int)(g * G + cur.hh), qt_of(cur), tid);
  for (int j = 0; j < nitems; j += 2) {
    visit(j, Qs0, Gs0, Ls0, Ds0, Qs1, Gs1, Ls1, Ds1);
    if (j + 1 < nitems) visit(j + 1, Qs1, Gs1, Ls1, Ds1, Qs0, Gs0, Ls0, Ds0);
  }

  // epilogue: stage as [key][dim] bf16 and store coalesced rows.
  // C layout: [key = 8(r/4) + 4*h32 + r%4 of block kw][dim = 32db + l32].
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = kw * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
      const int dim = db * 32 + l32;
      const int off = tile_off<D>(kr, dim >> 3) + (dim & 7);
      Qs0[off] = (bf16)(dk[db][r] * a.scale);
      Gs0[off] = (bf16)dv[db][r];
    }
  __syncthreads();
  {
    constexpr int CH = D / 8;
    const long base = ((long)b * n + (long)kt * TILE) * kvstride + (long)g * D;
#pragma unroll
    for (int it = 0; it < TILE * CH / NT; ++it) {
      const int cc = tid + it * NT;
      const int row = cc / CH, ch = cc % CH;
      if (kt * TILE + row < n) {
        *reinterpret_cast<u32x4*>(a.dk + base + (long)row * kvstride + ch * 8) =
            *reinterpret_cast<const u32x4*>(Qs0 + tile_off<D>(row, ch));
        *reinterpret_cast<u32x4*>(a.dv + base + (long)row * kvstride + ch * 8) =
            *reinterpret_cast<const u32x4*>(Gs0 + tile_off<D>(row, ch));
      }
    }
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
  {
    ProfScope ps(PK_DKDV, st);
    hipLaunchKernelGGL((dkdv_kernel<D, CAUSAL>), dim3(a.B * a.Hk * a.T), dim3(256), 0, st, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dq(a, D, CAUSAL, st);
}

hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                      const uint16_t* olo, const uint16_t* dout, const float* lse, const int32_t* qcnt,
                      const uint16_t* qidx, const int32_t* kcnt, const uint16_t* kidx, int B, int n,
                      int H, int Hk, int d, float scale, int causal, uint16_t* dq, uint16_t* dk,
                      uint16_t* dv, float* dbuf, float* kbar, hipStream_t st) {
  BwdArgs a{q,  k,  v,    o,    olo, dout, lse, qcnt, qidx, kcnt, kidx, dq,
            dk, dv, dbuf, kbar, B,   n,    H,   Hk,   (n + TILE - 1) / TILE, scale, scale * LOG2E};
  if (d == 64) return causal ? launch_bwd_t<64, true>(a, st) : launch_bwd_t<64, false>(a, st);
  return causal ? launch_bwd_t<128, true>(a, st) : launch_bwd_t<128, false>(a, st);
}

}  // namespace backlite
