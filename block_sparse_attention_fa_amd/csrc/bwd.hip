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

// ---------------------------------------------------------------------------
// G_K, G_V
// ---------------------------------------------------------------------------
// Sources of query tile qt of head h (Q, G_O rows; LSE, D words) as buffer
// resources whose range ends after the last valid row: the rows of the ragged
// last tile, and every row when `valid` is false, read as zero.  Zero rows
// contribute nothing to G_K and G_V (their G_O and D are zero), so no other
// padding is needed.
struct QgSrc {
  __amdgpu_buffer_rsrc_t q, g, l, d;
};
template <int D>
__device__ __forceinline__ QgSrc qg_src(const BwdArgs& a, long bh, int b, int h, int qt, bool valid) {
  const int n = a.n;
  const long qstride = (long)a.H * D;
  const int q0 = qt * TILE;
  const uint32_t rows = valid ? (uint32_t)min(TILE, n - q0) : 0u;
  const long off = ((long)b * n + q0) * qstride + (long)h * D;
  const uint32_t bytes = rows * (uint32_t)qstride * 2u;
  return QgSrc{buffer_rsrc(a.q + off, bytes), buffer_rsrc(a.dout + off, bytes),
               buffer_rsrc(a.lse2 + bh * n + q0, rows * 4u), buffer_rsrc(a.dbuf + bh * n + q0, rows * 4u)};
}

// LSE and D words of a staged query tile: one instruction each, waves 0 and 1
__device__ __forceinline__ void stage_ld(float* Ld, float* Dd, const QgSrc& s, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < TILE / 64; ++i) {
    if (wave == 0) load_lds4<true>(s.l, nullptr, lds_ptr(Ld + 64 * i), (uint32_t)(64 * i + lane) * 4u);
    if (wave == 1) load_lds4<true>(s.d, nullptr, lds_ptr(Dd + 64 * i), (uint32_t)(64 * i + lane) * 4u);
  }
}

// Copy instruction i (of 2 NI) of a staged query tile: Q rows, then G_O rows.
template <int D, int NT, int I>
__device__ __forceinline__ void stage_qg_part(bf16* Qd, bf16* Gd, const QgSrc& s, const DmaOffsets<D, NT>& dmo,
                                              int wave) {
  constexpr int NI = DmaOffsets<D, NT>::NI, II = I % NI;
  lds_byte* dst = lds_ptr((I < NI ? Qd : Gd) + ((II * (NT / 64) + wave) * 64) * 8);
  load_lds16<true>(I < NI ? s.q : s.g, nullptr, dst, dmo.off[II]);
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
  constexpr int ITAB = 2048;  // work-list window held in LDS
  __shared__ uint32_t itab[ITAB];

  const int T = a.T, n = a.n;
  const int L = work_index(blockIdx.x);
  const int kt = L % T;
  const int bg = L / T;
  const int g = bg % a.Hk, b = bg / a.Hk;
  const int G = a.H / a.Hk;

  // wave index as a scalar: branches and LDS copy destinations built from it stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Flattened work list over the group's heads: item p is (head hh of the
  // group, query tile qt), heads in order, each head's k-list in order.  A
  // window of ITAB items is kept in LDS as (hh << 16 | qt), so reading the next
  // item is an LDS read, not a global load whose latency would stall the wave
  // between a tile's barrier and the copy of the next tile.
  const long bh0 = (long)b * a.H + (long)g * G;
  int nitems = 0;
  for (int hh = 0; hh < G; ++hh) nitems += a.kcnt[(bh0 + hh) * T + kt];
  auto fill_items = [&](int base) {  // items [base, base + ITAB) of the list, all threads
    int p0 = 0;
    for (int hh = 0; hh < G && p0 < base + ITAB; ++hh) {
      const long row = ((bh0 + hh) * T + kt);
      const int c = a.kcnt[row];
      const int lo_p = max(base, p0), hi_p = min(base + ITAB, p0 + c);
      for (int p = lo_p + tid; p < hi_p; p += NT) itab[p - base] = ((uint32_t)hh << 16) | a.kidx[row * T + (p - p0)];
      p0 += c;
    }
  };
  int ibase = 0;
  fill_items(0);
  __syncthreads();
  struct Item {
    int hh, qt;
  };
  auto item_at = [&](int p) -> Item {  // p in [ibase, ibase + ITAB)
    const uint32_t e = __builtin_amdgcn_readfirstlane(itab[p - ibase]);
    return Item{(int)(e >> 16), (int)(e & 0xFFFFu)};
  };
  Item it_cur = item_at(0);
  // stage S (a compile-time 0 or 1) holds item j; the other stage receives j + 1
  auto visit = [&](int j, auto stage) {
    constexpr int S = decltype(stage)::value;
    const bf16* Qc = S ? Qs1 : Qs0;
    const bf16* Gc = S ? Gs1 : Gs0;
    const float* Lc = S ? Ls1 : Ls0;
    const float* Dc = S ? Ds1 : Ds0;
    bf16* Qn = S ? Qs0 : Qs1;
    bf16* Gn = S ? Gs0 : Gs1;
    float* Ln = S ? Ls0 : Ls1;
    float* Dn = S ? Ds0 : Ds1;
    const int qt = it_cur.qt;
    wait_vmem();
    __syncthreads();  // item j staged in (Qc, Gc, Lc, Dc); stage n is free
    if (j + 1 >= ibase + ITAB && j + 1 < nitems) {  // slide the item window
      ibase += ITAB;
      fill_items(ibase);
      __syncthreads();
    }
    const Item it_nxt = (j + 1 < nitems) ? item_at(j + 1) : it_cur;
    // Stage item j + 1 into the free stage: its LSE and D words now, its Q and
    // G_O rows one copy instruction every few MFMAs in the first part of this
    // tile's stream (issued back to back they would stall the wave: the copy
    // pipeline holds few requests while rows stream in from HBM).  Without a
    // next item the copies read nothing and land zeros in the free stage.
    const QgSrc nsrc = qg_src<D>(a, bh0 + it_nxt.hh, b, (int)(g * G + it_nxt.hh), it_nxt.qt, j + 1 < nitems);
    stage_ld(Ln, Dn, nsrc, wave, lane);
    const int q0 = qt * TILE;
    // on the diagonal tile a query row drops keys after it
    const bool diag = CAUSAL && qt == kt;
    const int lim0 = key - (q0 + 4 * h32);
    // One tile: A(c) forms S and G_P of query chunk c (32 rows), B(c)
    // accumulates G_V and G_K from chunk c's P and G_S, in the order of
    // TileSched; chunk c's softmax (exp, mask, G_S) is spread over the MFMAs
    // between A(c) and B(c) so the VALU work hides under the matrix pipe.
    // Operands stream through a 4-slot ring fetched 3 MFMAs ahead;
    // sched_barrier fences keep that order.
    using SC = TileSched<2 * NKS, 4 * NDB>;
    constexpr int NSTEP = SC::total;
    constexpr int RING = 4, AHEAD = RING - 1;     // operand slots, MFMAs fetched ahead
    constexpr int NI = DmaOffsets<D, NT>::NI;
    constexpr int DSTEP = NSTEP / (2 * 2 * NI);   // the 2 NI copies span the first half
    auto fetch = [&](auto kc) -> bf16x8 {
      constexpr int k = decltype(kc)::value, ph = SC::phase_of(k), st = k - SC::start(ph), c4 = SC::chunk(ph);
      if constexpr (SC::is_b(ph)) {
        constexpr int sb = st >> 1;  // sub-step sb / NDB, head-dim block sb % NDB
        return rd_tr<D>((st & 1) ? Qc : Gc, lo, c4, sb / NDB, sb % NDB);
      } else {
        return rd_row<D>((st & 1) ? Gc : Qc, lo, c4, st >> 1);
      }
    };
    f32x16 sacc[2], gacc[2];  // S and G_P (later P and G_S) of the two chunks in flight
    bf16x8 pk[2][2], sk[2][2];  // packed bf16 P and G_S operands [chunk parity][sub-step]
    f32x4 l4[4], d4[4];         // LSE (log2 units) and D of the chunk in softmax
    bf16x8 ring[RING];
    static_for<0, AHEAD>([&](auto kc) { ring[decltype(kc)::value] = fetch(kc); });
    static_for<0, NSTEP>([&](auto kc) {
      constexpr int k = decltype(kc)::value, ph = SC::phase_of(k), st = k - SC::start(ph), c4 = SC::chunk(ph);
      if constexpr (k + AHEAD < NSTEP)
        ring[(k + AHEAD) % RING] = fetch(std::integral_constant<int, k + AHEAD>{});
      if constexpr (k % DSTEP == 0 && k / DSTEP < 2 * NI) stage_qg_part<D, NT, k / DSTEP>(Qn, Gn, nsrc, dmo, wave);
      if constexpr (st == 0 && !SC::is_b(ph)) {
        sacc[c4 & 1] = f32x16{};
        gacc[c4 & 1] = f32x16{};
      }
      static_for<0, 4>([&](auto cc) {
        constexpr int cs = decltype(cc)::value;
        if constexpr (SC::soft_begin(cs) == k) {
#pragma unroll
          for (int j4 = 0; j4 < 4; ++j4) {
            const int qr = cs * 32 + 8 * j4 + 4 * h32;
            l4[j4] = *reinterpret_cast<const f32x4*>(Lc + qr);
            d4[j4] = *reinterpret_cast<const f32x4*>(Dc + qr);
          }
        }
      });
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (SC::is_b(ph)) {
        constexpr int sb = st >> 1, s2 = sb / NDB, db = sb % NDB;
        if constexpr (st & 1) dk[db] = mfma32(sk[c4 & 1][s2], ring[k % RING], dk[db]);
        else dv[db] = mfma32(pk[c4 & 1][s2], ring[k % RING], dv[db]);
      } else {
        if constexpr (st & 1) gacc[c4 & 1] = mfma32(ring[k % RING], vf[st >> 1], gacc[c4 & 1]);
        else sacc[c4 & 1] = mfma32(ring[k % RING], kf[st >> 1], sacc[c4 & 1]);
      }
      static_for<0, 4>([&](auto cc) {
        constexpr int cs = decltype(cc)::value;
        f32x16& sv = sacc[cs & 1];
        f32x16& gv = gacc[cs & 1];
        if constexpr (CAUSAL && SC::soft_begin(cs) == k) {
          // on the diagonal tile a query drops the keys after it: score -inf,
          // so P = 0 there; only that tile takes this branch
          if (diag) {
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[r] = (8 * (r >> 2) + (r & 3) >= lim0 - cs * 32) ? sv[r] : -INFINITY;
          }
        }
        static_for<0, 16>([&](auto ec) {
          // register r holds query q0 + 32cs + 4*h32 + 8(r/4) + r%4
          constexpr int r = decltype(ec)::value, j4 = r >> 2, t = r & 3;
          if constexpr (SC::elem_step(cs, r) == k) {
            const float pv = fast_exp2(fmaf(sv[r], c, -l4[j4][t]));
            sv[r] = pv;
            gv[r] = pv * (gv[r] - d4[j4][t]);
          }
        });
        if constexpr (SC::soft_end(cs) - 1 == k) {
          pk[cs & 1][0] = pack8(sv, 0);
          pk[cs & 1][1] = pack8(sv, 1);
          sk[cs & 1][0] = pack8(gv, 0);
          sk[cs & 1][1] = pack8(gv, 1);
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    it_cur = it_nxt;
  };

  {
    const QgSrc s0 = qg_src<D>(a, bh0 + it_cur.hh, b, (int)(g * G + it_cur.hh), it_cur.qt, nitems > 0);
    stage_ld(Ls0, Ds0, s0, wave, lane);
    static_for<0, 2 * DmaOffsets<D, NT>::NI>([&](auto ic) { stage_qg_part<D, NT, decltype(ic)::value>(Qs0, Gs0, s0, dmo, wave); });
  }
  // pairs of items (stage 0, then stage 1), then the odd one out: no branch
  // between the two visits of an iteration, so the accumulators keep one
  // register assignment around the loop
  int j = 0;
  for (; j + 1 < nitems; j += 2) {
    visit(j, std::integral_constant<int, 0>{});
    visit(j + 1, std::integral_constant<int, 1>{});
  }
  if (j < nitems) visit(j, std::integral_constant<int, 0>{});

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
                      uint16_t* dv, float* dbuf, float* lse2, float* kbar, hipStream_t st) {
  BwdArgs a{q,    k,    v, o, olo, dout, lse, qcnt, qidx, kcnt, kidx, dq, dk, dv, dbuf,
            lse2, kbar, B, n, H,   Hk,   (n + TILE - 1) / TILE, scale, scale * LOG2E};
  if (d == 64) return causal ? launch_bwd_t<64, true>(a, st) : launch_bwd_t<64, false>(a, st);
  return causal ? launch_bwd_t<128, true>(a, st) : launch_bwd_t<128, false>(a, st);
}

}  // namespace backlite
