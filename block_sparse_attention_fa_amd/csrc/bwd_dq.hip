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
// Sources of key tile kt (K, V rows; the key mean) as buffer resources whose
// range ends after the last valid row: the rows of the ragged last tile, and
// everything when `valid` is false, read as zero.  Keys past the end are also
// masked out of P, so their zero rows never matter.
struct KvSrc {
  __amdgpu_buffer_rsrc_t k, v, m;
};
template <int D>
__device__ __forceinline__ KvSrc kv_src(const uint16_t* kbase, const uint16_t* vbase, const float* kbar, long stride,
                                        int n, int kt, bool valid) {
  const int key0 = kt * TILE;
  // list entries past the last tile (a malformed list) read as empty tiles
  const uint32_t rows = (valid && key0 < n) ? (uint32_t)min(TILE, n - key0) : 0u;
  const uint32_t bytes = rows * (uint32_t)stride * 2u;
  return KvSrc{buffer_rsrc(kbase + (long)key0 * stride, bytes), buffer_rsrc(vbase + (long)key0 * stride, bytes),
               buffer_rsrc(kbar + (long)kt * D, valid ? (uint32_t)D * 4u : 0u)};
}

// copy instruction I (of 2 NI) of a staged key tile: K rows, then V rows
template <int D, int NT, int I>
__device__ __forceinline__ void stage_kv_part(bf16* Kd, bf16* Vd, const KvSrc& s, const DmaOffsets<D, NT>& dmo,
                                              int wave) {
  constexpr int NI = DmaOffsets<D, NT>::NI, II = I % NI;
  lds_byte* dst = lds_ptr((I < NI ? Kd : Vd) + ((II * (NT / 64) + wave) * 64) * 8);
  load_lds16(I < NI ? s.k : s.v, dst, dmo.off[II]);
}

// the key mean of a staged key tile: wave 0, D / 64 instructions
template <int D>
__device__ __forceinline__ void stage_kbar(float* Bd, const KvSrc& s, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < D / 64; ++i)
    if (wave == 0) load_lds4(s.m, lds_ptr(Bd + 64 * i), (uint32_t)(64 * i + lane) * 4u);
}

// One workgroup of 4 waves (one per SIMD) per (b, h, query tile qt).  Wave w
// owns query rows 32w .. +31: their Q, G_O fragments and the G_Q^T accumulator
// stay in registers.  The next listed key tile is copied into the other LDS
// stage while the current one is consumed.
//
// With 64-row backward query tiles the workgroup still covers 128 rows (the
// tiles 2p and 2p+1: waves 0-1 and 2-3) and walks the union of the two
// q-lists, each entry flagged with the halves that keep it; a wave pair whose
// half does not keep the tile only issues its share of the staging copies.
// A half whose G_Q comes from stored G_S (dqs_kernel) is skipped entirely and
// its rows are not written here.
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
  __shared__ uint32_t itab[MAX_TILES];  // q-list (union of both halves): kt | halves keeping it << 16
  __shared__ uint8_t fl[2][MAX_TILES];  // 64-row tiles: which half keeps each key tile
  __shared__ int red[NT / 64];

  // with G_S slots, the query tiles whose kept tiles all have a slot take G_Q
  // from the stored tiles (dqs_kernel); only the others are recomputed here.
  // When every tile had a slot the workgroup leaves before any other load.
  if (a.gsinfo != nullptr && a.gsinfo[0] != 0) return;
  const int T = a.T, n = a.n;
  const int L = work_index(blockIdx.x);
  const int qt = L % T;
  const int bh = L / T;
  const int h = bh % a.H, b = bh / a.H;
  const int g = h / (a.H / a.Hk);

  // wave index as a scalar: branches and LDS copy destinations built from it stay scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const float lse2 = (qrow < n) ? a.lse2[(long)bh * n + qrow] : INFINITY;
  const float dl = (qrow < n) ? a.dbuf[(long)bh * n + qrow] : 0.f;
  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};
  const float c = a.scale_log2;
  const long kvstride = (long)a.Hk * D;
  const uint16_t* kbase = a.k + ((long)b * n) * kvstride + (long)g * D;
  const uint16_t* vbase = a.v + ((long)b * n) * kvstride + (long)g * D;
  const float* kbar = a.kbar + (long)(b * a.Hk + g) * T * D;
  const bool split = a.qrows != TILE;                     // two 64-row query tiles
  const int Tq = a.Tq;
  int cnt_h[2] = {0, 0};
  bool mine_h[2] = {false, false};                        // half recomputed here
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int t = split ? 2 * qt + hf : qt;
    if ((split || hf == 0) && t < Tq) {
      const long bq = (long)bh * Tq + t;
      cnt_h[hf] = max(0, min(a.qcnt[bq], T));
      mine_h[hf] = a.gsinfo == nullptr || (long long)a.qbase[bq] + cnt_h[hf] > a.gs_cap;
    }
  }
  if (!split) mine_h[1] = mine_h[0];
  if (!mine_h[0] && !mine_h[1]) return;
  int cnt;
  if (!split) {
    // the q-list in LDS: reading the next key tile is then an LDS read, not a
    // global load whose latency would stall the wave before the next copy
    cnt = cnt_h[0];
    const uint16_t* list = a.qidx + ((long)bh * Tq + qt) * T;
    for (int i = tid; i < cnt; i += NT) itab[i] = list[i] | (3u << 16);
  } else {
    // union of the two halves' lists (only halves recomputed here), in kt order
    for (int i = tid; i < T; i += NT) fl[0][i] = fl[1][i] = 0;
    __syncthreads();
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (!mine_h[hf]) continue;
      const uint16_t* list = a.qidx + ((long)bh * Tq + 2 * qt + hf) * T;
      for (int i = tid; i < cnt_h[hf]; i += NT) {
        const int kt = list[i];
        if (kt < T) fl[hf][kt] = 1;
      }
    }
    __syncthreads();
    constexpr int PER = MAX_TILES / NT;
    int f[PER], m = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int kt = tid * PER + u;
      f[u] = kt < T ? (fl[0][kt] | (fl[1][kt] << 1)) : 0;
      m += f[u] != 0;
    }
    // block-wide exclusive scan of m
    int x = m;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) red[wave] = x;
    __syncthreads();
    int base = 0;
    cnt = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      const int r = red[w];
      if (w < wave) base += r;
      cnt += r;
    }
    int pos = base + x - m;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (f[u]) itab[pos++] = (uint32_t)(tid * PER + u) | ((uint32_t)f[u] << 16);
  }
  LdsOffsets<D> lo;
  lo.init(lane);
  DmaOffsets<D, NT> dmo;
  dmo.init(kvstride, tid);
  __syncthreads();
  const int my_bit = split ? 1 << (wave >> 1) : 3;
  int kt_cur = (cnt > 0) ? (int)(__builtin_amdgcn_readfirstlane(itab[0]) & 0xFFFFu) : 0;
  int fl_cur = (cnt > 0) ? (int)(__builtin_amdgcn_readfirstlane(itab[0]) >> 16) : 0;

  using SC = TileSched<2 * NKS, 2 * NDB>;  // A: S^T, G_P^T of 32 keys; B: G_Q^T
  constexpr int NSTEP = SC::total;
  constexpr int NI = DmaOffsets<D, NT>::NI;
  constexpr int DSTEP = NSTEP / (2 * 2 * NI);  // the 2 NI copies span the first half
  constexpr int RING = 4, AHEAD = RING - 1;    // operand slots, MFMAs fetched ahead

  // stage S (a compile-time 0 or 1) holds item j; the other stage receives j + 1
  auto visit = [&](int j, auto stage) {
    constexpr int S = decltype(stage)::value;
    const bf16* Kc = S ? Ks1 : Ks0;
    const bf16* Vc = S ? Vs1 : Vs0;
    const float* Bc = S ? Kb1 : Kb0;
    bf16* Kn = S ? Ks0 : Ks1;
    bf16* Vn = S ? Vs0 : Vs1;
    float* Bn = S ? Kb0 : Kb1;
    const int kt = kt_cur;
    wait_vmem();
    __syncthreads();  // key tile kt staged in (Kc, Vc, Bc); stage n is free
    // Stage item j + 1: its key mean now, its K and V rows one copy instruction
    // every few MFMAs in the first half of this tile's stream (issued back to
    // back they would stall the wave).  Without a next item the copies read
    // nothing and land zeros in the free stage.
    const bool more = j + 1 < cnt;
    const uint32_t e_nxt = more ? __builtin_amdgcn_readfirstlane(itab[j + 1]) : 0u;
    const int kt_nxt = more ? (int)(e_nxt & 0xFFFFu) : kt;
    const int fl_nxt = (int)(e_nxt >> 16);
    const KvSrc nsrc = kv_src<D>(kbase, vbase, kbar, kvstride, n, kt_nxt, more);
    stage_kbar<D>(Bn, nsrc, wave, lane);
    if (!(fl_cur & my_bit)) {
      // this wave's half does not keep tile kt: only its share of the copies
      static_for<0, 2 * NI>([&](auto ic) { stage_kv_part<D, NT, decltype(ic)::value>(Kn, Vn, nsrc, dmo, wave); });
      kt_cur = kt_nxt;
      fl_cur = fl_nxt;
      return;
    }

    const int key0 = kt * TILE;
    // register r of chunk kb holds key key0 + 32kb + 4*h32 + 8(r/4) + r%4; a key
    // is dropped when it is padding (>= n) or, on the diagonal, after the row
    const bool diag = CAUSAL && (qt == kt);
    const bool edge = key0 + TILE > n;
    // with a sliding window, tiles reaching down to a row's window edge also drop
    // the keys <= row - window
    const bool wedge = CAUSAL && a.window != 0 && key0 <= qt * TILE + TILE - 1 - a.window;
    const int lim0 = (diag ? min(n - 1, qrow) : n - 1) - (key0 + 4 * h32);  // keep offsets <= lim0 - 32kb
    auto fetch = [&](auto kc) -> bf16x8 {
      constexpr int k = decltype(kc)::value, ph = SC::phase_of(k), st = k - SC::start(ph), cb = SC::chunk(ph);
      if constexpr (SC::is_b(ph)) return rd_tr<D>(Kc, lo, cb, st / NDB, st % NDB);
      else return rd_row<D>((st & 1) ? Vc : Kc, lo, cb, st >> 1);
    };
    f32x16 sacc[2], gacc[2];  // S^T and G_P^T (later P and G_S) of the two chunks in flight
    bf16x8 sb[2][2];          // packed bf16 G_S^T operands [chunk parity][sub-step]
    float csum = 0.f, bsum = 0.f;  // this row's sums over the tile's keys of G_S and of bf16(G_S)
    bf16x8 ring[RING];
    static_for<0, AHEAD>([&](auto kc) { ring[decltype(kc)::value] = fetch(kc); });
    static_for<0, NSTEP>([&](auto kc) {
      constexpr int k = decltype(kc)::value, ph = SC::phase_of(k), st = k - SC::start(ph), cb = SC::chunk(ph);
      if constexpr (k + AHEAD < NSTEP)
        ring[(k + AHEAD) % RING] = fetch(std::integral_constant<int, k + AHEAD>{});
      if constexpr (k % DSTEP == 0 && k / DSTEP < 2 * NI) stage_kv_part<D, NT, k / DSTEP>(Kn, Vn, nsrc, dmo, wave);
      if constexpr (st == 0 && !SC::is_b(ph)) {
        sacc[cb & 1] = f32x16{};
        gacc[cb & 1] = f32x16{};
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (SC::is_b(ph)) {
        dq[st % NDB] = mfma32(ring[k % RING], sb[cb & 1][st / NDB], dq[st % NDB]);
      } else {
        if constexpr (st & 1) gacc[cb & 1] = mfma32(ring[k % RING], gf[st >> 1], gacc[cb & 1]);
        else sacc[cb & 1] = mfma32(ring[k % RING], qf[st >> 1], sacc[cb & 1]);
      }
      // softmax elements whose turn is this MFMA
      static_for<0, 4>([&](auto cc) {
        constexpr int c4 = decltype(cc)::value;
        if constexpr (SC::soft_begin(c4) == k) {
          // masked keys (padding, or after the row on the diagonal) get score
          // -inf, so P = 0 there; only diagonal and ragged tiles take this branch
          if (diag || edge || wedge) {
            // and offsets > limw - 32kb
            const int limw = wedge ? (qrow - a.window) - (key0 + 4 * h32) : -(1 << 30);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int off = 8 * (r >> 2) + (r & 3);
              sacc[c4 & 1][r] = (off <= lim0 - 32 * c4 && off > limw - 32 * c4) ? sacc[c4 & 1][r] : -INFINITY;
            }
          }
        }
        static_for<0, 16>([&](auto ec) {
          constexpr int r = decltype(ec)::value;
          if constexpr (SC::elem_step(c4, r) == k) {
            const float pv = fast_exp2(fmaf(sacc[c4 & 1][r], c, -lse2));
            const float gs = pv * (gacc[c4 & 1][r] - dl);
            gacc[c4 & 1][r] = gs;
            csum += gs;
          }
        });
        if constexpr (SC::soft_end(c4) - 1 == k) {
          sb[c4 & 1][0] = pack8(gacc[c4 & 1], 0);
          sb[c4 & 1][1] = pack8(gacc[c4 & 1], 1);
          // sum of the bf16 operands: pairs of bf16 dotted with (1, 1)
          const bf16x2 one = {(bf16)1.f, (bf16)1.f};
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const bf16x2 pr = {sb[c4 & 1][s2][2 * u], sb[c4 & 1][s2][2 * u + 1]};
              bsum = __builtin_amdgcn_fdot2_f32_bf16(pr, one, bsum, false);
            }
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    // Rounding compensation.  The MFMA used bf16(G_S); the residual
    // lo = G_S - bf16(G_S) contributes sum_j lo_ij K_j, whose dominant part when
    // the tile's keys share a large common vector is (sum_j lo_ij) * kbar.  Rows
    // of G_S nearly sum to zero, so without this term that common vector would
    // multiply the rounding error.  Exact algebra: the leftover error is
    // sum_j lo_ij (K_j - kbar).  The rank-1 update kbar (x) losum is one MFMA per
    // 32-dim block whose A and B operands are zero except for contraction slot 0
    // (bf16 operands: the term is already a rounding-sized correction).
    float losum = csum - bsum;
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
    kt_cur = kt_nxt;
    fl_cur = fl_nxt;
  };

  {
    const KvSrc s0 = kv_src<D>(kbase, vbase, kbar, kvstride, n, kt_cur, cnt > 0);
    stage_kbar<D>(Kb0, s0, wave, lane);
    static_for<0, 2 * NI>([&](auto ic) { stage_kv_part<D, NT, decltype(ic)::value>(Ks0, Vs0, s0, dmo, wave); });
  }
  // pairs of items (stage 0, then stage 1), then the odd one out: no branch
  // between the two visits of an iteration
  int j = 0;
  for (; j + 1 < cnt; j += 2) {
    visit(j, std::integral_constant<int, 0>{});
    visit(j + 1, std::integral_constant<int, 1>{});
  }
  if (j < cnt) visit(j, std::integral_constant<int, 0>{});

  // epilogue: dq C layout is [dim = 32db + 8(r/4) + 4*h32 + r%4][query l32]
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int dim = db * 32 + 8 * jj + 4 * h32;
      bf16x4 w4 = {(bf16)(dq[db][4 * jj] * a.scale), (bf16)(dq[db][4 * jj + 1] * a.scale),
                   (bf16)(dq[db][4 * jj + 2] * a.scale), (bf16)(dq[db][4 * jj + 3] * a.scale)};
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
      if (qt * TILE + row < n && mine_h[split ? row / 64 : 0])  // rows of a stored half are dqs_kernel's
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
