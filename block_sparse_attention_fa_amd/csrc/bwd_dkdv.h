// G_K / G_V pass of the block-sparse backward ("Introducing BackLite",
// backward equations and "Using Sparsity"): one workgroup per (b, kv head g,
// key tile kt) walks, for every query head of the group, that head's list of
// kept query tiles.  Per query tile, Q and G_O sit row-major in LDS; S = Q K^T
// and G_P = G_O V^T read them as row operands, G_V and G_K read them through
// the LDS transpose read.
//
// With GS (the stored-G_S variant) the pass also writes every tile's G_S in
// bf16 to its slot of the workspace, with fp32 row sums of G_S over each
// quarter of the key tile, so that the G_Q pass is a plain product G_S K
// instead of a recomputation of S, P and G_P.  Included by bwd.hip (GS = false) and
// bwd_gs.hip (GS = true).
#pragma once
#include "bl_device.h"
#include "bwd_common.h"

namespace backlite {

// Sources of query tile qt (of a.qrows rows) of head h (Q, G_O rows; LSE, D
// words) as buffer resources whose range ends after the last valid row: the
// rows of the ragged last tile, and every row when `valid` is false, read as
// zero.  Zero rows contribute nothing to G_K and G_V (their G_O and D are
// zero), so no other padding is needed.  With shift = 64 the resources start 64
// rows before the tile, so that the copy offsets of stage rows 64..127 land on
// the tile's rows 0..63 (the second 64-row item of a visit); offsets below the
// shift are never issued for it.
struct QgSrc {
  __amdgpu_buffer_rsrc_t q, g, l, d;
};
template <int D>
__device__ __forceinline__ QgSrc qg_src(const BwdArgs& a, long bh, int b, int h, int qt, bool valid, int shift) {
  const int n = a.n;
  const long qstride = (long)a.H * D;
  const int q0 = qt * a.qrows;
  // list entries past the last tile (a malformed list) read as empty tiles
  const uint32_t rows = (valid && q0 < n) ? (uint32_t)min(a.qrows, n - q0) : 0u;
  const long r0 = (long)q0 - shift;
  const long off = ((long)b * n + r0) * qstride + (long)h * D;
  const uint32_t bytes = (rows + (uint32_t)shift) * (uint32_t)qstride * 2u;
  const uint32_t words = (rows + (uint32_t)shift) * 4u;
  return QgSrc{buffer_rsrc(a.q + off, bytes), buffer_rsrc(a.dout + off, bytes),
               buffer_rsrc(a.lse2 + bh * n + r0, words), buffer_rsrc(a.dbuf + bh * n + r0, words)};
}

// LSE and D words of a staged unit: one instruction each for stage rows 0..63
// (from sa) and 64..127 (from sb, the same source for a 128-row item), waves 0
// and 1
__device__ __forceinline__ void stage_ld(float* Ld, float* Dd, const QgSrc& sa, const QgSrc& sb, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < TILE / 64; ++i) {
    const QgSrc& s = i ? sb : sa;
    if (wave == 0) load_lds4(s.l, lds_ptr(Ld + 64 * i), (uint32_t)(64 * i + lane) * 4u);
    if (wave == 1) load_lds4(s.d, lds_ptr(Dd + 64 * i), (uint32_t)(64 * i + lane) * 4u);
  }
}

// Copy instruction i (of 2 NI) of a staged unit: Q rows, then G_O rows; the
// instructions of stage rows 64..127 read from sb.
template <int D, int NT, int I>
__device__ __forceinline__ void stage_qg_part(bf16* Qd, bf16* Gd, const QgSrc& sa, const QgSrc& sb,
                                              const DmaOffsets<D, NT>& dmo, int wave) {
  constexpr int NI = DmaOffsets<D, NT>::NI, II = I % NI;
  const QgSrc& s = II < NI / 2 ? sa : sb;  // instruction II covers stage rows 64 II / (NI / 2) ..
  lds_byte* dst = lds_ptr((I < NI ? Qd : Gd) + ((II * (NT / 64) + wave) * 64) * 8);
  load_lds16(I < NI ? s.q : s.g, dst, dmo.off[II]);
}

// The two results of v_permlane16_swap: x receives y's even 16-lane rows in
// place of its odd ones, y receives x's odd rows in place of its even ones.
__device__ __forceinline__ void swap16(float& x, float& y) {
  const uint64_t u = __builtin_bit_cast(
      uint64_t, __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, y),
                                                 false, false));
  x = __builtin_bit_cast(float, (uint32_t)u);
  y = __builtin_bit_cast(float, (uint32_t)(u >> 32));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// cache policy of the G_S stores and loads: non-temporal (streamed through the
// caches at low priority, so the 32 KB per tile does not evict the Q / G_O /
// K tiles the passes re-read)
constexpr int CPOL_NT = 2;
constexpr int DPP_ROW_MIRROR = 0x140, DPP_ROW_HALF_MIRROR = 0x141, DPP_XOR2 = 0x4E, DPP_XOR1 = 0xB1;

// One workgroup of 4 waves (one per SIMD, so each wave may hold up to 512
// registers) per (b, kv head g, key tile kt).  Wave w owns keys 32w .. +31 of
// the tile; their K, V fragments and G_K, G_V accumulators stay in registers.
// A visit consumes one unit of 128 query rows in four 32-row chunks: one
// 128-row query tile, or, with 64-row backward query tiles, two consecutive
// list items (chunks 0-1 from the first, 2-3 from the second).  The next unit
// is copied into the other LDS stage while the current one is consumed.
//
// The GS variant runs whenever the workspace carries G_S slots (a.gsinfo !=
// NULL); tiles whose slot index is past the capacity are computed without
// storing their G_S (their query tile's G_Q is recomputed by dq_kernel).
//
// RAGGED (stored variant, non-causal, n % 128 != 0 only): this instance serves
// only the last key tile, whose padded keys need masking; the main instance
// skips that tile, so its loop carries no per-element mask at all.  (Causal
// attention masks them through the diagonal, and without G_S stores their
// rows are simply never written.)
//
// ATOM (the fused single-pass variant, 128-row query tiles, no G_S stores):
// after each chunk's softmax the wave also forms its share of G_Q, the chunk's
// G_S (32 rows x the wave's 32 keys, transposed through a 2 KB LDS scratch)
// times the wave's 32 K rows, and adds it to the fp32 accumulator a.dqacc
// with global atomics.  G_S enters as bf16 hi + lo (two products), so no
// rounding compensation is needed.  The order of the atomic adds varies from
// run to run, so G_Q is not bit-reproducible in this variant.
template <int D, bool CAUSAL, bool GS, bool RAGGED, bool ATOM = false>
__global__ __launch_bounds__(256, 1) void dkdv_kernel(BwdArgs a) {
  static_assert(!RAGGED || (GS && !CAUSAL), "the ragged instance is the stored non-causal one");
  static_assert(!ATOM || (!GS && !RAGGED), "the atomic G_Q variant stores no G_S");
  constexpr int NT = 256;
  constexpr int NKS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 Qs0[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Gs0[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Qs1[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Gs1[TILE * D];
  __shared__ __attribute__((aligned(16))) float Ls0[TILE];  // row LSE, log2 units
  __shared__ __attribute__((aligned(16))) float Ds0[TILE];
  __shared__ __attribute__((aligned(16))) float Ls1[TILE];
  __shared__ __attribute__((aligned(16))) float Ds1[TILE];
  constexpr int ITAB = 2048;  // work-list window held in LDS
  __shared__ uint32_t itab[ITAB];
  __shared__ uint32_t stab[GS ? ITAB : 1];  // G_S slot of each windowed item
  __shared__ __attribute__((aligned(16))) bf16 Gt[ATOM ? 4 * 2048 : 8];  // per wave: G_S hi, lo [32 keys][32 rows]

  const int T = a.T, n = a.n;
  // this workgroup's chunk of the work: items [i0, i1) of key tile bgk's list
  // (long lists are split over several workgroups; see dk_plan_kernel)
  const int NK = a.B * a.Hk * T;
  int4 chunk;
  if constexpr (RAGGED) {
    // workgroup j * B*Hk + (b*Hk + g) takes chunk j of the ragged last key
    // tile of (b, g) (chunk-major: the first chunks of all (b, g), the long
    // ones, sit next to each other and spread over the XCDs); a list of
    // m <= G*Tq items makes at most ragged_chunks_max chunks
    const int nbg = a.B * a.Hk;
    const int k = (int)(blockIdx.x % nbg) * T + T - 1, j = blockIdx.x / nbg;
    const int32_t* items = a.dkplan + 4 + 8 * NK;
    const int m = items[k], CH = a.dkplan[3];
    if (j >= (m <= CH ? 1 : (m + CH - 1) / CH)) return;
    chunk = reinterpret_cast<const int4*>(a.dkplan + 4)[items[NK + k] + j];
  } else {
    if ((int)blockIdx.x >= a.dkplan[0]) return;  // past the plan's chunk count
    chunk = reinterpret_cast<const int4*>(a.dkplan + 4)[work_index(blockIdx.x)];
    // the ragged last key tile of the stored non-causal pass belongs to the
    // RAGGED instance
    if (GS && !CAUSAL && chunk.x % T == T - 1 && T * TILE != n) return;
  }
  const int kt = chunk.x % T;
  const int bg = chunk.x / T;
  const int g = bg % a.Hk, b = bg / a.Hk;
  const int G = a.H / a.Hk;
  const int i0 = chunk.y, i1 = chunk.z, pslot = chunk.w;
  (void)NK;

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
  // ATOM: the wave's 32 K rows as B operands of G_Q = G_S K: block db, 16-key
  // step s, lane (dim 32db + l32, h32) holds keys 16s + 8h32 + 0..7
  bf16x8 kT[ATOM ? NDB : 1][2];
  if constexpr (ATOM) {
    const uint16_t* kb = a.k + ((long)b * n) * kvstride + (long)g * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int kj = kt * TILE + kw * 32 + 16 * s2 + 8 * h32 + j;
          const uint16_t u = kj < n ? kb[(long)kj * kvstride + 32 * db + l32] : (uint16_t)0;
          kT[db][s2][j] = __builtin_bit_cast(bf16, u);
        }
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
  const int nitems = i1 - i0;
  auto fill_items = [&](int base) {  // items [base, base + ITAB) of the chunk, all threads
    const int f0 = i0 + base, f1 = min(i0 + base + ITAB, i1);  // in the flattened list
    int p0 = 0;
    for (int hh = 0; hh < G && p0 < f1; ++hh) {
      const long row = ((bh0 + hh) * T + kt);
      const int c = max(0, min(a.kcnt[row], a.Tq));  // as dk_plan_kernel counts it
      const int lo_p = max(f0, p0), hi_p = min(f1, p0 + c);
      for (int p = lo_p + tid; p < hi_p; p += NT) {
        itab[p - f0] = ((uint32_t)hh << 16) | a.kidx[row * a.Tq + (p - p0)];
        if constexpr (GS) stab[p - f0] = a.kslot[row * a.Tq + (p - p0)];
      }
      p0 += c;
    }
  };
  int ibase = 0;
  fill_items(0);
  __syncthreads();
  struct Item {
    int hh, qt;
    uint32_t slot;
  };
  auto item_at = [&](int p) -> Item {  // p in [ibase, ibase + ITAB)
    const uint32_t e = __builtin_amdgcn_readfirstlane(itab[p - ibase]);
    uint32_t s = 0;
    if constexpr (GS) s = __builtin_amdgcn_readfirstlane(stab[p - ibase]);
    return Item{(int)(e >> 16), (int)(e & 0xFFFFu), s};
  };
  // units of 128 stage rows: one item of 128 rows, or two of 64 (see above)
  const bool half = a.qrows == 64;
  const int QR = a.qrows, CPI = QR / 32;  // rows and 32-row chunks per item
  const int nunits = half ? (nitems + 1) / 2 : nitems;
  constexpr uint32_t NO_SLOT = 0xFFFFFFFFu;  // never below the capacity: stores dropped
  Item A_cur = item_at(0);
  bool vB_cur = half && nitems > 1;
  Item B_cur = vB_cur ? item_at(1) : A_cur;
  // Stored-G_S constants.  Slot layout (QR x 128 bf16): 1 KB blocks
  // ((kw * CPI + chunk of the item) * 2 + s), each the 64 lanes' 16-byte
  // operands sk[s] of that wave and chunk, lane (h32, l32) at position
  // 2 * l32 + h32.  Row sums (4 QR fp32 per slot): [kw][query row of the item],
  // the fp32 G_S summed over the wave's 32 keys; the G_Q pass subtracts the
  // sums of the bf16 values it reads to get the rounding residual's row sums.
  // After the butterfly in the unit's B phases, lane (bits b0..b5) holds the
  // sum for query row 16 b3 + 8 b2 + 4 b5 + 2 b1 + b4 of the chunk; odd lanes
  // hold a copy and store out of range (dropped).  The stores of chunk 3 (the
  // last chunk of its item) are issued after the next unit's barrier (or after
  // the last unit): issued at the end of a unit they would still be in flight
  // at the next unit's wait for its staged operands, which counts stores too.
  const uint32_t slot_elems = (uint32_t)QR * TILE, slot_sums = 4u * QR;
  auto gs_rsrc = [&](uint32_t slot) {
    const bool ok = GS && (long long)slot < a.gs_cap;
    return buffer_rsrc(GS && ok ? a.gs + (size_t)slot * slot_elems : nullptr, ok ? slot_elems * 2u : 0u);
  };
  auto gsl_rsrc = [&](uint32_t slot) {
    const bool ok = GS && (long long)slot < a.gs_cap;
    return buffer_rsrc(GS && ok ? a.gsl + (size_t)slot * slot_sums : nullptr, ok ? slot_sums * 4u : 0u);
  };

  const uint32_t gs_voff = (uint32_t)(2 * l32 + h32) * 16u;
  const uint32_t ls_q = 16 * ((lane >> 3) & 1) + 8 * ((lane >> 2) & 1) + 4 * (lane >> 5) + 2 * ((lane >> 1) & 1) +
                        ((lane >> 4) & 1);
  const bool sel3 = (lane >> 3) & 1, sel2 = (lane >> 2) & 1, sel1 = (lane >> 1) & 1;
  bf16x8 pk[2][2], sk[2][2];  // packed bf16 P and G_S operands [chunk parity][sub-step]
  float bw_def = 0.f;             // row sums of chunk 3 awaiting their store
  bool def_pending = false;       // chunk 3 of the previous unit not stored yet
  uint32_t def_slot = 0;
  // stores of chunk 3 (the last chunk of its item) in slot `slot` (its
  // operands are still in sk[1])
  auto store_late = [&](uint32_t slot) {
    const __amdgpu_buffer_rsrc_t r1 = gs_rsrc(slot), r2 = gsl_rsrc(slot);
    const int ci = CPI - 1;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sk[1][s2]), r1, gs_voff,
                                             ((kw * CPI + ci) * 2 + s2) * 1024, CPOL_NT);
    const uint32_t off = (lane & 1) ? 0x40000000u : (uint32_t)(kw * QR + 32 * ci + ls_q) * 4u;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, bw_def), r2, off, 0, CPOL_NT);
  };
  // stage S (a compile-time 0 or 1) holds unit u; the other stage receives u + 1
  auto visit = [&](int u, auto stage) {
    constexpr int S = decltype(stage)::value;
    const bf16* Qc = S ? Qs1 : Qs0;
    const bf16* Gc = S ? Gs1 : Gs0;
    const float* Lc = S ? Ls1 : Ls0;
    const float* Dc = S ? Ds1 : Ds0;
    bf16* Qn = S ? Qs0 : Qs1;
    bf16* Gn = S ? Gs0 : Gs1;
    float* Ln = S ? Ls0 : Ls1;
    float* Dn = S ? Ds0 : Ds1;
    wait_vmem();
    __syncthreads();  // unit u staged in (Qc, Gc, Lc, Dc); stage n is free
    const int jn = half ? 2 * (u + 1) : u + 1;  // first item of the next unit
    if (jn >= ibase + ITAB && jn < nitems) {     // slide the item window (ITAB is even)
      ibase += ITAB;
      fill_items(ibase);
      __syncthreads();
    }
    const bool vA_nxt = jn < nitems, vB_nxt = half && jn + 1 < nitems;
    const Item A_nxt = vA_nxt ? item_at(jn) : A_cur;
    const Item B_nxt = vB_nxt ? item_at(jn + 1) : A_nxt;
    // slots of the current unit's items (a missing second item stores nothing)
    const uint32_t slotA = A_cur.slot, slotB = half ? (vB_cur ? B_cur.slot : NO_SLOT) : A_cur.slot;
    if constexpr (GS) {
      if (def_pending) store_late(def_slot);
      def_pending = true;
      def_slot = slotB;
    }
    // Stage unit u + 1 into the free stage: its LSE and D words now, its Q and
    // G_O rows one copy instruction every few MFMAs in the first part of this
    // unit's stream (issued back to back they would stall the wave: the copy
    // pipeline holds few requests while rows stream in from HBM).  Without a
    // next item the copies read nothing and land zeros in the free stage.
    const QgSrc nsrcA = qg_src<D>(a, bh0 + A_nxt.hh, b, (int)(g * G + A_nxt.hh), A_nxt.qt, vA_nxt, 0);
    const QgSrc nsrcB =
        half ? qg_src<D>(a, bh0 + B_nxt.hh, b, (int)(g * G + B_nxt.hh), B_nxt.qt, vB_nxt, 64) : nsrcA;
    stage_ld(Ln, Dn, nsrcA, nsrcB, wave, lane);
    // first rows of the unit's items; chunk cs covers rows row0(cs) .. +31
    const int q0A = A_cur.qt * QR, q0B = B_cur.qt * QR;
    // the items' slots; a slot index past the capacity (lists that disagree)
    // gets empty ranges, so its stores are dropped
    const __amdgpu_buffer_rsrc_t gsrA = gs_rsrc(slotA), lsrA = gsl_rsrc(slotA);
    const __amdgpu_buffer_rsrc_t gsrB = gs_rsrc(slotB), lsrB = gsl_rsrc(slotB);
    // One tile: A(c) forms S and G_P of query chunk c (32 rows), B(c)
    // accumulates G_V and G_K from chunk c's P and G_S, in the order of
    // TileSched; chunk c's softmax (exp, mask, G_S) is spread over the MFMAs
    // between A(c) and B(c) so the VALU work hides under the matrix pipe.
    // Operands stream through a 4-slot ring fetched 3 MFMAs ahead;
    // a sched_barrier fence before each MFMA keeps that order.
    using SC = TileSched<2 * NKS, 4 * NDB>;
    constexpr int NSTEP = SC::total;
    constexpr int LB = 4 * NDB;
    // (a ring of 6 or 8 slots measured within 0.5% of this one: the pass is
    // bound by instruction issue, not by LDS latency)
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
    f32x16 sacc[2], gacc[2];  // S and G_P of the two chunks in flight
    f32x16 pv16[2], gs16[2];  // P and G_S formed from them (fresh registers, not the accumulators)
    f32x4 l4[4], d4[4];         // LSE (log2 units) and D of the chunk in softmax
    float bt[8], bu[4], bv[2], bw;  // row-sum butterfly of the chunk in its B phase
    bf16x8 ring[RING];
    static_for<0, AHEAD>([&](auto kc) { ring[decltype(kc)::value] = fetch(kc); });
    static_for<0, NSTEP>([&](auto kc) {
      constexpr int k = decltype(kc)::value, ph = SC::phase_of(k), st = k - SC::start(ph), c4 = SC::chunk(ph);
      if constexpr (k + AHEAD < NSTEP)
        ring[(k + AHEAD) % RING] = fetch(std::integral_constant<int, k + AHEAD>{});
      if constexpr (k % DSTEP == 0 && k / DSTEP < 2 * NI)
        stage_qg_part<D, NT, k / DSTEP>(Qn, Gn, nsrcA, nsrcB, dmo, wave);
      if constexpr (st == 0 && !SC::is_b(ph)) {
        sacc[c4 & 1] = f32x16{};
        gacc[c4 & 1] = f32x16{};
      }
      if constexpr (GS && SC::is_b(ph) && st == 0 && c4 < 3) {
        // chunk c4's bf16 G_S operands to its item's slot
        const int ci = half ? (c4 & 1) : c4;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sk[c4 & 1][s2]), c4 >= 2 ? gsrB : gsrA,
                                                 gs_voff, ((kw * CPI + ci) * 2 + s2) * 1024, CPOL_NT);
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
      if constexpr (GS && SC::is_b(ph)) {
        // Row sums of chunk c4's G_S over the wave's 32 keys (lanes): 16 groups
        // spread over the phase's LB MFMAs.  Groups 0-7: rows 2j, 2j+1 of the
        // lane, summed over lanes l, l ^ 16 by the 16-lane row swap (row parity
        // picks the row).  Groups 8-14: halving exchanges within 16-lane rows
        // (mirror, half mirror, xor 2), each lane keeping the half its lane bit
        // selects.  Group 15: the xor-1 sum and the store (chunks 0-2) or its
        // deferral (chunk 3).
        f32x16& gv = gs16[c4 & 1];
        static_for<0, 16>([&](auto gc) {
          constexpr int gi = decltype(gc)::value;
          if constexpr (gi * LB / 16 == st) {
            if constexpr (gi < 8) {
              float x = gv[2 * gi], y = gv[2 * gi + 1];
              swap16(x, y);
              bt[gi] = x + y;
            } else if constexpr (gi < 12) {
              constexpr int jj = gi - 8;
              const float snd = sel3 ? bt[jj] : bt[jj + 4];
              const float kp = sel3 ? bt[jj + 4] : bt[jj];
              bu[jj] = kp + dpp<DPP_ROW_MIRROR>(snd);
            } else if constexpr (gi < 14) {
              constexpr int jj = gi - 12;
              const float snd = sel2 ? bu[jj] : bu[jj + 2];
              const float kp = sel2 ? bu[jj + 2] : bu[jj];
              bv[jj] = kp + dpp<DPP_ROW_HALF_MIRROR>(snd);
            } else if constexpr (gi == 14) {
              const float snd = sel1 ? bv[0] : bv[1];
              const float kp = sel1 ? bv[1] : bv[0];
              bw = kp + dpp<DPP_XOR2>(snd);
            } else {
              bw += dpp<DPP_XOR1>(bw);
              if constexpr (c4 < 3) {
                const int ci = half ? (c4 & 1) : c4;
                const uint32_t off = (lane & 1) ? 0x40000000u : (uint32_t)(kw * QR + 32 * ci + ls_q) * 4u;
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, bw), c4 >= 2 ? lsrB : lsrA, off, 0,
                                                      CPOL_NT);
              } else {
                bw_def = bw;
              }
            }
          }
        });
      }
      static_for<0, 4>([&](auto cc) {
        constexpr int cs = decltype(cc)::value;
        f32x16& sv = sacc[cs & 1];
        f32x16& gv = gacc[cs & 1];
        if constexpr (SC::soft_begin(cs) == k) {
          if constexpr (CAUSAL) {
            // rows row0 .. row0+31 of this chunk drop the keys after them (score
            // -inf, so P = 0), and with a sliding window the keys <= row -
            // window; only chunks that reach such keys take this branch
            const int row0 = half ? (cs < 2 ? q0A : q0B) + 32 * (cs & 1) : q0A + 32 * cs;
            const bool diag = kt * TILE + TILE - 1 > row0;
            const bool wedge = a.window != 0 && kt * TILE <= row0 + 31 - a.window;
            if (diag || wedge) {
              // keep query offsets in [lim, limw): at or after the key, and before
              // key + window
              const int lim = key - (row0 + 4 * h32);
              const int limw = wedge ? lim + a.window : (1 << 30);
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int off = 8 * (r >> 2) + (r & 3);
                sv[r] = (off >= lim && off < limw) ? sv[r] : -INFINITY;
              }
            }
          } else if constexpr (RAGGED) {
            // padded keys of the ragged last tile: P = 0, so their G_S and its
            // rounding residuals are zero in the stored slot (their zero K rows
            // would otherwise give P = exp(-LSE))
#pragma unroll
            for (int r = 0; r < 16; ++r) sv[r] = key < n ? sv[r] : -INFINITY;
          }
        }
        static_for<0, 16>([&](auto ec) {
          // register r holds query q0 + 32cs + 4*h32 + 8(r/4) + r%4
          constexpr int r = decltype(ec)::value, j4 = r >> 2, t = r & 3;
          if constexpr (SC::elem_step(cs, r) == k) {
            const float pv = fast_exp2(fmaf(sv[r], c, -l4[j4][t]));
            pv16[cs & 1][r] = pv;
            gs16[cs & 1][r] = pv * (gv[r] - d4[j4][t]);
          }
        });
        if constexpr (SC::soft_end(cs) - 1 == k) {
          pk[cs & 1][0] = pack8(pv16[cs & 1], 0);
          pk[cs & 1][1] = pack8(pv16[cs & 1], 1);
          sk[cs & 1][0] = pack8(gs16[cs & 1], 0);
          sk[cs & 1][1] = pack8(gs16[cs & 1], 1);
          if constexpr (ATOM) {
            // G_S of this chunk as hi + lo bf16, row key l32 of the wave's scratch
            // (columns = the chunk's 32 query rows): register r is row 8(r/4) + 4h32 + r%4
            bf16* gt = Gt + kw * 2048;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              bf16x4 hi4, lo4;
#pragma unroll
              for (int t = 0; t < 4; ++t) {
                const float x = gs16[cs & 1][4 * g4 + t];
                hi4[t] = (bf16)x;
                lo4[t] = (bf16)(x - (float)hi4[t]);
              }
              *reinterpret_cast<bf16x4*>(gt + l32 * 32 + 8 * g4 + 4 * h32) = hi4;
              *reinterpret_cast<bf16x4*>(gt + 1024 + l32 * 32 + 8 * g4 + 4 * h32) = lo4;
            }
            // A operands (lane = query row l32, keys 16s + 8h32 + 0..7) by transpose reads:
            // 16-lane group gi covers rows 16(gi%2) .. +15 and keys 8(gi/2) + {0..3, 4..7}
            const int gi = lane >> 4, i16 = lane & 15;
            bf16x8 ah[2], al[2];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
              const int k0 = 16 * s2 + 8 * (gi >> 1) + (i16 >> 2);
              const int col = 16 * (gi & 1) + 4 * (i16 & 3);
#pragma unroll
              for (int part = 0; part < 2; ++part) {
                const bf16* base = gt + part * 1024;
                const bf16x4 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4*)(base + k0 * 32 + col));
                const bf16x4 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (__attribute__((address_space(3))) bf16x4*)(base + (k0 + 4) * 32 + col));
                (part ? al : ah)[s2] = cat8(x0, x1);
              }
            }
            // the chunk's rows of G_Q (query head of the unit's item), C layout
            // [row 8(r/4) + 4h32 + r%4][dim 32db + l32]: 32 consecutive floats per half wave
            const long row0 = ((bh0 + A_cur.hh) * (long)(a.T * TILE) + q0A + 32 * cs) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
              f32x16 acc = mfma32(ah[0], kT[db][0], f32x16{});
              acc = mfma32(ah[1], kT[db][1], acc);
              acc = mfma32(al[0], kT[db][0], acc);
              acc = mfma32(al[1], kT[db][1], acc);
              float* dst = a.dqacc + row0 + 32 * db + l32;
#pragma unroll
              for (int r = 0; r < 16; ++r)
                atomicAdd(dst + (long)(8 * (r >> 2) + 4 * h32 + (r & 3)) * D, acc[r]);
            }
          }
        }
      });
      // (no fence after the step: the next step's operand read and copy may be
      // scheduled among this step's VALU work; measured 2.4% faster than
      // fencing both sides)
    });
    A_cur = A_nxt;
    B_cur = B_nxt;
    vB_cur = vB_nxt;
  };

  {
    const QgSrc s0 = qg_src<D>(a, bh0 + A_cur.hh, b, (int)(g * G + A_cur.hh), A_cur.qt, nitems > 0, 0);
    const QgSrc s1 = half ? qg_src<D>(a, bh0 + B_cur.hh, b, (int)(g * G + B_cur.hh), B_cur.qt, vB_cur, 64) : s0;
    stage_ld(Ls0, Ds0, s0, s1, wave, lane);
    static_for<0, 2 * DmaOffsets<D, NT>::NI>(
        [&](auto ic) { stage_qg_part<D, NT, decltype(ic)::value>(Qs0, Gs0, s0, s1, dmo, wave); });
  }
  // pairs of units (stage 0, then stage 1), then the odd one out: no branch
  // between the two visits of an iteration, so the accumulators keep one
  // register assignment around the loop
  int j = 0;
  for (; j + 1 < nunits; j += 2) {
    visit(j, std::integral_constant<int, 0>{});
    visit(j + 1, std::integral_constant<int, 1>{});
  }
  if (j < nunits) visit(j, std::integral_constant<int, 0>{});
  if constexpr (GS) {
    if (def_pending) store_late(def_slot);
  }

  // epilogue.  C layout: [key = 8(r/4) + 4*h32 + r%4 of block kw][dim = 32db + l32].
  wait_vmem();
  if (pslot >= 0) {
    // a chunk of a split list: fp32 partial sums, reduced by dk_reduce_kernel
    float* pk_ = a.dkpart + (size_t)pslot * 2 * TILE * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = kw * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        pk_[kr * D + db * 32 + l32] = dk[db][r];
        pk_[(TILE + kr) * D + db * 32 + l32] = dv[db][r];
      }
    return;
  }
  // a whole list: stage as [key][dim] bf16 and store coalesced rows
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

}  // namespace backlite
