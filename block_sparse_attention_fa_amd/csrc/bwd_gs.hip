// Stored-G_S backward path: the G_K/G_V pass keeps each kept tile's G_S (bf16)
// in a workspace slot, and the G_Q pass computes G_Q += scale * G_S K from the
// stored tiles ("Introducing BackLite", backward equations: G_Q = G_S K / sqrt(d)
// over the kept tiles) instead of rebuilding S, P, G_P and G_S.  One slot is
// 32 KB of G_S plus 2 KB of fp32 row sums; at the 32k-token video shape with
// ~79% of the tiles skipped that is ~19 GB of the GPU's 288 GB, and the G_Q
// pass becomes a stream over those bytes.
//
// Slots: the kept tiles of query tile (b, h, qt), in q-list order, take the
// slots qbase[b,h,qt] + i, where qbase is the exclusive prefix sum of qcnt
// over (b, h, qt).  kslot gives the same slot to each k-list entry, which is
// what the G_K/G_V pass (walking k-lists) needs.
//
// Which query tiles take the path is decided on the device: tile (b, h, qt) is
// stored iff qbase + qcnt <= the slot capacity, i.e. all of its kept tiles have
// a slot.  dqs_kernel serves those tiles and dq_kernel the others, each
// returning at once for a tile that is not its own; the G_K/G_V pass drops the
// stores of slots past the capacity.  A budget smaller than the kept tiles
// thus stores a prefix of the query tiles instead of giving up the path.
#include "bl_device.h"
#include "bwd_common.h"
#include "bwd_dkdv.h"  // CPOL_NT
#include "prof.h"

namespace backlite {

// qbase = exclusive prefix sum of qcnt over the B*H*T query tiles; gsinfo[0] =
// (kept tiles <= capacity), gsinfo[1] = kept tiles, gsinfo[2] = kept tiles
// with a slot (both clamped to int32).  One
// workgroup: each thread sums a contiguous run, the run totals are scanned in
// LDS, then each thread writes its run's prefix values.
__global__ __launch_bounds__(1024) void gs_scan_kernel(BwdArgs a) {
  __shared__ long long part[1024];
  const long N = (long)a.B * a.H * a.Tq;
  const int tid = threadIdx.x;
  const long per = (N + 1023) / 1024;
  const long s0 = min(N, (long)tid * per), s1 = min(N, s0 + per);
  long long sum = 0;
  for (long i = s0; i < s1; ++i) sum += max(0, min(a.qcnt[i], a.T));
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const long long v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  long long run = part[tid] - sum;
  for (long i = s0; i < s1; ++i) {
    a.qbase[i] = (uint32_t)run;
    run += max(0, min(a.qcnt[i], a.T));
  }
  if (tid == 1023) {
    const long long total = part[1023];
    a.gsinfo[1] = (int32_t)min(total, 0x7fffffffLL);
    a.gsinfo[0] = total <= a.gs_cap ? 1 : 0;
    a.gsinfo[2] = (int32_t)min(min(total, a.gs_cap), 0x7fffffffLL);
  }
}

// kslot[b,h,kt,p] = slot of the tile (qt, kt) listed at position p of key tile
// kt's k-list.  One workgroup per (b, h, qt): each kept kt of the q-list finds
// qt in kt's ascending k-list by binary search.
__global__ __launch_bounds__(256) void gs_slot_kernel(BwdArgs a) {
  const int T = a.T, Tq = a.Tq;
  const long bq = blockIdx.x;  // (b * H + h) * Tq + qt
  const int qt = (int)(bq % Tq);
  const long bh = bq / Tq;
  const int cnt = max(0, min(a.qcnt[bq], T));
  const uint32_t base = a.qbase[bq];
  for (int i = threadIdx.x; i < cnt; i += 256) {
    const int kt = a.qidx[bq * T + i];
    if (kt >= T) continue;
    const long row = bh * T + kt;
    const int kc = max(0, min(a.kcnt[row], Tq));
    const uint16_t* list = a.kidx + row * Tq;
    int lo = 0, hi = kc;  // first position whose entry is >= qt
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int)list[mid] < qt) lo = mid + 1;
      else hi = mid;
    }
    if (lo < kc && (int)list[lo] == qt) a.kslot[row * Tq + lo] = base + (uint32_t)i;
  }
}

// ---------------------------------------------------------------------------
// G_Q from stored G_S.  One workgroup of 4 waves per (b, h, query tile qt of
// QR rows).  QR = 128: wave w owns query rows 32w .. +31 and the whole head
// dimension.  QR = 64 (half-height backward tiles): wave w owns rows
// 32 (w % 2) .. +31 and half of the head dimension (columns 64 (w / 2) ..).
// Each wave accumulates G_Q^T (C layout [dim][query]) over the q-list:
// G_Q^T += K^T G_S^T, both operands read from LDS with the transpose read.  K
// rows are shared by the waves (three LDS stages, copied two tiles ahead).
// The G_S rows of each 32-row group (8 KB per tile, the HBM stream of this
// pass) are loaded into registers three tiles ahead and written to LDS at the
// start of their tile: with QR = 128 by the wave that owns them, into a buffer
// of its own; with QR = 64 half by each of the two waves that share the rows,
// into a buffer of the row group, double-buffered by tile parity (a wave may
// still read one tile's rows while its partner writes the next tile's).
//
// G_S operand, per 16-key step ks (keys 16ks + 4*h32 + {0..3, 8..11}, the same
// order as the K operand): the slot's fragment-order block of wave kw =
// ks / 2, 16-byte position 2*key32 + hq (hq: which 4-row group of the 8 rows
// the G_K/G_V lane packed), 8-byte half v.  A transpose read by lane i of a
// 16-lane group supplies the address of key row k0 + i/4, query columns
// n0 + 4(i%4) .. +3, i.e. position 2*key32 + (i & 1) and half (i >> 1) & 1.
// Blocks of the second 16-row half (s = 1) are kept with 16-byte positions
// XOR 8 (a 128-byte shift), so the four groups of one read cover all banks.
// ---------------------------------------------------------------------------
template <int D, int NT, int I>
__device__ __forceinline__ void stage_k_part(bf16* Kd, const __amdgpu_buffer_rsrc_t& rs,
                                             const DmaOffsets<D, NT>& dmo, int wave) {
  lds_byte* dst = lds_ptr(Kd + ((I * (NT / 64) + wave) * 64) * 8);
  load_lds16(rs, dst, dmo.off[I]);
}

// lanes 0-31 and 32-63 of x added: the sum in every lane
__device__ __forceinline__ float add_halves(float x) {
  const uint64_t u = __builtin_bit_cast(
      uint64_t, __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                 false, false));
  return __builtin_bit_cast(float, (uint32_t)u) + __builtin_bit_cast(float, (uint32_t)(u >> 32));
}

template <int D, int QR>
__global__ __launch_bounds__(256, 1) void dqs_kernel(BwdArgs a) {
  constexpr int NT = 256;
  constexpr int NDB = QR == TILE ? D / 32 : D / 64;  // 32-wide head-dimension blocks per wave
  constexpr int NKS = TILE / 16;  // 16-key contraction steps per key tile
  constexpr int GW = 8 * 1024;    // G_S bytes of one 32-row group per tile
  constexpr int NI = DmaOffsets<D, NT>::NI;
  constexpr int NST = 3;          // K stages (two tiles ahead) and G_S register sets (three ahead)
  // vector-memory operations one visit issues per wave: NI K copies, 2 row-sum
  // words, 1 key-mean word, NGS G_S loads (8 blocks of 1 KB per 32-row group,
  // shared by two waves when QR = 64)
  constexpr int NSMALL = 3, NGS = QR == TILE ? 8 : 4, PER_VISIT = NI + NSMALL + NGS;
  // one variable per stage: the compiler then knows a copy into one stage
  // does not alias reads of another and waits for it only where it is read
  __shared__ __attribute__((aligned(16))) bf16 Ks0[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Ks1[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 Ks2[TILE * D];
  __shared__ __attribute__((aligned(16))) char Gw[4 * GW];
  __shared__ __attribute__((aligned(16))) float Lw0[4 * TILE];  // per wave: [key quarter][32 rows]
  __shared__ __attribute__((aligned(16))) float Lw1[4 * TILE];
  __shared__ __attribute__((aligned(16))) float Lw2[4 * TILE];
  __shared__ __attribute__((aligned(16))) float Kb0[D];
  __shared__ __attribute__((aligned(16))) float Kb1[D];
  __shared__ __attribute__((aligned(16))) float Kb2[D];
  __shared__ uint16_t itab[MAX_TILES];

  const int T = a.T, n = a.n, Tq = a.Tq;
  const int L = work_index(blockIdx.x);
  const int qt = L % Tq;
  const int bh = L / Tq;
  const int h = bh % a.H, b = bh / a.H;
  const int g = h / (a.H / a.Hk);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h32 = lane >> 5;
  const int rw = QR == TILE ? wave : (wave & 1);       // 32-row group of the wave
  const int dh = QR == TILE ? 0 : (wave >> 1);         // head-dimension half (QR = 64)
  const int lrow = rw * 32 + l32;
  const long qstride = (long)a.H * D;
  const long kvstride = (long)a.Hk * D;
  const uint16_t* kbase = a.k + ((long)b * n) * kvstride + (long)g * D;
  const float* kbar = a.kbar + (long)(b * a.Hk + g) * T * D;
  const long bq = (long)bh * Tq + qt;
  const int cnt = max(0, min(a.qcnt[bq], T));
  const uint32_t sbase = a.qbase[bq];
  // only query tiles whose kept tiles all have a slot; dq_kernel recomputes the rest
  if ((long long)sbase + cnt > a.gs_cap) return;
  {
    const uint16_t* list = a.qidx + bq * T;
    for (int i = tid; i < cnt; i += NT) itab[i] = list[i];
  }
  LdsOffsets<D> lo;
  lo.init(lane, dh * NDB);
  DmaOffsets<D, NT> dmo;
  dmo.init(kvstride, tid);
  const int i16 = lane & 15, sh = (lane >> 4) & 1;
  const uint32_t goff = (uint32_t)(sh * 1024 + 128 * (h32 ^ sh) + 32 * (i16 >> 2) + 16 * (i16 & 1) +
                                   8 * ((i16 >> 1) & 1));
  // this wave's G_S buffer (QR = 128), or its row group's pair (QR = 64, by parity)
  char* gw = QR == TILE ? Gw + wave * GW : Gw + rw * GW;
  f32x16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = f32x16{};
  __syncthreads();

  // K rows, row sums and key-mean words of list item i into K stage st; past
  // the list, zero-range sources (nothing is read, zeros land)
  auto k_of = [&](auto st) -> bf16* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? Ks0 : S == 1 ? Ks1 : Ks2;
  };
  auto l_of = [&](auto st) -> float* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? Lw0 : S == 1 ? Lw1 : Lw2;
  };
  auto b_of = [&](auto st) -> float* {
    constexpr int S = decltype(st)::value;
    return S == 0 ? Kb0 : S == 1 ? Kb1 : Kb2;
  };
  // kt_raw: the list entry itab[i], read a visit ahead so no LDS wait sits
  // here.  Issues the row-sum and key-mean copies and returns the resource of
  // item i's K rows.
  auto stage_small = [&](int i, int kt_raw, auto st) -> __amdgpu_buffer_rsrc_t {
    int kt = i < cnt ? (int)__builtin_amdgcn_readfirstlane(kt_raw) : 0;
    const bool valid = i < cnt && kt < T;  // entries past the last tile read as empty
    if (!valid) kt = 0;
    const int key0 = kt * TILE;
    const uint32_t rows = valid ? (uint32_t)min(TILE, n - key0) : 0u;
    const size_t slot = (size_t)sbase + (size_t)i;
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kbase + (long)key0 * kvstride, rows * (uint32_t)kvstride * 2u);
    const __amdgpu_buffer_rsrc_t rl = buffer_rsrc(a.gsl + slot * (4 * QR), valid ? 4u * QR * 4u : 0u);
    // key mean: D/64 copy instructions; wave w issues number w % (D/64), so
    // waves beyond the first D/64 repeat a copy (same words to the same place)
    // and every wave issues one
    const int kb_part = wave % (D / 64);
    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(kbar + (long)kt * D, valid ? (uint32_t)D * 4u : 0u);
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int e = lane + 64 * it;
      load_lds4(rl, lds_ptr(l_of(st) + wave * TILE + 64 * it),
                      (uint32_t)((e >> 5) * QR + 32 * rw + (e & 31)) * 4u);
    }
    load_lds4(rb, lds_ptr(b_of(st) + 64 * kb_part), (uint32_t)(64 * kb_part + lane) * 4u);
    return rk;
  };
  auto stage_k = [&](int i, int kt_raw, auto st) {
    const __amdgpu_buffer_rsrc_t rk = stage_small(i, kt_raw, st);
    static_for<0, NI>([&](auto ic) { stage_k_part<D, NT, decltype(ic)::value>(k_of(st), rk, dmo, wave); });
  };
  // the wave's NGS blocks of item i's G_S into registers: block ib = (kw, s) of
  // its row group (kw = 2 dh + ib / 2 when QR = 64), lane l takes the 16 bytes
  // at position l ^ 8s
  u32x4 gr[NST][NGS];
  auto gs_rsrc = [&](int i) {
    const size_t slot = (size_t)sbase + (size_t)i;
    return buffer_rsrc(a.gs + slot * (QR * TILE), i < cnt ? QR * TILE * 2u : 0u);
  };
  auto load_gs_block = [&](u32x4& r, const __amdgpu_buffer_rsrc_t& rs, int ib) {
    const int kw = (QR == TILE ? 0 : 2 * dh) + (ib >> 1), s2 = ib & 1;
    r = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((lane ^ (8 * s2)) * 16),
                                                                       ((kw * (QR / 32) + rw) * 2 + s2) * 1024,
                                                                       CPOL_NT));
  };
  auto load_gs = [&](u32x4 (&r)[NGS], int i) {
    const __amdgpu_buffer_rsrc_t rs = gs_rsrc(i);
#pragma unroll
    for (int ib = 0; ib < NGS; ++ib) load_gs_block(r[ib], rs, ib);
  };

  // prologue, in the order the steady state keeps: G_S 0, K 0, G_S 1, K 1, G_S 2
  load_gs(gr[0], 0);
  stage_k(0, itab[0], std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  load_gs(gr[1], 1);
  stage_k(1, itab[1], std::integral_constant<int, 1>{});
  __builtin_amdgcn_sched_barrier(0);
  load_gs(gr[2], 2);
  int kt_ahead = itab[2];  // list entry of the next K stage (entries past cnt are never used)

  const bf16x2 one2 = {(bf16)1.f, (bf16)1.f};
  // rounding-compensation operands of the current group of NST items, item j
  // in contraction slot j % NST (see the end of visit); zero elsewhere
  bf16x8 cal[NDB], cbl = {};
#pragma unroll
  for (int db = 0; db < NDB; ++db) cal[db] = bf16x8{};
  auto flush_comp = [&]() {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dq[db] = mfma32(cal[db], cbl, dq[db]);
      cal[db] = bf16x8{};
    }
    cbl = bf16x8{};
  };
  // item j in K stage and G_S register set S = j % 3
  auto visit = [&](int j, auto stage) {
    constexpr int S = decltype(stage)::value;
    const std::integral_constant<int, S> cur;
    const bf16* Kc = k_of(cur);
    const float* Lc = l_of(cur);
    const float* Bc = b_of(cur);
    // item j's K, sums and G_S have landed once at most the operations of the
    // two later visits' worth (G_S j+1, K j+1, G_S j+2) are outstanding
    constexpr int VM = NGS + PER_VISIT;
    static_assert(VM < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((VM & 0xF) | ((VM >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    char* gb0 = QR == TILE ? gw : gw + (j & 1) * (2 * GW);  // this tile's G_S buffer
#pragma unroll
    for (int ib = 0; ib < NGS; ++ib)
      *reinterpret_cast<u32x4*>(gb0 + ((QR == TILE ? 0 : 4 * dh) + ib) * 1024 + lane * 16) = gr[S][ib];
    // Barrier without the workgroup fence of __syncthreads: the fence would
    // make every wave finish all its pending LDS copies here (item j + 1's K
    // too), which would leave K only one tile of lead.  What the barrier must
    // order is covered explicitly: item j's copies are complete in every wave
    // (the vmcnt wait above), and every wave's LDS reads of item j - 1, whose
    // stage the copies issued next overwrite, have returned (lgkmcnt(0)).
    // The memory clobber keeps the compiler from moving LDS accesses across.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
    float hsum = 0.f;  // this row's sum of the bf16 G_S operands over the lane's 64 keys
    if constexpr (QR == TILE) {
      // Item j + 2's K copies and item j + 3's G_S loads go out a few per 16-key
      // step between the MFMAs (the K copies over the first half of the steps,
      // the G_S loads over the second: the order the wait above counts).
      // Issued back to back they stall the wave until the copy pipeline takes
      // them, with nothing else to issue meanwhile.
      constexpr std::integral_constant<int, (S + 2) % NST> nxt;
      const __amdgpu_buffer_rsrc_t rk = stage_small(j + 2, kt_ahead, nxt);
      kt_ahead = itab[min(j + 3, MAX_TILES - 1)];
      const __amdgpu_buffer_rsrc_t rg = gs_rsrc(j + 3);  // into the register set just written to LDS
      // operands of one 16-key step (the G_S fragment, the K fragments of the
      // wave's head-dimension blocks), read one step ahead
      auto fetch = [&](auto kc, bf16x8& gop, bf16x8 (&kop)[NDB]) {
        constexpr int ks = decltype(kc)::value;
        const char* gb = gb0 + (ks >> 1) * 2048 + (ks & 1) * 512 + goff;
        const bf16x4 g0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(gb));
        const bf16x4 g1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(gb + 256));
        gop = cat8(g0, g1);
#pragma unroll
        for (int db = 0; db < NDB; ++db) kop[db] = rd_tr<D>(Kc, lo, ks >> 1, ks & 1, db);
      };
      constexpr int HALF = NKS / 2;
      bf16x8 gop[2], kop[2][NDB];
      fetch(std::integral_constant<int, 0>{}, gop[0], kop[0]);
      static_for<0, NKS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        if constexpr (ks + 1 < NKS) fetch(std::integral_constant<int, ks + 1>{}, gop[(ks + 1) & 1], kop[(ks + 1) & 1]);
        static_for<0, NI>([&](auto ic) {  // K copy c in step c HALF / NI
          constexpr int c = decltype(ic)::value;
          if constexpr (c * HALF / NI == ks) stage_k_part<D, NT, c>(k_of(nxt), rk, dmo, wave);
        });
        static_for<0, NGS>([&](auto ic) {  // G_S block ib in step HALF + ib HALF / NGS
          constexpr int ib = decltype(ic)::value;
          if constexpr (HALF + ib * HALF / NGS == ks) load_gs_block(gr[S][ib], rg, ib);
        });
        const bf16x8 bop = gop[ks & 1];
#pragma unroll
        for (int db = 0; db < NDB; ++db) dq[db] = mfma32(kop[ks & 1][db], bop, dq[db]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x2 pr = {bop[2 * u], bop[2 * u + 1]};
          hsum = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, hsum, false);
        }
        __builtin_amdgcn_sched_barrier(0);
      });
    } else {
      // 64-row tiles (two waves per row group): the copies issued together
      // after the barrier and the compiler's own schedule of the stream
      // measured faster than the spread form (4.5 against 6.2 ms at 32k)
      stage_k(j + 2, kt_ahead, std::integral_constant<int, (S + 2) % NST>{});
      kt_ahead = itab[min(j + 3, MAX_TILES - 1)];
      __builtin_amdgcn_sched_barrier(0);
      load_gs(gr[S], j + 3);  // the register set just written to LDS takes item j + 3
      static_for<0, NKS>([&](auto kc) {
        constexpr int ks = decltype(kc)::value;
        const char* gb = gb0 + (ks >> 1) * 2048 + (ks & 1) * 512 + goff;
        const bf16x4 g0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(gb));
        const bf16x4 g1 =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)(gb + 256));
        const bf16x8 bop = cat8(g0, g1);
#pragma unroll
        for (int db = 0; db < NDB; ++db) dq[db] = mfma32(rd_tr<D>(Kc, lo, ks >> 1, ks & 1, db), bop, dq[db]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x2 pr = {bop[2 * u], bop[2 * u + 1]};
          hsum = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, hsum, false);
        }
      });
    }
    // Rounding compensation: the stored G_S is bf16.  Its rounding residual lo
    // contributes sum_j lo_ij K_j, whose dominant part when the tile's keys
    // share a large common vector is (sum_j lo_ij) * kbar (rows of G_S nearly
    // sum to zero, so that vector would otherwise multiply the rounding
    // error).  sum_j lo_ij = (fp32 row sum of G_S, from the G_K/G_V pass) -
    // (sum of the bf16 operands).  Each item's rank-1 term goes into
    // contraction slot S of the group's operands (lanes 0-31; every lane
    // loads and selects, so no branch splits the wave), and one MFMA per
    // 32-dim block adds the NST items' terms at the end of the group.
    {
      hsum = add_halves(hsum);
      const float* lw = Lc + wave * TILE + l32;
      const float ls = ((lw[0] + lw[32]) + (lw[64] + lw[96])) - hsum;
      cbl[S] = (bf16)(h32 == 0 ? ls : 0.f);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const float kb = Bc[(dh * NDB + db) * 32 + l32];
        cal[db][S] = (bf16)(h32 == 0 ? kb : 0.f);
      }
      if constexpr (S == NST - 1) flush_comp();
    }
  };
  int j = 0;
  for (; j + 2 < cnt; j += 3) {
    visit(j, std::integral_constant<int, 0>{});
    visit(j + 1, std::integral_constant<int, 1>{});
    visit(j + 2, std::integral_constant<int, 2>{});
  }
  if (j < cnt) visit(j, std::integral_constant<int, 0>{});
  if (j + 1 < cnt) visit(j + 1, std::integral_constant<int, 1>{});
  flush_comp();  // the tail's items (zero operands when there is no tail)

  // epilogue: dq C layout is [dim = 32db + 8(r/4) + 4*h32 + r%4][query l32]
  // (db counted from the wave's head-dimension slice)
  wait_vmem();
  __syncthreads();
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int dim = (dh * NDB + db) * 32 + 8 * jj + 4 * h32;
      bf16x4 w4 = {(bf16)(dq[db][4 * jj] * a.scale), (bf16)(dq[db][4 * jj + 1] * a.scale),
                   (bf16)(dq[db][4 * jj + 2] * a.scale), (bf16)(dq[db][4 * jj + 3] * a.scale)};
      *reinterpret_cast<bf16x4*>(Ks0 + tile_off<D>(lrow, dim >> 3) + (dim & 7)) = w4;
    }
  __syncthreads();
  {
    constexpr int CH = D / 8;
    uint16_t* op = a.dq + ((long)b * n + (long)qt * QR) * qstride + (long)h * D;
#pragma unroll
    for (int it = 0; it < QR * CH / NT; ++it) {
      const int cc = tid + it * NT;
      const int row = cc / CH, ch = cc % CH;
      if (qt * QR + row < n)
        *reinterpret_cast<u32x4*>(op + (long)row * qstride + ch * 8) =
            *reinterpret_cast<const u32x4*>(Ks0 + tile_off<D>(row, ch));
    }
  }
}

hipError_t launch_gs_slots(const BwdArgs& a, hipStream_t st) {
  ProfScope ps(PK_GS_SLOTS, st);
  hipLaunchKernelGGL(gs_scan_kernel, dim3(1), dim3(1024), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gs_slot_kernel, dim3(a.B * a.H * a.Tq), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_dq_gs(const BwdArgs& a, int d, hipStream_t st) {
  ProfScope ps(PK_DQ, st);
  const dim3 grid(a.B * a.H * a.Tq), block(256);
  if (a.qrows == TILE) {
    if (d == 64) hipLaunchKernelGGL((dqs_kernel<64, TILE>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((dqs_kernel<128, TILE>), grid, block, 0, st, a);
  } else {
    if (d == 64) hipLaunchKernelGGL((dqs_kernel<64, 64>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((dqs_kernel<128, 64>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace backlite
