// Attention forward with per-(query row, key tile) log-sum-exp statistics.
//
// What it computes ("Introducing BackLite", "Backpropagation for attention";
// BackLite README, "How It Works", phase 1): S = scale * Q K^T with the causal
// rule j <= i when requested, P = row softmax(S), O = P V, the row LSE, and for
// every (row i, key tile kt) the LSE of row i restricted to tile kt.
//
// Method: single pass over key tiles with the online (running-max) softmax of
// the FlashAttention tutorial ("Online Softmax", "Flash Attention"), in base 2
// with scale*log2(e) folded into the exponent.  The tile statistic reuses the
// tile's rescaled row sum: LSE_tile = m_run + log2(sum_j 2^(s_j - m_run)), with
// m_run the running maximum after the tile, so it costs one log per row per
// tile.
//
// Work decomposition (gfx950): one workgroup of 8 waves (2 per SIMD) per
// (b, h, pair of query tiles); wave w owns 32 query rows.  The MFMA blocks run
// at raised wave priority, so the two waves of a SIMD settle into opposite
// phases and one's MFMAs overlap the other's softmax.  Each 128-key tile is
// consumed in two halves of 64 keys, which keeps S at 32 registers per lane and
// leaves room for LDS operand reads issued several MFMAs ahead.  S^T = K Q^T is
// formed with 32x32x16 bf16 MFMA (K from LDS as the A operand, the wave's Q fragment resident in registers as
// B), so each lane holds one query row and the row reductions stay in-lane
// plus one exchange between the two lane halves.  O^T += V^T P^T takes P^T
// straight from the S^T accumulators and V^T from the row-major V tile with the
// LDS transpose read.
#include <cfloat>

#include "bl_device.h"
#include "prof.h"

namespace backlite {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  uint16_t* olo;  // optional: bf16 rounding residual of O
  float* lse;
  float* tlse;
  double* tw;  // optional compact statistics: per tile pair and 64-row half, max over its rows of (tile LSE - row LSE)
  int B, n, H, Hk, T;
  int window;        // sliding window (causal only): key j visible to row i iff i - window < j; 0 = none
  float scale_log2;  // scale * log2(e)
};

// First key tile with a key inside the window of some row of query tile qt:
// the tile holding key qt*128 - window + 1 (0 without a window).
__device__ __forceinline__ int window_kt_lo(int qt, int window) {
  const int first = qt * TILE - window + 1;
  return (window == 0 || first <= 0) ? 0 : first / TILE;
}

// One workgroup of 8 waves per (b, h, pair of query tiles 2p, 2p+1); wave w owns
// rows 32(w%4) .. +31 of query tile 2p + w/4.  K and V tiles are each
// double-buffered in LDS.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_kernel(FwdArgs a) {
  constexpr int NT = 512;
  constexpr int NKS = D / 16;  // MFMA k-steps over the head dimension
  constexpr int NDB = D / 32;  // 32-wide blocks of the head dimension
  // V stages in the first 64 KiB, then the K stages: every operand read of
  // either V stage is one per-lane address plus an immediate offset (the
  // instruction's offset field reaches 64 KiB), and so is every read of either
  // K stage with the K base folded into the per-lane address, so the MFMA
  // blocks issue no address arithmetic.  (V takes the low half: it has two
  // transpose reads per MFMA, K one row read.)  Four separate arrays, not one:
  // the compiler then knows which stage an asynchronous copy writes, and does
  // not make the reads of the other stages wait for it.
  __shared__ __attribute__((aligned(16))) bf16 lds0_v[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 lds1_v[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 lds2_k[TILE * D];
  __shared__ __attribute__((aligned(16))) bf16 lds3_k[TILE * D];
  bf16* const Vs0 = lds0_v;
  bf16* const Vs1 = lds1_v;
  bf16* const Ks0 = lds2_k;
  bf16* const Ks1 = lds3_k;
  __shared__ float lse_s[2 * TILE];  // row LSEs of both query tiles (compact statistics)

  const int T = a.T;
  const int T2 = (T + 1) / 2;
  const int L = work_index(blockIdx.x);
  int p = L % T2;
  if (CAUSAL) p = T2 - 1 - p;  // heaviest query tiles first
  const int bh = L / T2;
  const int h = bh % a.H, b = bh / a.H;
  const int g = h / (a.H / a.Hk);
  const int n = a.n;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31, h32 = lane >> 5;
  const int qt = 2 * p + (wave >> 2);            // this wave's query tile
  const bool active = qt < T;                     // odd T: the last pair has one tile
  const int lrow = (wave & 3) * 32 + l32;         // row within the query tile
  const int qrow = qt * TILE + lrow;              // this lane's query row

  // Q fragment (B operand of S^T = K Q^T): dims 16ks + 8*h32 + 0..7 of row qrow
  bf16x8 qf[NKS];
  {
    const long qstride = (long)a.H * D;
    const uint16_t* qp = a.q + ((long)b * n) * qstride + (long)h * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (qrow < n) v = *reinterpret_cast<const u32x4*>(qp + (long)qrow * qstride + ks * 16 + h32 * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  // running max, in scaled log2 units.  It starts at the lowest finite float, not
  // -inf: a row that has seen only masked scores so far (possible with a sliding
  // window) then gets probabilities exp2(-inf) = 0 rather than exp2(-inf + inf).
  float m_run = -FLT_MAX;
  float l_run = 0.f;

  const long kvstride = (long)a.Hk * D;
  const uint16_t* kbase = a.k + ((long)b * n) * kvstride + (long)g * D;
  const uint16_t* vbase = a.v + ((long)b * n) * kvstride + (long)g * D;
  const int qt_hi = min(2 * p + 1, T - 1);
  const int nkt = CAUSAL ? qt_hi + 1 : T;        // key tiles the workgroup visits: kt0 .. nkt-1
  const int kt0 = CAUSAL ? window_kt_lo(2 * p, a.window) : 0;
  const int kt_lo = CAUSAL ? window_kt_lo(qt, a.window) : 0;  // this wave's first key tile
  // rows of this wave's tile see only keys > row - window: tiles that reach below
  // the last row's window edge are masked per element
  const int wedge_kt = a.window ? (qt * TILE + TILE - 1 - a.window) : -1;  // mask if key0 <= wedge_kt
  float* tl_row = nullptr;
  if (a.tlse) {
    const long pairs = CAUSAL ? (long)T * (T + 1) / 2 : (long)T * T;
    tl_row = a.tlse + (long)bh * pairs * TILE;
  }
  const float c = a.scale_log2;
  LdsOffsets<D> lo;
  lo.init(lane);
  DmaOffsets<D, NT> dmo;
  dmo.init(kvstride, tid);

  // Main loop: one barrier per key tile.  The copies of K and V of tile t+1 are
  // issued right after the barrier and have the whole visit of tile t to land;
  // the two waves of a SIMD run freely between barriers, so one's MFMAs overlap
  // the other's softmax.  Each tile is consumed in two halves of 64 keys
  // (scores, softmax, O update each), which keeps S at 32 registers and leaves
  // room for operand reads issued well ahead of their MFMAs.
  const int N = nkt - kt0;
  // The tile statistic is stored after the next barrier: the barrier waits for
  // all of the wave's memory operations, stores included, and a store issued
  // just before it would stall the wave for the whole write latency.
  float tl_val = 0.f;
  int tl_idx = 0;
  bool tl_pend = false;
  auto flush_tl = [&]() __attribute__((always_inline)) {
    if (tl_pend) {
      if (h32 == 0) tl_row[tl_idx] = tl_val;
      tl_pend = false;
    }
  };
  auto mine = [&](int t) __attribute__((always_inline)) -> bool {  // wave-uniform
    const int kt = kt0 + t;
    return active && !(CAUSAL && (kt > qt || kt < kt_lo));
  };
  // one K or V tile into LDS, asynchronously; the rows of a ragged last tile
  // past n arrive zero-filled (the copy's range ends at the last valid row), so
  // every tile takes the same path
  auto stage_one = [&](bf16* dst, const uint16_t* base, int key0) __attribute__((always_inline)) {
    const int nv = min(TILE, n - key0);
    const uint32_t range = (uint32_t)(((long)(nv - 1) * kvstride + D) * 2);
    dma_tile<D, NT>(dst, base + (long)key0 * kvstride, dmo, tid, range);
  };

  f32x16 s[2];      // S^T of one 64-key half: key blocks 2hh, 2hh+1
  bf16x8 pb[2][2];  // its probabilities, packed as B operands
  float ts = 0.f;   // the tile's row sum so far (relative to m_run)
  // S^T = K Q^T for key blocks 2hh, 2hh+1.  The K operands of k-step ks+1 are
  // read before the MFMAs of k-step ks.
  auto scores = [&](const bf16* Kc, int hh) __attribute__((always_inline)) {
    bf16x8 kr[2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) kr[0][j] = rd_row<D>(Kc, lo, 2 * hh + j, 0);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if (ks + 1 < NKS) {
#pragma unroll
        for (int j = 0; j < 2; ++j) kr[(ks + 1) & 1][j] = rd_row<D>(Kc, lo, 2 * hh + j, ks + 1);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) s[j] = mfma32(kr[ks & 1][j], qf[ks], ks ? s[j] : f32x16{});
    }
    // keep the reads three k-steps ahead of their MFMAs
    sched_interleave<6, NKS - 3, 2, 2, 6>();
  };
  // softmax of half hh of tile t: mask, running maximum (lazy rescale), the
  // probabilities, row sums; P^T packed into pb
  auto softmax = [&](int t, int hh) __attribute__((always_inline)) {
    const int key0 = (kt0 + t) * TILE + 64 * hh;
    // mask padded keys and, on the diagonal, keys after the row (and, with a
    // sliding window, keys at or below row - window)
    const bool need_mask = (key0 + 64 > n) || (CAUSAL && (key0 + 63 > qt * TILE || key0 <= wedge_kt));
    if (need_mask) {
      // register r of block j holds key key0 + 4*h32 + off, off = 32j + 8(r/4) + r%4;
      // it is kept iff lo_off < off <= hi_off
      const int hi_off = (CAUSAL ? min(qrow, n - 1) : n - 1) - (key0 + 4 * h32);
      const int lo_off = (CAUSAL && a.window) ? (qrow - a.window) - (key0 + 4 * h32) : -(1 << 30);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = j * 32 + 8 * (r >> 2) + (r & 3);
          s[j][r] = (off <= hi_off && off > lo_off) ? s[j][r] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[j][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // Lazy rescaling: the running maximum (and with it O, l and the tile's
    // partial sum) moves only when some row's maximum grows by more than 2^8;
    // otherwise the probabilities are taken against the old maximum (at most
    // 2^8, exact in fp32 and in the bf16 operand's relative precision).  Every
    // quantity is m + log2(sum 2^(s - m)) for whichever m is used, so the
    // result is the same softmax; the rescale of O is skipped in most halves.
    const float m_cand = fmaxf(m_run, mt * c);
    if (__any(m_cand - m_run > 8.f)) {
      const float alpha = fast_exp2(m_run - m_cand);
      l_run *= alpha;
      ts *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m_run = m_cand;
    }
    float hs = 0.f;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = fast_exp2(fmaf(s[j][r], c, -m_run));
        s[j][r] = pv;
        hs += pv;
      }
    hs += __shfl_xor(hs, 32);
    l_run += hs;
    ts += hs;
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int st = 0; st < 2; ++st) pb[j][st] = pack8(s[j], st);
  };
  // O^T += V^T P^T over key blocks 2hh, 2hh+1.  Step st of block kb covers keys
  // 32kb + 16st + 4*h32 + 0..3 and 32kb + 16st + 8 + 4*h32 + 0..3, i.e. C
  // registers 8st .. 8st+7.
  auto update = [&](const bf16* Vc, int hh) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = mfma32(rd_tr<D>(Vc, lo, 2 * hh + j, st, db), pb[j][st], oacc[db]);
    sched_interleave<12, 4 * NDB - 6, 1, 2, 6>();
  };
  auto visit = [&](int t, auto par) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par)::value;
    wait_vmem();
    __syncthreads();  // tile t has landed; every wave is done with tile t-1
    flush_tl();
    if (t + 1 < N) {
      stage_one(PAR ? Ks0 : Ks1, kbase, (kt0 + t + 1) * TILE);
      stage_one(PAR ? Vs0 : Vs1, vbase, (kt0 + t + 1) * TILE);
    }
    if (mine(t)) {
      ts = 0.f;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        // MFMA blocks at raised wave priority: a wave that reaches its MFMAs
        // issues them ahead of the other wave of the SIMD, which meanwhile
        // does its softmax, so the two drift into opposite phases
        __builtin_amdgcn_s_setprio(1);
        scores(PAR ? Ks1 : Ks0, hh);
        __builtin_amdgcn_s_setprio(0);
        softmax(t, hh);
        __builtin_amdgcn_s_setprio(1);
        update(PAR ? Vs1 : Vs0, hh);
        __builtin_amdgcn_s_setprio(0);
      }
      if (tl_row) {
        tl_val = (qrow < n) ? (m_run + __log2f(ts)) * LN2 : -INFINITY;
        tl_idx = (int)pair_index(qt, kt0 + t, T, CAUSAL) * TILE + lrow;
        tl_pend = true;
      }
    }
  };
  stage_one(Ks0, kbase, kt0 * TILE);
  stage_one(Vs0, vbase, kt0 * TILE);
  for (int t = 0; t < N; t += 2) {
    visit(t, std::integral_constant<int, 0>{});
    if (t + 1 < N) visit(t + 1, std::integral_constant<int, 1>{});
  }
  flush_tl();

  // epilogue: normalise, stage O (and its residual) through LDS as [row][dim],
  // store coalesced.  Query tile 2p + j uses Ks[j] / Vs[j].
  __syncthreads();
  bf16* Os = (wave >> 2) ? Ks1 : Ks0;
  bf16* Rs = (wave >> 2) ? Vs1 : Vs0;
  if (active) {
    const float inv = 1.f / l_run;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dim = db * 32 + 8 * j + 4 * h32;
        bf16x4 w4, r4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float f = oacc[db][4 * j + t] * inv;
          w4[t] = (bf16)f;
          r4[t] = (bf16)(f - (float)w4[t]);
        }
        *reinterpret_cast<bf16x4*>(Os + tile_off<D>(lrow, dim >> 3) + (dim & 7)) = w4;
        *reinterpret_cast<bf16x4*>(Rs + tile_off<D>(lrow, dim >> 3) + (dim & 7)) = r4;
      }
    const float lse_row = (m_run + __log2f(l_run)) * LN2;
    if (h32 == 0 && qrow < n) a.lse[(long)bh * n + qrow] = lse_row;
    if (h32 == 0) lse_s[(wave >> 2) * TILE + lrow] = lse_row;
  }
  __syncthreads();
  {
    constexpr int CH = D / 8;
    const long ostride = (long)a.H * D;
#pragma unroll
    for (int it = 0; it < 2 * TILE * CH / NT; ++it) {
      const int cc = tid + it * NT;
      const int r2 = cc / CH, ch = cc % CH;  // r2: row within the 256-row pair
      const int j = r2 / TILE, row = r2 % TILE;
      const int gi = (2 * p + j) * TILE + row;
      if (gi < n) {
        const long off = ((long)b * n + gi) * ostride + (long)h * D + ch * 8;
        *reinterpret_cast<u32x4*>(a.o + off) =
            *reinterpret_cast<const u32x4*>((j ? Ks1 : Ks0) + tile_off<D>(row, ch));
        if (a.olo)
          *reinterpret_cast<u32x4*>(a.olo + off) =
              *reinterpret_cast<const u32x4*>((j ? Vs1 : Vs0) + tile_off<D>(row, ch));
      }
    }
  }

  // Compact statistics: for each (query tile, key tile) the workgroup visited
  // and each 64-row half of the query tile, a = max over the half's valid rows
  // of (tile LSE - row LSE), in fp64 from the fp32 values just written (the
  // mask's own arithmetic, so the selection from a is the same as from the
  // per-row values, for 128-row query tiles as the larger of the two).  One
  // wave per tile pair: 64 lanes read the pair's 128 row values (512
  // contiguous bytes, still in L2).
  if (a.tw) {
    wait_vmem();      // this wave's tile-LSE stores have completed
    __syncthreads();  // ... and every other wave's, and lse_s is written
    const long pairs = CAUSAL ? (long)T * (T + 1) / 2 : (long)T * T;
    for (int j = 0; j < 2; ++j) {
      const int qj = 2 * p + j;
      if (qj >= T) break;
      const int lo = CAUSAL ? window_kt_lo(qj, a.window) : 0;
      const int hi = CAUSAL ? qj : T - 1;
      // rows lane and lane + 64 of the query tile; padded rows do not count
      const bool v0 = qj * TILE + lane < n, v1 = qj * TILE + lane + 64 < n;
      const double l0 = lse_s[j * TILE + lane], l1 = lse_s[j * TILE + lane + 64];
      constexpr int UN = 4;  // tile pairs per pass: their loads are issued together (8 spills at d=128)
      for (int kb = lo + wave; kb <= hi; kb += UN * (NT / 64)) {
        float x0[UN], x1[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int kt = kb + u * (NT / 64);
          x0[u] = x1[u] = -INFINITY;
          if (kt <= hi) {
            const float* src = a.tlse + ((long)bh * pairs + pair_index(qj, kt, T, CAUSAL)) * TILE;
            x0[u] = src[lane];
            x1[u] = src[lane + 64];
          }
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int kt = kb + u * (NT / 64);
          // one value per 64-row half: rows 0-63 (lane) and 64-127 (lane + 64)
          double m0 = v0 ? (double)x0[u] - l0 : -INFINITY;
          double m1 = v1 ? (double)x1[u] - l1 : -INFINITY;
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) {
            m0 = fmax(m0, __shfl_xor(m0, o));
            m1 = fmax(m1, __shfl_xor(m1, o));
          }
          if (lane == 0 && kt <= hi) {
            double* w2 = a.tw + 2 * ((long)bh * pairs + pair_index(qj, kt, T, CAUSAL));
            w2[0] = m0;
            w2[1] = m1;
          }
        }
      }
    }
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  const int total = a.B * a.H * ((a.T + 1) / 2);
  ProfScope ps(PK_FWD, st);
  hipLaunchKernelGGL((fwd_kernel<D, CAUSAL>), dim3(total), dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int n, int H,
                      int Hk, int d, float scale, int causal, int window, uint16_t* o, uint16_t* olo,
                      float* lse, float* tlse, double* tw, hipStream_t st) {
  // a window of n keys or more hides nothing beyond the causal rule
  FwdArgs a{q, k, v, o, olo, lse, tlse, tw, B, n, H, Hk, (n + TILE - 1) / TILE, window < n ? window : 0,
            scale * LOG2E};
  if (d == 64) return causal ? launch_fwd_t<64, true>(a, st) : launch_fwd_t<64, false>(a, st);
  return causal ? launch_fwd_t<128, true>(a, st) : launch_fwd_t<128, false>(a, st);
}

}  // namespace backlite
