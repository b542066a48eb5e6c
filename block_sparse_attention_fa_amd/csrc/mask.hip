// Mask from tile statistics: tile weights -> smallest-first cumulative cut ->
// keep bitmap and compacted work lists.
//
// What it computes (BackLite README, "How It Works", phase 2, and "Overview";
// "Introducing BackLite", "Using Sparsity"): for each query tile, the tile
// probability p_tile = exp(LSE_tile - LSE_row) of each candidate key tile,
// aggregated over the query tile's rows by the maximum; the candidates with the
// smallest weights are skipped while their cumulative weight stays below
// negl_prob.
//
// select_kernel: one workgroup per (b, h, query tile qt) of 128 or 64 rows (the
// backward's query tiles may be half the statistics' 128-row blocks: the README
// forms the mask "for each backward tile pair").
//   1. a[kt] = max_r (tile_lse[qt,kt,r] - lse_row[r]) in fp64: groups of 32
//      (or 16) lanes each take one key tile at a time, a lane reads 4 rows (one
//      16-byte load per lane, 512 or 256 contiguous bytes per tile).
//   2. bitonic sort of (a, kt) in LDS, ascending, ties by kt.
//   3. all threads form the weights exp(a) in fp64; one lane then walks the
//      sorted list adding them left to right and stops at the first running
//      sum >= negl_prob; everything before is skipped.
//   4. keep row and the ascending q-list (block-wide prefix count).
// transpose_kernel: one workgroup per (b, h, kt) turns column kt of the keep
// bitmap into the ascending k-list.
#include "bl_device.h"
#include "prof.h"

namespace backlite {

constexpr int MASK_NT = 256;
constexpr int MAX_T = 1024;   // key tiles: n <= 131072
constexpr int MAX_TQ = 2048;  // query tiles of 64 rows

// Exclusive prefix sum of one int per thread over the 256-thread block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* red, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < MASK_NT / 64; ++w) {
    const int r = red[w];
    if (w < wave) base += r;
    total += r;
  }
  __syncthreads();
  return base + x - v;
}

struct MaskArgs {
  const float* tlse;
  const float* lse;
  uint8_t* keep;
  int32_t* qcnt;
  uint16_t* qidx;
  int32_t* kcnt;
  uint16_t* kidx;
  unsigned long long* stats;
  int B, H, n, T, causal;  // T: key tiles (128 keys; also the statistics' row blocks)
  int window;  // sliding window (causal only), 0 = none
  const double* tw;  // compact statistics [B, H, pairs, 2] (log-weight per tile pair and 64-row half), or NULL
  double negl;
  int Tq, qrows;  // query tiles of the mask and their rows (64 or 128)
};

__global__ __launch_bounds__(MASK_NT) void mask_select_kernel(MaskArgs a) {
  __shared__ double sa[MAX_T];
  __shared__ int sk[MAX_T];
  __shared__ uint8_t flag[MAX_T];
  __shared__ int red[MASK_NT / 64];
  __shared__ int s_skip;

  const int T = a.T, Tq = a.Tq, QR = a.qrows;
  const int L = work_index(blockIdx.x);
  const int qt = L % Tq;
  const int bh = L / Tq;
  const int tid = threadIdx.x;
  // rows q_first .. q_last of this query tile lie in row block p of the
  // statistics, at offset ro (0, or 64 for the second half of a 64-row split)
  const int q_first = qt * QR, q_last = min(a.n, q_first + QR) - 1;
  const int p = q_first / TILE, ro = q_first % TILE;
  // candidates are kt = kt0 .. kt0+nc-1: causal tiles whose first key is at or
  // before the last row and, with a sliding window, from the tile holding key
  // q_first - window + 1
  const int first = q_first - a.window + 1;
  const int kt0 = (a.window == 0 || first <= 0) ? 0 : first / TILE;
  const int nc = (a.causal ? q_last / TILE : T - 1) - kt0 + 1;
  int P2 = 1;
  while (P2 < nc) P2 <<= 1;

  for (int i = tid; i < T; i += MASK_NT) flag[i] = 0;
  __syncthreads();  // flags are set below by other threads than the one that cleared them (kt0 > 0)

  if (a.tw != nullptr || a.tlse != nullptr) {
   if (a.tw != nullptr) {
    // ---- 1. log-weights, already reduced over each 64-row half by the forward
    const long pairs = a.causal ? (long)T * (T + 1) / 2 : (long)T * T;
    const double* tw = a.tw + (long)bh * pairs * 2;
    for (int i = tid; i < nc; i += MASK_NT) {
      const double* w2 = tw + 2 * pair_index(p, kt0 + i, T, a.causal);
      sa[i] = QR == TILE ? fmax(w2[0], w2[1]) : w2[ro / 64];
      sk[i] = kt0 + i;
    }
   } else {
    // ---- 1. log-weights: groups of QR/4 lanes each take one key tile at a
    // time, a lane reading 4 rows (one 16-byte load)
    const int GL = QR / 4, NG = MASK_NT / GL;
    const int grp = tid / GL, gl = tid % GL;
    const int r0 = q_first + gl * 4;
    double ls[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) ls[u] = (r0 + u < a.n) ? (double)a.lse[(long)bh * a.n + r0 + u] : 0.0;
    const long pairs = a.causal ? (long)T * (T + 1) / 2 : (long)T * T;
    const float* tl = a.tlse + (long)bh * pairs * TILE + ro;
    // four key tiles per group and pass: their loads are issued together, so
    // each lane has four 16-byte loads in flight instead of one
    constexpr int UN = 4;
    for (int kb = grp; kb < nc; kb += NG * UN) {
      f32x4 v[UN];
#pragma unroll
      for (int x = 0; x < UN; ++x) {
        const int kt = kb + x * NG;
        v[x] = kt < nc ? *reinterpret_cast<const f32x4*>(tl + pair_index(p, kt0 + kt, T, a.causal) * TILE + gl * 4)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int x = 0; x < UN; ++x) {
        const int kt = kb + x * NG;
        double m = -INFINITY;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (r0 + u < a.n) m = fmax(m, (double)v[x][u] - ls[u]);
        for (int o = GL / 2; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o, GL));
        if (gl == 0 && kt < nc) {
          sa[kt] = m;
          sk[kt] = kt0 + kt;
        }
      }
    }
   }
    for (int i = nc + tid; i < P2; i += MASK_NT) {
      sa[i] = INFINITY;
      sk[i] = 0x7fffffff;
    }
    __syncthreads();
    // ---- 2. bitonic sort ascending by (a, kt)
    for (int kk = 2; kk <= P2; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < P2 / 2; i += MASK_NT) {
          const int lo = 2 * j * (i / j) + (i % j);
          const int hi = lo + j;
          const bool up = ((lo & kk) == 0);
          const double alo = sa[lo], ahi = sa[hi];
          const int klo = sk[lo], khi = sk[hi];
          const bool gt = (alo > ahi) || (alo == ahi && klo > khi);
          if (gt == up) {
            sa[lo] = ahi;
            sa[hi] = alo;
            sk[lo] = khi;
            sk[hi] = klo;
          }
        }
        __syncthreads();
      }
    }
    // ---- 3. sequential fp64 prefix, stop at the first sum >= negl_prob.  The
    // weights exp(a) are formed by all threads first (in place; the sorted
    // log-weights are not needed afterwards), so the one walking lane only
    // adds, in the same left-to-right order.
    for (int i = tid; i < nc; i += MASK_NT) sa[i] = exp(sa[i]);
    __syncthreads();
    if (tid == 0) {
      double acc = 0.0;
      int r = 0;
      for (; r < nc; ++r) {
        acc += sa[r];
        if (!(acc < a.negl)) break;
      }
      s_skip = r;
    }
    __syncthreads();
    const int skip = s_skip;
    for (int r = skip + tid; r < nc; r += MASK_NT) flag[sk[r]] = 1;
  } else {
    for (int i = tid; i < nc; i += MASK_NT) flag[kt0 + i] = 1;
  }
  __syncthreads();

  // ---- 4. keep row + ascending q-list
  uint8_t* keep_row = a.keep + ((long)bh * Tq + qt) * T;
  for (int i = tid; i < T; i += MASK_NT) keep_row[i] = flag[i];
  constexpr int PER = MAX_T / MASK_NT;  // 4 consecutive kt per thread
  int f[PER], cnt = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int kt = tid * PER + u;
    f[u] = (kt < T) ? flag[kt] : 0;
    cnt += f[u];
  }
  int tot;
  int pos = block_exclusive_scan(cnt, red, tot);
  uint16_t* qrow = a.qidx + ((long)bh * Tq + qt) * T;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (f[u]) qrow[pos++] = (uint16_t)(tid * PER + u);
  if (tid == 0) {
    a.qcnt[(long)bh * Tq + qt] = tot;
    if (a.stats) {
      atomicAdd(&a.stats[0], (unsigned long long)nc);
      atomicAdd(&a.stats[1], (unsigned long long)tot);
    }
  }
}

__global__ __launch_bounds__(MASK_NT) void mask_transpose_kernel(MaskArgs a) {
  __shared__ int red[MASK_NT / 64];
  const int T = a.T, Tq = a.Tq;
  const int L = work_index(blockIdx.x);
  const int kt = L % T;
  const int bh = L / T;
  const int tid = threadIdx.x;
  constexpr int PER = MAX_TQ / MASK_NT;
  const uint8_t* col = a.keep + (long)bh * Tq * T + kt;
  int f[PER], cnt = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int qt = tid * PER + u;
    f[u] = (qt < Tq) ? col[(long)qt * T] : 0;
    cnt += f[u];
  }
  int tot;
  int pos = block_exclusive_scan(cnt, red, tot);
  uint16_t* krow = a.kidx + ((long)bh * T + kt) * Tq;
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (f[u]) krow[pos++] = (uint16_t)(tid * PER + u);
  if (tid == 0) a.kcnt[(long)bh * T + kt] = tot;
}

hipError_t launch_mask(const float* tlse, const double* tw, const float* lse, int B, int H, int n, int causal,
                       int window, int q_tile, double negl, uint8_t* keep, int32_t* qcnt, uint16_t* qidx,
                       int32_t* kcnt, uint16_t* kidx, int64_t* stats, hipStream_t st) {
  const int T = (n + TILE - 1) / TILE, Tq = (n + q_tile - 1) / q_tile;
  MaskArgs a{tlse, lse, keep, qcnt, qidx, kcnt, kidx, reinterpret_cast<unsigned long long*>(stats),
             B, H, n, T, causal, window < n ? window : 0, tw, negl, Tq, q_tile};
  {
    ProfScope ps(PK_MASK_SELECT, st);
    hipLaunchKernelGGL(mask_select_kernel, dim3(B * H * Tq), dim3(MASK_NT), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    ProfScope ps(PK_MASK_TRANSPOSE, st);
    hipLaunchKernelGGL(mask_transpose_kernel, dim3(B * H * T), dim3(MASK_NT), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace backlite
