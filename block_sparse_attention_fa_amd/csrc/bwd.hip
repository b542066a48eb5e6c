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
// Stored-G_S path (bwd_gs.hip), when the workspace has G_S slots: the G_K/G_V
//   pass also writes each kept tile's bf16 G_S, and the G_Q pass multiplies the
//   stored G_S by K instead of rebuilding P and G_S, for every query tile whose
//   kept tiles all found a slot (the rest are recomputed).
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
hipError_t launch_dkdv_d64_atom(const BwdArgs& a, bool causal, hipStream_t st);
hipError_t launch_dkdv_d128_atom(const BwdArgs& a, bool causal, hipStream_t st);
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

// ---------------------------------------------------------------------------
// Chunked G_K/G_V work.  A key tile's list (every kept query tile of every head
// of its group) is walked by one workgroup, so one long list serialises the
// whole pass: with attention sinks every query tile keeps key tile 0, a list
// of T (x group size) tiles.  Lists longer than the chunk length CH are split
// into chunks of CH items, each its own workgroup; split chunks leave fp32
// partial sums that dk_reduce_kernel adds up in chunk order (deterministic).
// CH = max(minimum, ceil(2 * items / P)) with P <= NK the partial slots the
// workspace holds (NK normally; fewer in a fixed-size scratch): a split list of
// m > CH items makes ceil(m / CH) < 2m / CH chunks, so all split chunks
// together are fewer than 2 * items / CH <= P.  That bounds the partial slots
// by P and the chunks by NK + P <= 2 NK without reading anything back.
// The ragged last key tile (n not a multiple of 128) takes the shorter chunk
// length CHR = max(minimum, ceil(CH / 8)) when the partial slots still fit P
// with it (else CHR = CH): in the stored non-causal pass its chunks run in a
// launch of their own after the main one, where the longest chunk is the
// launch's whole duration.
// Chunk order: the workgroups take chunks in table order, so a long chunk
// dealt late stretches the end of the pass.  Key tiles are placed in 16
// classes of their longest chunk (min(m, L) relative to CH), longest class
// first, in key-tile order within a class; a tile's chunks stay contiguous.
// (On the 32k video-DiT mask this comes within ~1% of ordering every chunk
// by length.)  The partial slots keep key-tile order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void dk_plan_kernel(BwdArgs a) {
  __shared__ long long part[1024];
  __shared__ long long part2[1024];
  __shared__ int chs, chr, nch;
  __shared__ long long red2[2][1024];
  constexpr int NCLS = 16;
  __shared__ int cpos[NCLS][1024];  // per class and thread: chunk counts, then running positions
  __shared__ int cstart[NCLS];
  const int T = a.T, G = a.H / a.Hk;
  const int NK = a.B * a.Hk * T;
  int32_t* items = a.dkplan + 4 + 8 * NK;
  int32_t* cbase = items + NK;
  int32_t* pbase = cbase + NK;
  const int tid = threadIdx.x;
  const int per = (NK + 1023) / 1024;
  const int s0 = min(NK, tid * per), s1 = min(NK, s0 + per);
  long long sum = 0;
  for (int k = s0; k < s1; ++k) {
    const int kt = k % T, bg = k / T;
    const int g = bg % a.Hk, b = bg / a.Hk;
    int m = 0;
    for (int hh = 0; hh < G; ++hh) m += max(0, min(a.kcnt[((long)b * a.H + g * G + hh) * T + kt], a.Tq));
    items[k] = m;
    sum += m;
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 512; off >= 1; off >>= 1) {
    if (tid < off) part[tid] += part[tid + off];
    __syncthreads();
  }
  const long long P = max(1, min(a.dk_pcap, NK));
  if (tid == 0) chs = (int)max((long long)a.dk_chmin, (2 * part[0] + P - 1) / P);
  __syncthreads();
  const bool ragged = T * TILE != a.n;
  const int CH = chs, CHR0 = max(a.dk_chmin, (CH + 7) / 8);
  auto split_slots = [](int m, int L) { return m <= L ? 0 : (m + L - 1) / L; };
  {
    // partial slots with CH everywhere, and the ragged tiles' extra with CHR0
    long long ps = 0, px = 0;
    for (int k = s0; k < s1; ++k) {
      const int m = items[k];
      ps += split_slots(m, CH);
      if (ragged && k % T == T - 1) px += split_slots(m, CHR0) - split_slots(m, CH);
    }
    red2[0][tid] = ps;
    red2[1][tid] = px;
    __syncthreads();
    for (int off = 512; off >= 1; off >>= 1) {
      if (tid < off) {
        red2[0][tid] += red2[0][tid + off];
        red2[1][tid] += red2[1][tid + off];
      }
      __syncthreads();
    }
    if (tid == 0) chr = red2[0][0] + red2[1][0] <= P ? CHR0 : CH;
    __syncthreads();
  }
  const int CHR = chr;
  auto tile_len = [&](int k) { return (ragged && k % T == T - 1) ? CHR : CH; };
  auto tile_cls = [&](int m, int L) { return min(NCLS - 1, (int)((long long)min(m, L) * NCLS / (CH + 1))); };
#pragma unroll
  for (int c = 0; c < NCLS; ++c) cpos[c][tid] = 0;
  long long psum = 0;
  for (int k = s0; k < s1; ++k) {
    const int m = items[k], L = tile_len(k);
    const int c = m <= L ? 1 : (m + L - 1) / L;
    cpos[tile_cls(m, L)][tid] += c;
    psum += m <= L ? 0 : c;
  }
  part2[tid] = psum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scans over the threads
    const long long v2 = tid >= off ? part2[tid - off] : 0;
    int v[NCLS];
#pragma unroll
    for (int c = 0; c < NCLS; ++c) v[c] = tid >= off ? cpos[c][tid - off] : 0;
    __syncthreads();
    part2[tid] += v2;
#pragma unroll
    for (int c = 0; c < NCLS; ++c) cpos[c][tid] += v[c];
    __syncthreads();
  }
  if (tid == 0) {  // class ranges of the table, longest class first
    int run = 0;
    for (int c = NCLS - 1; c >= 0; --c) {
      cstart[c] = run;
      run += cpos[c][1023];
    }
    nch = run;
  }
  int ex[NCLS];  // this thread's first position within each class
#pragma unroll
  for (int c = 0; c < NCLS; ++c) ex[c] = tid > 0 ? cpos[c][tid - 1] : 0;
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NCLS; ++c) cpos[c][tid] = cstart[c] + ex[c];
  long long pr = part2[tid] - psum;
  for (int k = s0; k < s1; ++k) {
    const int m = items[k], L = tile_len(k);
    const int c = m <= L ? 1 : (m + L - 1) / L, cl = tile_cls(m, L);
    cbase[k] = cpos[cl][tid];
    cpos[cl][tid] += c;
    pbase[k] = (int)pr;
    pr += m <= L ? 0 : c;
  }
  if (tid == 1023) {
    a.dkplan[0] = nch;
    a.dkplan[1] = (int)part2[1023];
    a.dkplan[2] = CH;
    a.dkplan[3] = CHR;
  }
}

// the chunk table: one thread per key tile writes its chunks
__global__ __launch_bounds__(256) void dk_fill_kernel(BwdArgs a) {
  const int NK = a.B * a.Hk * a.T;
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= NK) return;
  const int32_t* items = a.dkplan + 4 + 8 * NK;
  const int m = items[k], cb = items[NK + k], pb = items[2 * NK + k], CH = dk_chunk_len(a, k);
  int4* tab = reinterpret_cast<int4*>(a.dkplan + 4);
  if (m <= CH) {
    tab[cb] = int4{k, 0, m, -1};
  } else {
    const int c = (m + CH - 1) / CH;
    for (int i = 0; i < c; ++i) tab[cb + i] = int4{k, i * CH, min(m, (i + 1) * CH), pb + i};
  }
}

// G_K, G_V of split key tiles: sum of the chunks' fp32 partials, in chunk
// order.  Workgroup (key tile k, slice s) handles 1/RS of the tile's 2*128*d
// values, 8 per thread, so the partials of one tile are read by RS workgroups
// at once; unsplit tiles return at once.
constexpr int DK_RS = 16;
template <int D>
__global__ __launch_bounds__(256) void dk_reduce_kernel(BwdArgs a) {
  const int T = a.T, n = a.n;
  const int NK = a.B * a.Hk * T;
  const int k = blockIdx.x / DK_RS, sl = blockIdx.x % DK_RS;
  const int32_t* items = a.dkplan + 4 + 8 * NK;
  const int m = items[k], CH = dk_chunk_len(a, k);
  if (m <= CH) return;
  const int c = (m + CH - 1) / CH, pb = items[2 * NK + k];
  const int kt = k % T, bg = k / T;
  const int g = bg % a.Hk, b = bg / a.Hk;
  const long kvstride = (long)a.Hk * D;
  const long base = ((long)b * n + (long)kt * TILE) * kvstride + (long)g * D;
  constexpr int PER = 2 * TILE * D / DK_RS;  // values per workgroup (multiple of 2048)
#pragma unroll
  for (int h2 = 0; h2 < PER / 1024; ++h2) {
    const int e = sl * PER + h2 * 1024 + threadIdx.x * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const float* src = a.dkpart + (size_t)pb * 2 * TILE * D + e;
    int i = 0;
    for (; i + 4 <= c; i += 4) {  // four independent loads in flight, added in chunk order
      const f32x4 p0 = *reinterpret_cast<const f32x4*>(src + (size_t)(i + 0) * 2 * TILE * D);
      const f32x4 p1 = *reinterpret_cast<const f32x4*>(src + (size_t)(i + 1) * 2 * TILE * D);
      const f32x4 p2 = *reinterpret_cast<const f32x4*>(src + (size_t)(i + 2) * 2 * TILE * D);
      const f32x4 p3 = *reinterpret_cast<const f32x4*>(src + (size_t)(i + 3) * 2 * TILE * D);
      acc += p0;
      acc += p1;
      acc += p2;
      acc += p3;
    }
    for (; i < c; ++i) acc += *reinterpret_cast<const f32x4*>(src + (size_t)i * 2 * TILE * D);
    const int t = e / (TILE * D), row = (e % (TILE * D)) / D, dim = e % D;
    if (kt * TILE + row >= n) continue;
    const float sc = t == 0 ? a.scale : 1.f;
    const bf16x4 o = {(bf16)(acc[0] * sc), (bf16)(acc[1] * sc), (bf16)(acc[2] * sc), (bf16)(acc[3] * sc)};
    *reinterpret_cast<bf16x4*>((t == 0 ? a.dk : a.dv) + base + (long)row * kvstride + dim) = o;
  }
}

// ---------------------------------------------------------------------------
// fp32-atomic G_Q variant: zero the accumulator before the pass, convert it
// to bf16 G_Q = scale * acc afterwards (rows >= n are padding).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void zero_f32x4_kernel(float* p, long n4) {
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long)gridDim.x * 256)
    reinterpret_cast<f32x4*>(p)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <int D>
__global__ __launch_bounds__(256) void dq_convert_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;  // lanes per row, 8 values each
  const long rows = (long)a.B * a.n * a.H;
  const long row = (long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  if (row >= rows) return;
  // row = (b*n + i)*H + h of G_Q; the accumulator is [b*H + h][T*128][D]
  const int h = (int)(row % a.H);
  const long bi = row / a.H;
  const int i = (int)(bi % a.n), b = (int)(bi / a.n);
  const float* src = a.dqacc + (((long)b * a.H + h) * (long)(a.T * TILE) + i) * D + sub * 8;
  const f32x4 x0 = reinterpret_cast<const f32x4*>(src)[0], x1 = reinterpret_cast<const f32x4*>(src)[1];
  bf16x8 o;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    o[u] = (bf16)(x0[u] * a.scale);
    o[4 + u] = (bf16)(x1[u] * a.scale);
  }
  *reinterpret_cast<bf16x8*>(a.dq + row * D + sub * 8) = o;
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
  const int NK = a.B * a.Hk * a.T;
  {
    ProfScope ps(PK_DK_PLAN, st);
    hipLaunchKernelGGL(dk_plan_kernel, dim3(1), dim3(1024), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(dk_fill_kernel, dim3((NK + 255) / 256), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.dqacc) {
    // fused single pass: G_K/G_V and the atomic G_Q product, then the conversion
    const long n4 = (long)a.B * a.H * a.T * TILE * D / 4;
    {
      ProfScope ps(PK_DQ, st);
      hipLaunchKernelGGL(zero_f32x4_kernel, dim3(2048), dim3(256), 0, st, a.dqacc, n4);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    {
      ProfScope ps(PK_DKDV, st);
      e = D == 64 ? launch_dkdv_d64_atom(a, CAUSAL, st) : launch_dkdv_d128_atom(a, CAUSAL, st);
      if (e != hipSuccess) return e;
    }
    {
      ProfScope ps(PK_DK_REDUCE, st);
      hipLaunchKernelGGL((dk_reduce_kernel<D>), dim3(NK * DK_RS), dim3(256), 0, st, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    ProfScope ps(PK_DQ, st);
    const long rows = (long)a.B * a.n * a.H;
    const long rpb = 256 / (D / 8);
    hipLaunchKernelGGL((dq_convert_kernel<D>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, st, a);
    return hipGetLastError();
  }
  // With slots in the workspace the G_K/G_V pass stores G_S for every kept
  // tile that has a slot (slots are dealt in query-tile order); each query tile
  // whose kept tiles all have one takes its G_Q from the stored tiles
  // (dqs_kernel), the others are recomputed (dq_kernel).  The choice per query
  // tile is made on the device, so the host reads nothing back.
  if (a.gsinfo) {
    e = launch_gs_slots(a, st);
    if (e != hipSuccess) return e;
    ProfScope ps(PK_DKDV, st);
    e = D == 64 ? launch_dkdv_d64_gs(a, CAUSAL, st) : launch_dkdv_d128_gs(a, CAUSAL, st);
  } else {
    ProfScope ps(PK_DKDV, st);
    e = D == 64 ? launch_dkdv_d64(a, CAUSAL, st) : launch_dkdv_d128(a, CAUSAL, st);
  }
  if (e != hipSuccess) return e;
  {
    ProfScope ps(PK_DK_REDUCE, st);
    hipLaunchKernelGGL((dk_reduce_kernel<D>), dim3(NK * DK_RS), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  e = launch_dq(a, D, CAUSAL, st);
  if (e != hipSuccess || !a.gsinfo) return e;
  return launch_dq_gs(a, D, st);
}

hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                      const uint16_t* olo, const uint16_t* dout, const float* lse, const int32_t* qcnt,
                      const uint16_t* qidx, const int32_t* kcnt, const uint16_t* kidx, int B, int n,
                      int H, int Hk, int d, float scale, int causal, int window, int q_tile, uint16_t* dq,
                      uint16_t* dk, uint16_t* dv, float* dbuf, float* lse2, float* kbar, int32_t* gsinfo, uint32_t* qbase,
                      uint32_t* kslot, uint16_t* gs, float* gsl, long long gs_cap, int32_t* dkplan,
                      float* dkpart, int dk_chmin, int dk_pcap, float* dqacc, hipStream_t st) {
  BwdArgs a{q,    k,      v,     o,     olo,    dout,   lse,      qcnt, qidx, kcnt, kidx, dq,
            dk,   dv,     dbuf,  lse2,  kbar,   gsinfo, qbase,    kslot, gs, gsl, gs_cap, dkplan,
            dkpart, dk_chmin, dk_pcap, dqacc, B, n, H, Hk, (n + TILE - 1) / TILE, (n + q_tile - 1) / q_tile, q_tile,
            window < n ? window : 0, scale, scale * LOG2E};
  if (d == 64) return causal ? launch_bwd_t<64, true>(a, st) : launch_bwd_t<64, false>(a, st);
  return causal ? launch_bwd_t<128, true>(a, st) : launch_bwd_t<128, false>(a, st);
}

}  // namespace backlite
