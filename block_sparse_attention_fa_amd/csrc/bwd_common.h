// Argument block shared by the backward kernels (bwd.hip: D, key means,
// G_K/G_V; bwd_dq.hip: G_Q).
#pragma once
#include "bl_device.h"

namespace backlite {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* olo;  // optional bf16 residual of O (O_fp32 ~ O + olo)
  const uint16_t* dout;
  const float* lse;
  const int32_t* qcnt;
  const uint16_t* qidx;
  const int32_t* kcnt;
  const uint16_t* kidx;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dbuf;  // D, [B, H, n]
  float* lse2;  // row LSE in log2 units (LSE * log2 e), [B, H, n]
  float* kbar;  // per key tile mean of K over its valid keys, [B, Hk, T, d]
  // Stored-G_S state (all NULL when the workspace holds no slots).
  int32_t* gsinfo;     // [0] 1 = every kept tile had a slot, [1] kept tiles, [2] kept tiles with a slot
  uint32_t* qbase;     // [B, H, Tq]: first slot of each query tile's kept tiles
  uint32_t* kslot;     // [B, H, T, Tq]: slot of each k-list entry, laid out like kidx
  uint16_t* gs;        // slots of qrows x 128 bf16 G_S
  float* gsl;          // per slot, [4 key quarters][qrows rows] sums of the G_S rounding residual
  long long gs_cap;    // slots available
  // Chunked G_K/G_V work (always present): header [4] = {chunks, partial slots,
  // chunk length, chunk length of the ragged last key tile}, then the chunk table int4 [2 * NK] = {key tile (b, g, kt)
  // index, first item, end item, partial slot or -1}, then per key tile the
  // item count, first chunk and first partial slot (int32 [NK] each), where
  // NK = B * Hk * T.
  int32_t* dkplan;
  float* dkpart;       // partial G_K, G_V of split key tiles: [slot][2][128][d] fp32, NK slots
  int dk_chmin;        // smallest chunk length
  int dk_pcap;         // partial slots available (<= NK); bounds the number of split chunks
  float* dqacc;        // fp32-atomic G_Q variant: [B, H, T * 128, d] accumulator of G_S K (else NULL)
  int B, n, H, Hk, T;  // T: key tiles of 128 keys
  int Tq, qrows;       // query tiles of the lists and their rows (128, or 64: half-height backward tiles)
  int window;          // sliding window (causal only): key j visible to row i iff i - window < j; 0 = none
  float scale;
  float scale_log2;
};

// Chunk length of key tile k's G_K/G_V list in the plan (header word 2; word 3
// for the ragged last key tile when n is not a multiple of 128).
__device__ inline int dk_chunk_len(const BwdArgs& a, int k) {
  return (k % a.T == a.T - 1 && a.T * TILE != a.n) ? a.dkplan[3] : a.dkplan[2];
}

// Most chunks one key tile's G_K/G_V list can split into: the list holds at
// most G * Tq items (every query tile of every head of the group) and a chunk
// holds at least dk_chmin of them.
__host__ __device__ inline int ragged_chunks_max(const BwdArgs& a) {
  const int cm = a.dk_chmin < 1 ? 1 : a.dk_chmin;
  return ((a.H / a.Hk) * a.Tq + cm - 1) / cm;
}

// Issue order of the MFMAs of one tile in the backward passes: 8 phases,
// A0 A1 B0 A2 B1 A3 B2 B3.  A(c) (LA MFMAs) forms the scores and G_P of 32-row
// chunk c, B(c) (LB MFMAs) accumulates gradients from that chunk's P / G_S.
// The softmax of chunk c runs between the end of A(c) and the start of B(c),
// its 16 register elements spread evenly over the MFMAs issued there (A1 for
// chunk 0, B0 A2 for chunk 1, B1 A3 for chunk 2, B2 for chunk 3).
template <int LA, int LB>
struct TileSched {
  static constexpr bool is_b(int ph) { return (0xD4 >> ph) & 1; }
  static constexpr int chunk(int ph) {
    return ph == 0 ? 0 : ph == 1 ? 1 : ph == 2 ? 0 : ph == 3 ? 2 : ph == 4 ? 1 : ph == 5 ? 3 : ph == 6 ? 2 : 3;
  }
  static constexpr int len(int ph) { return is_b(ph) ? LB : LA; }
  static constexpr int start(int ph) {
    int s = 0;
    for (int i = 0; i < ph; ++i) s += len(i);
    return s;
  }
  static constexpr int total = 4 * (LA + LB);
  static constexpr int phase_of(int k) {
    int ph = 0;
    while (ph < 7 && start(ph + 1) <= k) ++ph;
    return ph;
  }
  static constexpr int a_phase(int c) { return c == 0 ? 0 : c == 1 ? 1 : c == 2 ? 3 : 5; }
  static constexpr int b_phase(int c) { return c == 0 ? 2 : c == 1 ? 4 : c == 2 ? 6 : 7; }
  static constexpr int soft_begin(int c) { return start(a_phase(c)) + LA; }
  static constexpr int soft_end(int c) { return start(b_phase(c)); }
  static constexpr int elem_step(int c, int e) { return soft_begin(c) + e * (soft_end(c) - soft_begin(c)) / 16; }
};

}  // namespace backlite
