// Device-side building blocks shared by the BackLite kernels (gfx950 / CDNA4).
//
// MFMA v_mfma_f32_32x32x16_bf16 lane layout (lane l, half h = l / 32):
//   A (32x16, MxK): lane holds A[m = l % 32][k = 8h .. 8h+7]
//   B (16x32, KxN): lane holds B[k = 8h .. 8h+7][n = l % 32]
//   C (32x32):      lane holds C[m = 8(r/4) + 4h + r%4][n = l % 32], r = 0..15
//
// LDS tiles hold 128 rows x D bf16, row-major, in 16-byte chunks.  Chunk c of
// row r is stored at chunk position c ^ swz<D>(r).  For D = 128 (16 chunks, one
// 256-byte row of the 64 LDS banks) swz(r) = 4(r%4) + (r/4)%4: any 16
// consecutive rows (from a multiple of 16) take 16 distinct positions, so 16
// lanes reading one chunk of 16 rows (ds_read_b128) hit every bank once, and
// rows 4j .. 4j+3 put an aligned group of 4 chunks into 4 different bank
// quarters, so 32 lanes reading 4 rows x 64 bytes (two 16-lane groups of
// ds_read_b64_tr_b16) are conflict-free as well.  (An earlier swz, 8(r%2) +
// (r/2)%8, left rows r and r+2 in the same quarter: two-way conflicts on every
// transpose read, a third of the forward's LDS cycles on MI355X.)  For D = 64
// (8 chunks per row) swz(r) = 2(r%4) + (r/4)%2.  swz depends on r % 16 only, so
// shifting a read by a multiple of 16 rows is a constant offset.
//
// ds_read_b64_tr_b16 (transpose read, per 16-lane group): lane i of the group
// supplies the address of 4 bf16 at (row k0 + i/4, col n0 + 4(i%4)); lane j of
// the group then receives column n0 + j of rows k0 .. k0+3.  This serves the
// MFMA operands whose contraction index runs along the tile's rows.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace backlite {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int TILE = 128;
constexpr int MAX_TILES = 1024;  // tiles per sequence: n <= 131072 (checked at the C ABI)
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 1) | ((r >> 2) & 1);
}

// element offset of (row, chunk) in a swizzled tile with D columns
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * D + ((chunk ^ swz<D>(row)) << 3);
}

// Per-lane byte offsets of the two MFMA operand read patterns on a tile, so that
// every read in the inner loops is "lane offset + compile-time immediate".
//   row pattern: lane reads row blk*32 + l32, chunk 2ks + h32 (A rows of S/dP,
//                8 consecutive elements along the head dimension)
//   tr pattern:  16-lane group g reads rows 32kb + 16st + 4*h32 + 8*half + i/4,
//                columns 32db + 16(g%2) + 4(i%4) (ds_read_b64_tr_b16)
//   db_shift: the tr offsets of column block db are those of block db + db_shift
//   (a wave that works on a slice of the head dimension); blocks past D / 32
//   are left unset.
template <int D>
struct LdsOffsets {
  int row[D / 16];
  int tr[2][D / 32];
  __device__ __forceinline__ void init(int lane, int db_shift = 0) {
    const int l32 = lane & 31, h32 = lane >> 5, i = lane & 15, g = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) row[ks] = 2 * tile_off<D>(l32, 2 * ks + h32);
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int r = 4 * h32 + 8 * half + (i >> 2);
        const int col = 32 * (db + db_shift) + 16 * (g & 1) + 4 * (i & 3);
        tr[half][db] = col < D ? 2 * (tile_off<D>(r, col >> 3) + (col & 7)) : 0;
      }
  }
};

template <int D>
__device__ __forceinline__ bf16x8 rd_row(const bf16* tile, const LdsOffsets<D>& o, int blk, int ks) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(tile) + o.row[ks] + blk * 32 * D * 2);
}

// bf16x8 operand over rows 32kb + 16st + 4*h32 + {0..3, 8..11} of column block db
template <int D>
__device__ __forceinline__ bf16x8 rd_tr(const bf16* tile, const LdsOffsets<D>& o, int kb, int st, int db) {
  const char* base = reinterpret_cast<const char*>(tile) + (32 * kb + 16 * st) * D * 2;
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(base + o.tr[0][db]));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(base + o.tr[1][db]));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte row read: 8 consecutive columns of one row
template <int D>
__device__ __forceinline__ bf16x8 lds_row8(const bf16* tile, int row, int chunk) {
  return *reinterpret_cast<const bf16x8*>(tile + tile_off<D>(row, chunk));
}

// Transposed read (see header): 4 rows k0..k0+3 of column n0 + (lane % 16).
// k0 and n0 may differ per 16-lane group; n0 must be a multiple of 16.
template <int D>
__device__ __forceinline__ bf16x4 lds_tr4(const bf16* tile, int k0, int n0, int lane) {
  const int i = lane & 15;
  const int row = k0 + (i >> 2);
  const int col = n0 + ((i & 3) << 2);
  const bf16* p = tile + tile_off<D>(row, col >> 3) + (col & 7);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (__attribute__((address_space(3))) bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Registers r = 8s .. 8s+7 of a C fragment, converted to bf16 (RNE).
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int s) {
  bf16x8 o;
#pragma unroll
  for (int u = 0; u < 8; ++u) o[u] = (bf16)c[8 * s + u];
  return o;
}

// As pack8, and also accumulate the rounding residuals c - bf16(c) into lo.
__device__ __forceinline__ bf16x8 pack8_lo(const f32x16& c, int s, float& lo) {
  bf16x8 o;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const bf16 b = (bf16)c[8 * s + u];
    o[u] = b;
    lo += c[8 * s + u] - (float)b;
  }
  return o;
}

// Asynchronous copies global -> LDS with the load-to-LDS instructions, in
// their buffer form (buffer_load_dword{,x4} ... lds): the wave's 64 lanes fill
// 64 consecutive LDS slots (slot = lane).  With the buffer form the compiler
// keeps counting LDS reads precisely while a copy is in flight; with the
// global form (global_load_lds_dword{,x4}) it made every MFMA wait for all
// outstanding LDS reads, so only the buffer form is used.  Completion:
// s_waitcnt vmcnt(0) in the issuing wave, then a barrier.
// raw buffer resource: stride 0, `range` bytes (loads at or past it read 0), dword format word
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t range = 0x7FFFFFFFu) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)range, 0x00020000);
}

typedef __attribute__((address_space(3))) char lds_byte;
__device__ __forceinline__ lds_byte* lds_ptr(const void* p) { return (lds_byte*)(p); }

// one lane's share of a load-to-LDS instruction: bytes at boff of the buffer
// land in slot `lane` of the LDS block at lds
__device__ __forceinline__ void load_lds16(const __amdgpu_buffer_rsrc_t& rs, lds_byte* lds, uint32_t boff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 16, boff, 0, 0, 0);
}
__device__ __forceinline__ void load_lds4(const __amdgpu_buffer_rsrc_t& rs, lds_byte* lds, uint32_t boff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds, 4, boff, 0, 0, 0);
}

// Asynchronous copy of a full [128 x D] bf16 tile (every row valid) into a
// swizzled LDS tile: lane l fetches the global chunk that belongs at its slot,
// i.e. the inverse swizzle.  The per-thread source offsets depend only on the
// row stride and are computed once.
template <int D, int NT>
struct DmaOffsets {
  static constexpr int NI = TILE * (D / 8) / NT;  // instructions per thread per tile
  uint32_t off[NI];                               // byte offsets within the source tile
  __device__ __forceinline__ void init(long stride, int tid) {
    constexpr int CH = D / 8;
    constexpr int NW = NT / 64;
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int s = (i * NW + wave) * 64 + lane;
      const int row = s / CH, pch = s % CH;
      off[i] = (uint32_t)(row * stride + ((pch ^ swz<D>(row)) << 3)) * 2u;
    }
  }
};

// `range` (bytes from src) bounds the copy: chunks at or past it read as
// zero, so a ragged tile is copied with range = (nvalid - 1) * row stride + D
// elements, and its padding rows arrive zero-filled.
template <int D, int NT>
__device__ __forceinline__ void dma_tile(bf16* tile, const uint16_t* src, const DmaOffsets<D, NT>& o, int tid,
                                         uint32_t range = 0x7FFFFFFFu) {
  constexpr int NW = NT / 64;
  const int wave = tid >> 6;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src, range);
#pragma unroll
  for (int i = 0; i < DmaOffsets<D, NT>::NI; ++i) {
    const int slot0 = (i * NW + wave) * 64;  // first slot of this wave instruction
    load_lds16(rs, lds_ptr(tile + slot0 * 8), o.off[i]);
  }
}

// Scheduling hints (instruction classes of __builtin_amdgcn_sched_group_barrier).
constexpr int SG_VALU = 0x002, SG_MFMA = 0x008, SG_DS_READ = 0x100;

// Ask the scheduler for: `ahead` LDS reads, then `steps` x [m MFMA, r LDS reads],
// then the remaining MFMAs `tail`.  Keeps operand loads a few MFMAs ahead of use.
template <int AHEAD, int STEPS, int M, int R, int TAIL>
__device__ __forceinline__ void sched_interleave() {
  __builtin_amdgcn_sched_group_barrier(SG_DS_READ, AHEAD, 0);
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, M, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, TAIL, 0);
}

// Compile-time loop: calls f(std::integral_constant<int, I>) for I = I0 .. N-1,
// so every index inside f is a constant expression (a plain loop of this size
// is not always unrolled, and a rolled loop indexes registers dynamically).
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Work order.  Workgroups are dealt round-robin over the 8 XCDs (each with its
// own L2); measured on MI355X, the plain order (consecutive workgroups = tiles
// of the same head, so the whole chip works through one head's K/V or Q/G_O
// at a time and the 256 MB Infinity Cache holds it) beats grouping each head
// on one XCD by 20% in the backward, so no remapping is applied.  (A finer
// grouping, 32 consecutive key tiles per XCD within each chip-wide group of
// 256, measured no change in the G_K/G_V pass either: 12.96 vs 12.93 ms.)
__device__ __forceinline__ int work_index(int bid) { return bid; }
__device__ __forceinline__ long pair_index(int qt, int kt, int T, bool causal) {
  return causal ? (long)qt * (qt + 1) / 2 + kt : (long)qt * T + kt;
}

}  // namespace backlite
