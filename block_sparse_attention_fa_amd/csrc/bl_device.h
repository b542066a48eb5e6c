// Device-side building blocks shared by the BackLite kernels (gfx950 / CDNA4).
//
// MFMA v_mfma_f32_32x32x16_bf16 lane layout (lane l, half h = l / 32):
//   A (32x16, MxK): lane holds A[m = l % 32][k = 8h .. 8h+7]
//   B (16x32, KxN): lane holds B[k = 8h .. 8h+7][n = l % 32]
//   C (32x32):      lane holds C[m = 8(r/4) + 4h + r%4][n = l % 32], r = 0..15
//
// LDS tiles hold 128 rows x D bf16, row-major, in 16-byte chunks.  Chunk c of
// row r is stored at chunk position c ^ swz(r) with swz(r) = 2(r%4) + (r/4)%2,
// so that eight consecutive rows read at the same chunk, and four consecutive
// rows read as two adjacent chunks by ds_read_b64_tr_b16, fall in distinct
// bank groups.
//
// ds_read_b64_tr_b16 (transpose read, per 16-lane group): lane i of the group
// supplies the address of 4 bf16 at (row k0 + i/4, col n0 + 4(i%4)); lane j of
// the group then receives column n0 + j of rows k0 .. k0+3.  This serves the
// MFMA operands whose contraction index runs along the tile's rows.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace backlite {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int TILE = 128;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// element offset of (row, chunk) in a swizzled tile with D columns
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {
  return row * D + ((chunk ^ swz(row)) << 3);
}

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

// Copy a [128 x D] bf16 tile from global rows (row r at src + r*stride
// elements) into a swizzled LDS tile; rows >= nvalid are zero-filled.
template <int D, int NT>
__device__ __forceinline__ void load_tile(bf16* tile, const uint16_t* src, long stride, int nvalid,
                                          int tid) {
  constexpr int CH = D / 8;
#pragma unroll
  for (int it = 0; it < TILE * CH / NT; ++it) {
    const int c = tid + it * NT;
    const int row = c / CH, ch = c % CH;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (row < nvalid) v = *reinterpret_cast<const u32x4*>(src + (long)row * stride + ch * 8);
    *reinterpret_cast<u32x4*>(tile + tile_off<D>(row, ch)) = v;
  }
}

// Asynchronous copy of a full [128 x D] bf16 tile (every row valid) from global
// memory into a swizzled LDS tile with global_load_lds_dwordx4: each wave
// instruction fills 64 consecutive 16-byte LDS slots (slot = lane), so lane l
// fetches the global chunk that belongs at its slot, i.e. the inverse swizzle.
// Completion: s_waitcnt vmcnt(0) in the issuing wave, then a barrier.
template <int D, int NT>
__device__ __forceinline__ void dma_tile(bf16* tile, const uint16_t* src, long stride, int tid) {
  constexpr int CH = D / 8;
  constexpr int NW = NT / 64;
  constexpr int NI = TILE * CH / NT;  // instructions per thread
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot0 = (i * NW + wave) * 64;  // first slot of this wave instruction
    const int s = slot0 + lane;
    const int row = s / CH, pch = s % CH;
    const uint16_t* g = src + (long)row * stride + ((pch ^ swz(row)) << 3);
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(g),
                                     (__attribute__((address_space(3))) void*)(tile + slot0 * 8), 16, 0, 0);
  }
}

// Asynchronous copy of n32 4-byte words (n32 a multiple of 64) into LDS by one
// wave: lane l of instruction i lands word 64i + l.
__device__ __forceinline__ void dma_words(float* lds, const float* src, int n32, int lane) {
  for (int i = 0; i < n32 / 64; ++i)
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src + 64 * i + lane),
                                     (__attribute__((address_space(3))) void*)(lds + 64 * i), 4, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Map a hardware workgroup id to a logical work index so that consecutive
// logical indices run on the same XCD (workgroups are dealt round-robin over
// the 8 XCDs; each XCD has its own L2).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int NX = 8;
  const int per = total / NX, rem = total % NX;
  const int x = bid % NX, i = bid / NX;
  return (x < rem) ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

__device__ __forceinline__ long pair_index(int qt, int kt, int T, bool causal) {
  return causal ? (long)qt * (qt + 1) / 2 + kt : (long)qt * T + kt;
}

}  // namespace backlite
