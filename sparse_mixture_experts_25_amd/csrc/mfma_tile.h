// LDS tile layouts and v_mfma_f32_32x32x16_bf16 fragment reads shared by the
// bf16 matrix-core kernels.
#pragma once

#include "common.h"

namespace moe {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------ LDS layouts
// Offsets in elements; a chunk is 16 bytes (8 bf16). The XOR swizzles are
// chosen so that the fragment reads below hit distinct LDS banks whether the
// LDS serves 8 lanes x 16 bytes or 16 lanes x 16 bytes per cycle (direct
// loads write whole 1 KB blocks and are conflict-free either way).
//
// K-contiguous tile: rows of BK elements. A fragment read touches one chunk
// of 32 consecutive rows; with 64-byte rows (BK = 32) rows r, r+2, r+4, r+6
// share a 128-byte bank window and r, r+4, r+8, r+12 a 256-byte one, so the
// chunk is XORed with ((r >> 1) ^ (r >> 2)) & 3, which differs within both
// sets. With 128-byte rows (BK = 64) it is XORed with r & 7.
template <int BK>
__device__ __forceinline__ int kc_swz(int r) {
  return BK == 32 ? (((r >> 1) ^ (r >> 2)) & 3) : (r & (BK / 8 - 1));
}
template <int BK>
__device__ __forceinline__ int kc_off(int r, int c) { return r * BK + ((c ^ kc_swz<BK>(r)) << 3); }
// MN-contiguous tile: k-rows of R elements. A transpose read touches, per 16
// lanes, chunk pairs of 4 consecutive k-rows (k & 3 = 0..3), and per 32 lanes
// 4 consecutive chunks of them. For R >= 128 (16 or more chunks per k-row) the
// low 4 bits of the chunk index are XORed with 0, 4, 10, 14 for k & 3 = 0..3,
// which puts those reads on distinct banks in both bank models; for R = 64 the
// low 3 bits are XORed with k & 7.
template <int R>
__device__ __forceinline__ int mn_chunk(int k, int c) {
  if (R >= 128) return (c & ~15) | ((c ^ (((k & 1) << 2) | (((k >> 1) & 1) * 10))) & 15);
  return (c & ~7) | ((c ^ k) & 7);
}
template <int R>
__device__ __forceinline__ int mn_off(int k, int c) { return k * R + (mn_chunk<R>(k, c) << 3); }

// ------------------------------------------------------------ fragments
// A/B fragment of v_mfma_f32_32x32x16_bf16: lane l holds 8 consecutive k
// (8*(l/32) .. +7 of the 16-k step s) of row/column (base + l % 32).
template <int BK>
__device__ __forceinline__ bf16x8 frag_kc(const uint16_t* tile, int base, int s, int lane) {
  return *reinterpret_cast<const bf16x8*>(tile + kc_off<BK>(base + (lane & 31), 2 * s + (lane >> 5)));
}

__device__ __forceinline__ shortx4 read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) shortx4*)(p));
}

// From a [BK k][R] tile: per 16-lane group, the transpose read gives lane i
// the 4 k-values of column c0 + i when source lane j reads 4 columns
// c0 + 4*(j & 3) .. +3 of k-row k0 + (j >> 2). Two reads cover 8 k.
template <int R>
__device__ __forceinline__ bf16x8 frag_mn(const uint16_t* tile, int base, int s, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int col = base + 16 * (g & 1) + 4 * (j & 3);
  const int k = 16 * s + 8 * (g >> 1) + (j >> 2);
  const shortx4 lo = read_tr(tile + mn_off<R>(k, col >> 3) + (col & 7));
  const shortx4 hi = read_tr(tile + mn_off<R>(k + 4, col >> 3) + (col & 7));
  const shortx8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace moe
