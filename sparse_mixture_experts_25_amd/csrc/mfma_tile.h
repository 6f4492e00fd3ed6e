// LDS tile layouts and v_mfma_f32_32x32x16_bf16 fragment reads shared by the
// bf16 matrix-core kernels.
#pragma once

#include "common.h"

namespace moe {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef short shortx8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------ LDS layouts
// offsets in elements
// K-contiguous rows hold BK/8 chunks; the swizzle permutes chunks within a row
template <int BK>
__device__ __forceinline__ int kc_swz(int r) { return r & (BK / 8 - 1); }
__device__ __forceinline__ int mn_swz(int k) { return k & 7; }
template <int BK>
__device__ __forceinline__ int kc_off(int r, int c) { return r * BK + ((c ^ kc_swz<BK>(r)) << 3); }
template <int R>
__device__ __forceinline__ int mn_off(int k, int c) {
  return k * R + (((c & ~7) | ((c ^ mn_swz(k)) & 7)) << 3);
}

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
