// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// 16-byte vector of raw bits.
struct alignas(16) u128 {
  uint32_t w[4];
};

__device__ __forceinline__ u128 ld128(const void* p) {
  u128 r;
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  return r;
}
// 16-byte load with the non-temporal (streaming) cache policy, for gathered rows
// that are read once.
__device__ __forceinline__ u128 ld128_nt(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  u128 r;
  r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
  return r;
}
__device__ __forceinline__ void st128(void* p, const u128& r) {
  *reinterpret_cast<uint4*>(p) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
}
// 16-byte store with the non-temporal (streaming) cache policy, for outputs
// that are written once and not read again soon.
__device__ __forceinline__ void st128_nt(void* p, const u128& r) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = {r.w[0], r.w[1], r.w[2], r.w[3]};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ u128 zero128() {
  u128 r;
  r.w[0] = r.w[1] = r.w[2] = r.w[3] = 0u;
  return r;
}

// bf16 <-> fp32. The narrowing conversion rounds to nearest even (gfx950 has a
// hardware convert for it).
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  bf16 h = (bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// An fp32 value as three bf16 terms hi + mid + lo (each the RNE rounding of
// what the previous terms leave), exact to about 2^-24 relative: products of
// two such terms are exact in fp32, so fp32-accumulated bf16 matrix products
// of the terms reproduce fp32 products.
struct Split3 {
  uint16_t h, m, l;
};
__device__ __forceinline__ Split3 split3(float v) {
  Split3 s;
  s.h = f2bf(v);
  const float r1 = v - bf2f(s.h);
  s.m = f2bf(r1);
  const float r2 = r1 - bf2f(s.m);
  s.l = f2bf(r2);
  return s;
}

// Processing order of the groups of a weight-gradient launch, computed by one
// workgroup of `nthreads` threads: order[position] = group. Groups with rows
// come largest first (ties: lower index), so the longest contractions start
// first; groups without rows (whose gradient is all zeros, a pure store) are
// spread evenly between them, so their stores overlap other workgroups' matrix
// work instead of forming a store-bound tail. With N groups with rows and Z
// without, the i-th with rows sits at time (2i+1)/(2N) and the j-th without at
// (2j+1)/(2Z) (ties: the one with rows first); position = rank by time.
// rows_s: LDS scratch of at least E + has_shared ints (at most 1025).
__device__ __forceinline__ void rank_groups_by_rows(const int32_t* __restrict__ offsets, int E, int shared_rows,
                                                    int has_shared, int32_t* __restrict__ order, int* rows_s,
                                                    int nthreads) {
  const int G = E + has_shared;
  for (int g = threadIdx.x; g < G; g += nthreads) rows_s[g] = g < E ? offsets[g + 1] - offsets[g] : shared_rows;
  __syncthreads();
  int Z = 0;
  for (int h = 0; h < G; ++h) Z += rows_s[h] == 0;
  const int N = G - Z;
  for (int g = threadIdx.x; g < G; g += nthreads) {
    const int r = rows_s[g];
    int rank = 0;  // among the groups of the same kind
    for (int h = 0; h < G; ++h) {
      const int rh = rows_s[h];
      rank += r > 0 ? ((rh > r) || (rh == r && h < g)) : (rh == 0 && h < g);
    }
    int before;  // groups of the other kind placed before it
    if (r > 0) {
      const int64_t x = (int64_t)(2 * rank + 1) * Z - N;
      before = x <= 0 ? 0 : (int)((x + 2 * (int64_t)N - 1) / (2 * (int64_t)N));
      before = before < Z ? before : Z;
    } else {
      const int64_t x = (int64_t)(2 * rank + 1) * N - Z;
      before = x < 0 ? 0 : (int)(x / (2 * (int64_t)Z)) + 1;
      before = before < N ? before : N;
    }
    order[rank + before] = g;
  }
}

// Thread u of the router-weight split: the 16 bytes (8 values of row r) of the
// split weights wsp [kp, d] = [W_hi ; W_mid ; W_hi ; 0 ...] (bf16), for
// u < kp * d / 8, and the row ranges of the router products (offs[0..1] = the
// single input-gradient group, offs[2 + c] = the first token of weight-gradient
// chunk c, for c <= nsw). Threads past both do nothing.
__device__ __forceinline__ void split_router_weights(int64_t u, const float* __restrict__ w, int E, int d, int kp,
                                                     uint16_t* __restrict__ wsp, int T, int nsw, int chunk,
                                                     int32_t* __restrict__ offs) {
  if (u <= nsw) offs[2 + u] = (int)min((int64_t)u * chunk, (int64_t)T);
  if (u == 0) {
    offs[0] = 0;
    offs[1] = T;
  }
  if (u >= (int64_t)kp * (d / 8)) return;
  const int r = (int)(u / (d / 8)), j0 = (int)(u % (d / 8)) * 8;
  const int e = r % E, band = r / E;
  u128 o = zero128();
  if (band < 3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const Split3 p = split3(w[(int64_t)e * d + j0 + 2 * i]), q = split3(w[(int64_t)e * d + j0 + 2 * i + 1]);
      const uint16_t x0 = band == 1 ? p.m : p.h, x1 = band == 1 ? q.m : q.h;
      o.w[i] = (uint32_t)x0 | ((uint32_t)x1 << 16);
    }
  }
  st128(wsp + (int64_t)r * d + j0, o);
}
__device__ __forceinline__ uint32_t pack2bf(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}

// Element access for the two activation types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16 bytes
  __device__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ static void store(float* p, int64_t i, float v) { p[i] = v; }
  __device__ static void unpack(const u128& r, float* v) {
    for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(r.w[i]);
  }
  __device__ static u128 pack(const float* v) {
    u128 r;
    for (int i = 0; i < 4; ++i) r.w[i] = __float_as_uint(v[i]);
    return r;
  }
};
template <> struct Elem<uint16_t> {
  static constexpr int kVec = 8;
  __device__ static float load(const uint16_t* p, int64_t i) { return bf2f(p[i]); }
  __device__ static void store(uint16_t* p, int64_t i, float v) { p[i] = f2bf(v); }
  __device__ static void unpack(const u128& r, float* v) {
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(r.w[i] << 16);
      v[2 * i + 1] = __uint_as_float(r.w[i] & 0xFFFF0000u);
    }
  }
  __device__ static u128 pack(const float* v) {
    u128 r;
    for (int i = 0; i < 4; ++i) r.w[i] = pack2bf(v[2 * i], v[2 * i + 1]);
    return r;
  }
};

// Wave-level reductions (fixed butterfly order, so results are reproducible).
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

}  // namespace moe
