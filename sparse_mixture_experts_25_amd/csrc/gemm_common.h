// Tile decoding and epilogues shared by the bf16 (matrix-core) and fp32 (SIMT)
// grouped matmuls.
#pragma once

#include "common.h"
#include "internal.h"

namespace moe {

// Where one workgroup's tile lives.
struct TileInfo {
  int g;        // group (== E for the shared expert), -1 = no work
  int64_t r0;   // first row of the group in A (and C for ragged-M)
  int rows;     // rows of the group (M for ragged-M, K for ragged-K)
  int m0;       // first tile row inside the group (ragged-M)
};

// Ragged-M: map a linear row-tile index to (group, first row) by an exclusive
// scan of ceil(rows_g / BM) over the groups. Wave 0 does the scan; the result
// goes through LDS to the whole workgroup.
template <int BM>
__device__ TileInfo decode_row_tile(const GemmArgs& a, int64_t tile, int* lds4) {
  const int ngroups = a.E + (a.shared_rows > 0 ? 1 : 0);
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int per = (ngroups + 63) / 64;
    const int g0 = lane * per;
    int64_t local = 0;
    for (int i = 0; i < per; ++i) {
      const int g = g0 + i;
      if (g < ngroups) {
        const int rows = (g < a.E) ? (a.offsets[g + 1] - a.offsets[g]) : a.shared_rows;
        local += (rows + BM - 1) / BM;
      }
    }
    int64_t incl = local;
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    const int64_t excl = incl - local;
    if (lane == 0) lds4[0] = -1;
    // exactly one lane owns the tile (if it exists)
    if (tile >= excl && tile < incl) {
      int64_t acc = excl;
      for (int i = 0; i < per; ++i) {
        const int g = g0 + i;
        const int rows = (g < a.E) ? (a.offsets[g + 1] - a.offsets[g]) : a.shared_rows;
        const int64_t nt = (rows + BM - 1) / BM;
        if (tile < acc + nt) {
          lds4[0] = g;
          lds4[1] = (g < a.E) ? a.offsets[g] : 0;
          lds4[2] = rows;
          lds4[3] = (int)(tile - acc) * BM;
          break;
        }
        acc += nt;
      }
    }
  }
  __syncthreads();
  TileInfo ti;
  ti.g = lds4[0];
  ti.r0 = lds4[1];
  ti.rows = lds4[2];
  ti.m0 = lds4[3];
  return ti;
}

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + __expf(-z)); }

// Epilogue for 8 consecutive output columns of one row (bf16 outputs), or
// fewer for fp32 (V = 4). `v` holds the fp32 accumulators. For SwiGLU forward,
// `v` holds the gate and `u` the up pre-activations of the same columns.
template <typename TO, int V>
struct Epi {
  __device__ static void store(TO* p, const float* v) {
    st128(p, Elem<TO>::pack(v));
  }
  __device__ static void load(const TO* p, float* v) { Elem<TO>::unpack(ld128(p), v); }
};

}  // namespace moe
