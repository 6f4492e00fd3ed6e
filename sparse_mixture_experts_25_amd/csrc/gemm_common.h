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

// Upper bound on the number of row tiles of a ragged-M launch: sum over the
// groups of ceil(rows_g / BM) <= ceil(R / BM) + E (+ the shared group's tiles).
__host__ __device__ inline int64_t row_tile_bound(const GemmArgs& a, int BM) {
  const int64_t b = (a.max_rows + BM - 1) / BM + a.E + (a.shared_rows + BM - 1) / BM;
  if (a.split_part != 2) return b;
  // only groups under split_rows rows: at most ceil(split_rows / BM) tiles each
  const int64_t s = (int64_t)(a.E + 1) * ((a.split_rows + BM - 1) / BM);
  return s < b ? s : b;
}
// whether a group with `rows` rows belongs to this launch (GemmArgs::split_part)
__host__ __device__ inline bool group_in_part(const GemmArgs& a, int rows) {
  return a.split_part == 0 || (a.split_part == 1 ? rows >= a.split_rows : rows < a.split_rows);
}

// XCD-aware grouped rasterization. The dispatcher hands workgroup ids to the
// 8 XCDs round-robin (id % 8), and each XCD has its own L2. Workgroup ids are
// remapped so that each XCD owns one contiguous range of logical tiles, and the
// logical order walks groups of GM row tiles across all column tiles, so that
// concurrently running workgroups on one XCD share operand tiles in its L2.
// The grid is 1-D with at least nrow * ncol rounded up to a multiple of 8
// workgroups (a ragged-M launch sizes it from an upper bound on nrow). The map
// bid -> L is a bijection from the workgroups with bid / 8 < per onto
// [0, 8 * per); every other workgroup has no tile.
constexpr int kXcds = 8;
__host__ __device__ inline int64_t raster_grid(int64_t nrow, int64_t ncol) {
  return (nrow * ncol + kXcds - 1) / kXcds * kXcds;
}
__device__ inline bool raster_tile(int64_t nrow, int64_t ncol, int GM, int64_t& row, int64_t& col) {
  const int64_t total = nrow * ncol;
  const int64_t per = raster_grid(nrow, ncol) / kXcds;
  const int64_t bid = blockIdx.x;
  if (bid / kXcds >= per) return false;
  const int64_t L = (bid % kXcds) * per + bid / kXcds;
  if (L >= total) return false;
  const int64_t gsize = (int64_t)GM * ncol;
  const int64_t first = (L / gsize) * GM;
  const int64_t gm = (nrow - first) < GM ? (nrow - first) : GM;
  const int64_t local = L % gsize;
  row = first + local % gm;
  col = local / gm;
  return true;
}

// Ragged-M tile placement. Wave 0 scans ceil(rows_g / BM) over the groups
// (each lane owns a run of groups) to get the actual number of row tiles; the
// workgroup id is then mapped XCD-aware over (actual row tiles) x ncol (see
// raster_tile), and the owning lane resolves the row tile to (group, first row).
// Everything goes through LDS to the whole workgroup. Returns false when this
// workgroup has no tile.
template <int BM>
__device__ bool locate_ragged_m(const GemmArgs& a, int64_t ncol, int GM, int* lds, TileInfo& ti, int& col) {
  const int ngroups = a.E + (a.shared_rows > 0 ? 1 : 0);
  const int per = (ngroups + 63) / 64;
  int64_t* lds64 = reinterpret_cast<int64_t*>(lds + 8);  // [0]: total row tiles
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int64_t local = 0;
    for (int i = 0; i < per; ++i) {
      const int g = lane * per + i;
      if (g < ngroups) {
        const int rows = (g < a.E) ? (a.offsets[g + 1] - a.offsets[g]) : a.shared_rows;
        if (group_in_part(a, rows)) local += (rows + BM - 1) / BM;
      }
    }
    int64_t incl = local;
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    if (lane == 63) lds64[0] = incl;
    if (lane == 0) lds[0] = -1;
  }
  __syncthreads();
  const int64_t nrow = lds64[0];
  int64_t row, c;
  const bool have = raster_tile(nrow, ncol, GM, row, c);
  if (have && threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int64_t local = 0;
    for (int i = 0; i < per; ++i) {
      const int g = lane * per + i;
      if (g < ngroups) {
        const int rows = (g < a.E) ? (a.offsets[g + 1] - a.offsets[g]) : a.shared_rows;
        if (group_in_part(a, rows)) local += (rows + BM - 1) / BM;
      }
    }
    int64_t incl = local;
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    const int64_t excl = incl - local;
    if (row >= excl && row < incl) {
      int64_t accum = excl;
      for (int i = 0; i < per; ++i) {
        const int g = lane * per + i;
        const int rows = (g < a.E) ? (a.offsets[g + 1] - a.offsets[g]) : a.shared_rows;
        const int64_t nt = group_in_part(a, rows) ? (rows + BM - 1) / BM : 0;
        if (row < accum + nt) {
          lds[0] = g;
          lds[1] = (g < a.E) ? a.offsets[g] : 0;
          lds[2] = rows;
          lds[3] = (int)(row - accum) * BM;
          break;
        }
        accum += nt;
      }
    }
  }
  __syncthreads();
  if (!have || lds[0] < 0) return false;
  ti.g = lds[0];
  ti.r0 = lds[1];
  ti.rows = lds[2];
  ti.m0 = lds[3];
  col = (int)c;
  return true;
}

// Ragged-K tile placement. Workgroups of one group are consecutive and the
// per-group count is a multiple of 8, so workgroup t of a group runs on XCD
// t % 8. The group's tiles are numbered with the block index of the larger
// output dimension slowest, and XCD x takes the x-th eighth of that range
// (balanced to one tile): each block of the larger dimension, whose operand
// panel is the larger one, is read into at most two XCDs' L2s.
__host__ __device__ inline int64_t ragged_k_per_group(int nM, int nN) {
  return (((int64_t)nM * nN + 7) / 8) * 8;
}
__device__ inline bool k_tile(int64_t t, int nM, int nN, int& mb, int& nb) {
  const int64_t per = ((int64_t)nM * nN + 7) / 8;
  const int64_t L = (t % 8) * per + t / 8;
  if (L >= (int64_t)nM * nN) return false;
  if (nM <= nN) {
    nb = (int)(L / nM);
    mb = (int)(L % nM);
  } else {
    mb = (int)(L / nN);
    nb = (int)(L % nN);
  }
  return true;
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
