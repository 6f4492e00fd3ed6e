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

// Grouped rasterization. Logical tile L = workgroup id, walked in bands of GM
// row tiles across all column tiles (row fastest inside a band). The
// dispatcher hands workgroup ids to the 8 XCDs round-robin (id % 8), and each
// XCD has its own L2: with GM = 4 (the row-ragged launches), XCDs x and x + 4
// take row tile x of a band against alternate column tiles, so a row tile's
// activation panel is read into two L2s, and the weight panel of a column
// tile, which four XCDs read at about the same time, comes to the later ones
// from the last-level cache. (Measured per step: GM = 4 beat 8 by about 1 %
// and 16, 2 and 1 by more; remapping ids so that each XCD owned a contiguous
// range of logical tiles, 8 row tiles x 4 column tiles at a time, was 1-2 %
// slower than this on the DeepSeek-V3-, GShard- and Switch-shaped layers.)
// The grid is 1-D with at least nrow * ncol rounded up to a multiple of
// 8 workgroups (a ragged-M launch sizes it from an upper bound on nrow); the
// workgroups past nrow * ncol have no tile.
constexpr int kXcds = 8;
__host__ __device__ inline int64_t raster_grid(int64_t nrow, int64_t ncol) {
  return (nrow * ncol + kXcds - 1) / kXcds * kXcds;
}
__device__ inline bool raster_tile(int64_t nrow64, int64_t ncol64, int GM, int64_t& row, int64_t& col) {
  // nrow * ncol is at most the 1-D grid size (below 2^32), so every quotient
  // here is 32-bit (64-bit divisions are long instruction sequences)
  const uint32_t nrow = (uint32_t)nrow64, ncol = (uint32_t)ncol64;
  const uint32_t total = nrow * ncol;
  const uint32_t L = blockIdx.x;
  if (L >= total) return false;
  const uint32_t gsize = (uint32_t)GM * ncol;
  const uint32_t first = (L / gsize) * (uint32_t)GM;
  const uint32_t gm = (nrow - first) < (uint32_t)GM ? (nrow - first) : (uint32_t)GM;
  const uint32_t local = L % gsize;
  row = first + local % gm;
  col = local / gm;
  return true;
}

// Ragged-M tile placement. Wave 0 scans ceil(rows_g / BM) over the groups
// (each lane owns a run of groups) to get the actual number of row tiles; the
// workgroup id is then placed over (actual row tiles) x ncol in bands (see
// raster_tile), and the lane owning that row tile resolves it to (group, first
// row). One pass of wave 0, then one barrier: the result reaches the whole
// workgroup through LDS (lds[0..4]). Returns false when this workgroup has no
// tile.
template <int BM>
__device__ bool locate_ragged_m(const GemmArgs& a, int64_t ncol, int GM, int* lds, TileInfo& ti, int& col) {
  const int ngroups = a.E + (a.shared_rows > 0 ? 1 : 0);
  const int per = (ngroups + 63) / 64;
  // the first kKeep groups of each lane keep their first row and row count in
  // registers, so the owning lane resolves its tile without loading them again
  constexpr int kKeep = 8;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    auto group_rows = [&](int g) { return (g < a.E) ? (a.offsets[g + 1] - a.offsets[g]) : a.shared_rows; };
    auto group_tiles = [&](int rows) { return group_in_part(a, rows) ? (rows + BM - 1) / BM : 0; };
    int off[kKeep], rws[kKeep];
    int local = 0;  // row tiles of this lane's groups (every count is below 2^31)
#pragma unroll
    for (int i = 0; i < kKeep; ++i) {
      const int g = lane * per + i;
      off[i] = 0;
      rws[i] = 0;
      if (i < per && g < ngroups) {
        off[i] = (g < a.E) ? a.offsets[g] : 0;
        rws[i] = group_rows(g);
        local += group_tiles(rws[i]);
      }
    }
    for (int i = kKeep; i < per; ++i) {  // more than 64 * kKeep groups
      const int g = lane * per + i;
      if (g < ngroups) local += group_tiles(group_rows(g));
    }
    int incl = local;
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(incl, o, 64);
      if (lane >= o) incl += n;
    }
    const int nrow = __shfl(incl, 63, 64);  // row tiles of the launch
    int64_t row, c;
    const bool have = raster_tile(nrow, ncol, GM, row, c);
    if (lane == 0) {
      lds[0] = -1;  // replaced below by the owning lane (a later LDS write of this wave)
      lds[4] = have ? (int)c : 0;
    }
    const int excl = incl - local;
    if (have && row >= excl && row < incl) {
      const int r = (int)row;
      int accum = excl;
      bool found = false;
#pragma unroll
      for (int i = 0; i < kKeep; ++i) {
        const int nt = group_tiles(rws[i]);
        if (!found && i < per && r < accum + nt) {
          lds[0] = lane * per + i;
          lds[1] = off[i];
          lds[2] = rws[i];
          lds[3] = (r - accum) * BM;
          found = true;
        }
        accum += nt;
      }
      for (int i = kKeep; i < per && !found; ++i) {
        const int g = lane * per + i;
        const int rows = group_rows(g);
        const int nt = group_tiles(rows);
        if (r < accum + nt) {
          lds[0] = g;
          lds[1] = (g < a.E) ? a.offsets[g] : 0;
          lds[2] = rows;
          lds[3] = (r - accum) * BM;
          found = true;
        }
        accum += nt;
      }
    }
  }
  __syncthreads();
  if (lds[0] < 0) return false;
  ti.g = lds[0];
  ti.r0 = lds[1];
  ti.rows = lds[2];
  ti.m0 = lds[3];
  col = lds[4];
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
__device__ inline bool k_tile(int64_t t64, int nM, int nN, int& mb, int& nb) {
  // 32-bit quotients: a group has far fewer than 2^31 tiles
  const uint32_t t = (uint32_t)t64, tiles = (uint32_t)nM * (uint32_t)nN;
  const uint32_t per = (tiles + 7) / 8;
  const uint32_t L = (t % 8) * per + t / 8;
  if (L >= tiles) return false;
  if (nM <= nN) {
    nb = (int)(L / (uint32_t)nM);
    mb = (int)(L % (uint32_t)nM);
  } else {
    mb = (int)(L / (uint32_t)nN);
    nb = (int)(L % (uint32_t)nN);
  }
  return true;
}

// The expert activation's logistic function. The activation is not a rounding
// point of the layer (its value is rounded to bf16 when stored, or feeds the
// fp32 derivative), so 1 / (1 + e^-z) takes the hardware reciprocal (1 ulp)
// instead of the correctly rounded division sequence, which made the SwiGLU
// epilogues ALU-bound. (The router's sigmoid gate decides routing and keeps its
// exact contract in gate_math.h.)
__device__ __forceinline__ float act_sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float silu_f(float z) { return z * act_sigmoid(z); }

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
