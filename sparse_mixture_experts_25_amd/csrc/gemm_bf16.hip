// bf16 grouped matmuls on the gfx950 matrix cores, over ragged expert groups.
//
// [LRMOE] (ai-cafe.club LRMoE item, "この記事のポイント"): compacted
// expert-contiguous rows make the expert FFNs one variable-size grouped GEMM.
// [SW] ("Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散",
// ta-paperlens.web.app), section on replacing the FFN by N expert copies.
//
// One kernel template covers the six matmuls of the layer:
//   ragged-M (forward, and the input gradients): the row count of each group
//     comes from the device offsets; a linear row-tile index is decoded into
//     (group, row) in-kernel, so no host round trip is needed and empty
//     workgroups exit at once.
//   ragged-K (weight gradients): a fixed [M, N] output per group, contracted
//     over that group's rows; a group without rows writes zeros.
// Operands are staged in LDS as [rows][BK] with the K axis contiguous and the
// 16-byte chunks of each row XOR-swizzled by (row & 7) so that the fragment
// reads are bank-conflict free. An operand whose K axis is the slow one in
// memory ([K][MN], as in the gradient matmuls) is loaded as 4(k) x 8(mn)
// blocks and transposed in registers before the LDS store. Each of the four
// waves owns a (BM/2) x (BN/2) sub-tile computed with v_mfma_f32_32x32x16_bf16
// (fp32 accumulation). The epilogue stages the fp32 tile in LDS and writes
// 16-byte rows, fusing the activation (forward) or its derivative (backward).
#include "gemm_common.h"

namespace moe {

namespace {

constexpr int kBK = 64;
constexpr int kThreads = 256;

template <int R>
struct TileLoad {
  // registers staged between the global load and the LDS store
  static constexpr int kUnitsKC = R * kBK / 8 / kThreads;   // 16-byte units per thread (K-contig)
  static constexpr int kUnitsMN = (R / 8) * (kBK / 4) / kThreads;  // 4x8 blocks per thread (MN-contig)
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ (row & 7)) << 3); }

// K-contiguous operand: element (r, k) at base[r * ld + k]; rows >= rows_valid
// or k >= K read as zero. `rowmap` (SwiGLU weights) sends tile row r to a
// different source row.
template <int R, int MAP>
struct KcLoader {
  u128 reg[TileLoad<R>::kUnitsKC];
  __device__ void load(const uint16_t* base, int64_t ld, int rows_valid, int K, int k0, int map_half,
                       int map_f, int map_h0) {
#pragma unroll
    for (int i = 0; i < TileLoad<R>::kUnitsKC; ++i) {
      const int u = threadIdx.x + i * kThreads;
      const int r = u / (kBK / 8);
      const int c = u % (kBK / 8);
      const int k = k0 + c * 8;
      int64_t src;
      bool ok;
      if (MAP) {
        // tile rows [0, half) -> gate rows h0 + r; [half, R) -> up rows f + h0 + r - half
        const int hc = map_h0 + (r < map_half ? r : r - map_half);
        ok = hc < map_f && k < K;
        src = (int64_t)(r < map_half ? hc : map_f + hc) * ld + k;
      } else {
        ok = r < rows_valid && k < K;
        src = (int64_t)r * ld + k;
      }
      reg[i] = ok ? ld128(base + src) : zero128();
    }
  }
  __device__ void store(uint16_t* lds) const {
#pragma unroll
    for (int i = 0; i < TileLoad<R>::kUnitsKC; ++i) {
      const int u = threadIdx.x + i * kThreads;
      const int r = u / (kBK / 8);
      const int c = u % (kBK / 8);
      st128(lds + swz(r, c), reg[i]);
    }
  }
};

// MN-contiguous operand: element (r, k) at base[k * ld + r]; k >= k_valid or
// r >= rows_valid read as zero. Loaded as 4 (k) x 8 (r) blocks.
template <int R>
struct MnLoader {
  static constexpr int kU = TileLoad<R>::kUnitsMN;
  u128 reg[kU][4];
  __device__ void load(const uint16_t* base, int64_t ld, int rows_valid, int k_valid, int k0) {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int u = threadIdx.x + i * kThreads;
      const int ru = u % (R / 8);
      const int ku = u / (R / 8);
      const int r = ru * 8;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k = k0 + ku * 4 + j;
        const bool ok = r < rows_valid && k < k_valid;
        reg[i][j] = ok ? ld128(base + (int64_t)k * ld + r) : zero128();
      }
    }
  }
  __device__ void store(uint16_t* lds) const {
#pragma unroll
    for (int i = 0; i < kU; ++i) {
      const int u = threadIdx.x + i * kThreads;
      const int ru = u % (R / 8);
      const int ku = u / (R / 8);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int j = m >> 1;
        uint32_t d0, d1;
        if ((m & 1) == 0) {
          d0 = (reg[i][0].w[j] & 0xFFFFu) | (reg[i][1].w[j] << 16);
          d1 = (reg[i][2].w[j] & 0xFFFFu) | (reg[i][3].w[j] << 16);
        } else {
          d0 = (reg[i][0].w[j] >> 16) | (reg[i][1].w[j] & 0xFFFF0000u);
          d1 = (reg[i][2].w[j] >> 16) | (reg[i][3].w[j] & 0xFFFF0000u);
        }
        const int row = ru * 8 + m;
        const int kk = ku * 4;  // k offset inside the tile: chunk kk/8, half (kk/4)&1
        uint16_t* dst = lds + swz(row, kk >> 3) + (kk & 4);
        *reinterpret_cast<uint2*>(dst) = make_uint2(d0, d1);
      }
    }
  }
};

template <int BM, int BN, int KIND, int B_KC, int EPI>
__global__ __launch_bounds__(kThreads, (BM * BN >= 256 * 256) ? 1 : 2) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int A_KC = (KIND == 0);
  constexpr int B_IS_KC = (KIND == 0) && B_KC;
  constexpr int kOperandBytes = 2 * (BM + BN) * kBK * 2;
  constexpr int CP = BN + 8;  // padded row of the staged fp32 tile
  constexpr int HM = BM / 2;  // the fp32 tile is staged half (one wave row) at a time
  constexpr int kStageBytes = HM * CP * 4;
  constexpr int kLds = kOperandBytes > kStageBytes ? kOperandBytes : kStageBytes;
  __shared__ __attribute__((aligned(16))) uint8_t smem[kLds];
  __shared__ int info[4];

  uint16_t* As = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Bs = As + 2 * BM * kBK;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- locate the tile
  int g, rows, mrow0 = 0, nb, mb = 0;
  int64_t r0;
  if (KIND == 0) {
    TileInfo ti = decode_row_tile<BM>(a, blockIdx.x, info);
    if (ti.g < 0) return;
    g = ti.g; r0 = ti.r0; rows = ti.rows; mrow0 = ti.m0;
    nb = blockIdx.y;
  } else {
    g = blockIdx.y;
    const int nN = (a.N + BN - 1) / BN;
    mb = blockIdx.x / nN;
    nb = blockIdx.x % nN;
    if (g < a.E) {
      r0 = a.offsets[g];
      rows = a.offsets[g + 1] - a.offsets[g];
    } else {
      r0 = 0;
      rows = a.shared_rows;
    }
  }
  const bool sh = g >= a.E;
  const uint16_t* Ab = reinterpret_cast<const uint16_t*>(sh ? a.A_sh : a.A);
  const uint16_t* Bb = reinterpret_cast<const uint16_t*>(sh ? a.B_sh : a.B);
  if (!sh) Bb += (KIND == 0) ? (int64_t)g * a.strideB : 0;

  // K extent and operand origins
  int K;
  const uint16_t* Aorig;
  const uint16_t* Borig;
  int a_rows_valid, b_rows_valid;
  if (KIND == 0) {
    K = a.K;
    Aorig = Ab + (r0 + mrow0) * a.lda;
    a_rows_valid = rows - mrow0;
    if (B_KC) {
      Borig = Bb + (EPI == EPI_SWIGLU_FWD ? 0 : (int64_t)nb * BN * a.ldb);
      b_rows_valid = a.N - nb * BN;
    } else {
      Borig = Bb + (int64_t)nb * BN;  // [K][N]
      b_rows_valid = a.N - nb * BN;
    }
  } else {
    K = rows;
    Aorig = Ab + r0 * a.lda + (int64_t)mb * BM;  // [rows][M]
    Borig = Bb + r0 * a.ldb + (int64_t)nb * BN;  // [rows][N]
    a_rows_valid = a.M - mb * BM;
    b_rows_valid = a.N - nb * BN;
  }

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  KcLoader<BM, 0> la_kc;
  MnLoader<BM> la_mn;
  KcLoader<BN, (EPI == EPI_SWIGLU_FWD)> lb_kc;
  MnLoader<BN> lb_mn;
  const int map_half = BN / 2, map_h0 = nb * (BN / 2);

  auto load_tiles = [&](int k0) {
    if (A_KC) la_kc.load(Aorig, a.lda, a_rows_valid, K, k0, 0, 0, 0);
    else la_mn.load(Aorig, a.lda, a_rows_valid, K, k0);
    if (B_IS_KC) lb_kc.load(Borig, a.ldb, b_rows_valid, K, k0, map_half, a.f, map_h0);
    else lb_mn.load(Borig, a.ldb, b_rows_valid, K, k0);
  };
  auto store_tiles = [&](int buf) {
    if (A_KC) la_kc.store(As + buf * BM * kBK);
    else la_mn.store(As + buf * BM * kBK);
    if (B_IS_KC) lb_kc.store(Bs + buf * BN * kBK);
    else lb_mn.store(Bs + buf * BN * kBK);
  };

  const int nk = (K + kBK - 1) / kBK;
  if (nk > 0) {
    load_tiles(0);
    store_tiles(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * kBK);
    const uint16_t* Ab_l = As + buf * BM * kBK;
    const uint16_t* Bb_l = Bs + buf * BN * kBK;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int chunk = 2 * s + (lane >> 5);
      bf16x8 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * WM + i * 32 + (lane & 31);
        af[i] = *reinterpret_cast<const bf16x8*>(Ab_l + swz(row, chunk));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * WN + j * 32 + (lane & 31);
        bfr[j] = *reinterpret_cast<const bf16x8*>(Bb_l + swz(row, chunk));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: stage the fp32 tile in LDS one half (the rows of one wave
  // row) at a time, then write 16-byte row vectors
  float* Cs = reinterpret_cast<float*>(smem);
  uint16_t* C = reinterpret_cast<uint16_t*>(sh ? a.C_sh : a.C);
  uint16_t* C2 = reinterpret_cast<uint16_t*>(sh ? a.C2_sh : a.C2);
  const uint16_t* X = reinterpret_cast<const uint16_t*>(sh ? a.X_sh : a.X);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const int n = wn * WN + j * 32 + (lane & 31);
            Cs[m * CP + n] = acc[i][j][e];
          }
    }
    __syncthreads();
    const int mbase = half * HM;  // tile row of Cs row 0
    if (EPI == EPI_SWIGLU_FWD) {
      // columns [0, BN/2) hold gate, [BN/2, BN) up, for h columns nb*BN/2 + j
      constexpr int U = HM * (BN / 2) / 8;
      for (int u = tid; u < U; u += kThreads) {
        const int ml = u / (BN / 16);
        const int j = (u % (BN / 16)) * 8;
        const int m = mbase + ml;
        const int hc = nb * (BN / 2) + j;
        if (m >= rows - mrow0 || hc >= a.f) continue;
        const int64_t row = r0 + mrow0 + m;
        float gv[8], uv[8], hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          gv[e] = Cs[ml * CP + j + e];
          uv[e] = Cs[ml * CP + BN / 2 + j + e];
          hv[e] = silu_f(gv[e]) * uv[e];
        }
        st128(C + row * a.ldc + hc, Elem<uint16_t>::pack(gv));
        st128(C + row * a.ldc + a.f + hc, Elem<uint16_t>::pack(uv));
        st128(C2 + row * a.ldc2 + hc, Elem<uint16_t>::pack(hv));
      }
    } else {
      constexpr int U = HM * BN / 8;
      for (int u = tid; u < U; u += kThreads) {
        const int ml = u / (BN / 8);
        const int n = (u % (BN / 8)) * 8;
        const int m = mbase + ml;
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = Cs[ml * CP + n + e];
        if (KIND == 1) {
          const int mm = mb * BM + m, nn = nb * BN + n;
          if (mm >= a.M || nn >= a.N) continue;
          uint16_t* Cg = sh ? C : C + (int64_t)g * a.strideC;
          st128(Cg + (int64_t)mm * a.ldc + nn, Elem<uint16_t>::pack(v));
          continue;
        }
        const int col = nb * BN + n;
        if (m >= rows - mrow0 || col >= a.N) continue;
        const int64_t row = r0 + mrow0 + m;
        if (EPI == EPI_STORE) {
          st128(C + row * a.ldc + col, Elem<uint16_t>::pack(v));
        } else if (EPI == EPI_RELU_FWD) {
          float h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = fmaxf(v[e], 0.0f);
          st128(C + row * a.ldc + col, Elem<uint16_t>::pack(v));
          st128(C2 + row * a.ldc2 + col, Elem<uint16_t>::pack(h));
        } else if (EPI == EPI_RELU_BWD) {
          float xs[8];
          Elem<uint16_t>::unpack(ld128(X + row * a.ldx + col), xs);
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = xs[e] > 0.0f ? v[e] : 0.0f;
          st128(C + row * a.ldc + col, Elem<uint16_t>::pack(v));
        } else if (EPI == EPI_SWIGLU_BWD) {
          float gs[8], us[8], dg[8], du[8];
          Elem<uint16_t>::unpack(ld128(X + row * a.ldx + col), gs);
          Elem<uint16_t>::unpack(ld128(X + row * a.ldx + a.f + col), us);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float s = 1.0f / (1.0f + __expf(-gs[e]));
            du[e] = v[e] * gs[e] * s;
            dg[e] = v[e] * us[e] * s * (1.0f + gs[e] * (1.0f - s));
          }
          st128(C + row * a.ldc + col, Elem<uint16_t>::pack(dg));
          st128(C + row * a.ldc + a.f + col, Elem<uint16_t>::pack(du));
        }
      }
    }
    if (half == 0) __syncthreads();
  }
}

template <int BM, int BN, int KIND, int B_KC, int EPI>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  dim3 grid;
  if (KIND == 0) {
    const int ncols = (EPI == EPI_SWIGLU_FWD) ? a.f : a.N;
    const int bn = (EPI == EPI_SWIGLU_FWD) ? BN / 2 : BN;
    const int64_t tiles = (a.max_rows + BM - 1) / BM + a.E + (a.shared_rows + BM - 1) / BM;
    grid = dim3((unsigned)tiles, (ncols + bn - 1) / bn, 1);
  } else {
    const int ng = a.E + (a.has_shared ? 1 : 0);
    grid = dim3(((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN), ng, 1);
  }
  if (grid.x == 0 || grid.y == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, KIND, B_KC, EPI>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}


template <int BM, int BN>
hipError_t launch_tiles(const GemmArgs& a, hipStream_t st) {
  if (a.kind == 1) return launch_t<BM, BN, 1, 0, EPI_STORE>(a, st);
  if (a.b_kcontig) {
    switch (a.epi) {
      case EPI_STORE: return launch_t<BM, BN, 0, 1, EPI_STORE>(a, st);
      case EPI_RELU_FWD: return launch_t<BM, BN, 0, 1, EPI_RELU_FWD>(a, st);
      case EPI_SWIGLU_FWD: return launch_t<BM, BN, 0, 1, EPI_SWIGLU_FWD>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.epi) {
    case EPI_STORE: return launch_t<BM, BN, 0, 0, EPI_STORE>(a, st);
    case EPI_RELU_BWD: return launch_t<BM, BN, 0, 0, EPI_RELU_BWD>(a, st);
    case EPI_SWIGLU_BWD: return launch_t<BM, BN, 0, 0, EPI_SWIGLU_BWD>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Tile choice: 256x256 (each wave 128x128, one workgroup per CU) when the
// groups are large enough to fill it on average; 128x128 otherwise (small
// expert batches, where the weights stream from HBM and the row tile is mostly
// padding).
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t st) {
  const int64_t groups = a.E > 0 ? a.E : 1;
  const int64_t avg_rows = (a.kind == 0 ? a.max_rows : a.max_rows) / groups;
  const bool big = avg_rows >= 256 && (a.kind == 0 ? a.N >= 256 : (a.M >= 256 && a.N >= 256));
  return big ? launch_tiles<256, 256>(a, st) : launch_tiles<128, 128>(a, st);
}

}  // namespace moe
