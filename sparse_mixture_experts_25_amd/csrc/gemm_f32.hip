// fp32 grouped matmuls (SIMT) for layers stored in fp32.
//
// Same problem definition, tile decoding and fused epilogues as the bf16
// matrix-core kernels (ragged-M for the forward and input-gradient matmuls,
// ragged-K for the weight gradients), computed with plain fp32 fused
// multiply-adds: 64x64 output tiles, 16-deep K steps staged in LDS (k-major),
// 4x4 outputs per thread. The fp32 layers are small; this path is about
// exactness (fp32 accumulation), not throughput.
#include "gemm_common.h"

namespace moe {

namespace {

constexpr int BM = 64, BN = 64, BK = 16;
constexpr int kP = 68;  // padded LDS row (floats)

template <int KIND, int B_KC, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) float As[BK][kP];
  __shared__ __attribute__((aligned(16))) float Bs[BK][kP];
  __shared__ __attribute__((aligned(16))) float Cs[BM][BN + 1];
  __shared__ __attribute__((aligned(16))) int info[12];
  const int tid = threadIdx.x;
  const int tm = tid / 16, tn = tid % 16;

  int g, rows, mrow0 = 0, nb, mb = 0;
  int64_t r0;
  if (KIND == 0) {
    const int ncols = (EPI == EPI_SWIGLU_FWD) ? a.f : a.N;
    const int bn = (EPI == EPI_SWIGLU_FWD) ? BN / 2 : BN;
    TileInfo ti;
    if (!locate_ragged_m<BM>(a, (ncols + bn - 1) / bn, 8, info, ti, nb)) return;
    g = ti.g; r0 = ti.r0; rows = ti.rows; mrow0 = ti.m0;
  } else {
    // groups in the given order (largest first), tiles of one group
    // consecutive with the row block fastest
    const int nM = (a.M + BM - 1) / BM, nN = (a.N + BN - 1) / BN;
    const int64_t per_g = (int64_t)nM * nN;
    const int rank = (int)(blockIdx.x / per_g);
    const int t = (int)(blockIdx.x % per_g);
    g = a.order ? a.order[rank] : rank;
    mb = t % nM;
    nb = t / nM;
    if (g < a.E) {
      r0 = a.offsets[g];
      rows = a.offsets[g + 1] - a.offsets[g];
    } else {
      r0 = 0;
      rows = a.shared_rows;
    }
  }
  const bool sh = g >= a.E;
  const float* Ab = reinterpret_cast<const float*>(sh ? a.A_sh : a.A);
  const float* Bb = reinterpret_cast<const float*>(sh ? a.B_sh : a.B);
  if (!sh && KIND == 0) Bb += (int64_t)g * a.strideB;
  const int K = (KIND == 0) ? a.K : rows;

  float acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += BK) {
    __syncthreads();
    for (int u = tid; u < BM * BK; u += 256) {
      const int r = u / BK, kk = u % BK;  // A: tile row r, k index kk
      const int k = k0 + kk;
      float v = 0.0f;
      if (KIND == 0) {
        if (r < rows - mrow0 && k < K) {
          const int64_t row = r0 + mrow0 + r;
          v = Ab[(sh || !a.a_rows ? row : (int64_t)a.a_rows[row]) * a.lda + k];
        }
      } else {
        const int m = mb * BM + r;
        if (m < a.M && k < K) v = Ab[(r0 + k) * a.lda + m];
      }
      As[kk][r] = v;
    }
    for (int u = tid; u < BN * BK; u += 256) {
      const int c = u / BK, kk = u % BK;
      const int k = k0 + kk;
      float v = 0.0f;
      if (KIND == 0) {
        if (B_KC) {
          int64_t src;
          bool ok;
          if (EPI == EPI_SWIGLU_FWD) {
            const int hc = nb * (BN / 2) + (c < BN / 2 ? c : c - BN / 2);
            ok = hc < a.f && k < K;
            src = (int64_t)(c < BN / 2 ? hc : a.f + hc) * a.ldb + k;
          } else {
            const int n = nb * BN + c;
            ok = n < a.N && k < K;
            src = (int64_t)n * a.ldb + k;
          }
          if (ok) v = Bb[src];
        } else {
          const int n = nb * BN + c;
          if (n < a.N && k < K) v = Bb[(int64_t)k * a.ldb + n];
        }
      } else {
        const int n = nb * BN + c;
        if (n < a.N && k < K) {
          const int64_t row = r0 + k;
          v = Bb[(sh || !a.b_rows ? row : (int64_t)a.b_rows[row]) * a.ldb + n];
        }
      }
      Bs[kk][c] = v;
    }
    __syncthreads();
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], bv[4];
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tm * 4 + i];
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tn * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
  }
  __syncthreads();
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) Cs[tm * 4 + i][tn * 4 + j] = acc[i][j];
  __syncthreads();

  float* C = reinterpret_cast<float*>(sh ? a.C_sh : a.C);
  float* C2 = reinterpret_cast<float*>(sh ? a.C2_sh : a.C2);
  const float* X = reinterpret_cast<const float*>(sh ? a.X_sh : a.X);

  if (EPI == EPI_SWIGLU_FWD) {
    for (int u = tid; u < BM * (BN / 2); u += 256) {
      const int m = u / (BN / 2), j = u % (BN / 2);
      const int hc = nb * (BN / 2) + j;
      if (m >= rows - mrow0 || hc >= a.f) continue;
      const int64_t row = r0 + mrow0 + m;
      const float gv = Cs[m][j], uv = Cs[m][BN / 2 + j];
      C[row * a.ldc + hc] = gv;
      C[row * a.ldc + a.f + hc] = uv;
      C2[row * a.ldc2 + hc] = silu_f(gv) * uv;
    }
    return;
  }
  for (int u = tid; u < BM * BN; u += 256) {
    const int m = u / BN, n = u % BN;
    const float v = Cs[m][n];
    if (KIND == 1) {
      const int mm = mb * BM + m, nn = nb * BN + n;
      if (mm >= a.M || nn >= a.N) continue;
      float* Cg = sh ? C : C + (int64_t)g * a.strideC;
      Cg[(int64_t)mm * a.ldc + nn] = v;
      continue;
    }
    const int col = nb * BN + n;
    if (m >= rows - mrow0 || col >= a.N) continue;
    const int64_t row = r0 + mrow0 + m;
    if (EPI == EPI_STORE) {
      C[row * a.ldc + col] = v;
    } else if (EPI == EPI_RELU_FWD) {
      if (C) C[row * a.ldc + col] = v;  // pre-activation only if asked for
      C2[row * a.ldc2 + col] = fmaxf(v, 0.0f);
    } else if (EPI == EPI_RELU_BWD) {
      C[row * a.ldc + col] = X[row * a.ldx + col] > 0.0f ? v : 0.0f;
    } else if (EPI == EPI_SWIGLU_BWD) {
      const float gs = X[row * a.ldx + col], us = X[row * a.ldx + a.f + col];
      const float s = 1.0f / (1.0f + expf(-gs));
      C[row * a.ldc + a.f + col] = v * gs * s;
      C[row * a.ldc + col] = v * us * s * (1.0f + gs * (1.0f - s));
    }
  }
}

template <int KIND, int B_KC, int EPI>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  int64_t n;
  if (KIND == 0) {
    const int ncols = (EPI == EPI_SWIGLU_FWD) ? a.f : a.N;
    const int bn = (EPI == EPI_SWIGLU_FWD) ? BN / 2 : BN;
    n = raster_grid(row_tile_bound(a, BM), (ncols + bn - 1) / bn);
  } else {
    const int ng = a.E + (a.has_shared ? 1 : 0);
    n = (int64_t)ng * ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  }
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)n);
  hipLaunchKernelGGL((gemm_f32_kernel<KIND, B_KC, EPI>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace


hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t st) {
  if (a.kind == 1) return launch_t<1, 0, EPI_STORE>(a, st);
  if (a.b_kcontig) {
    switch (a.epi) {
      case EPI_STORE: return launch_t<0, 1, EPI_STORE>(a, st);
      case EPI_RELU_FWD: return launch_t<0, 1, EPI_RELU_FWD>(a, st);
      case EPI_SWIGLU_FWD: return launch_t<0, 1, EPI_SWIGLU_FWD>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.epi) {
    case EPI_STORE: return launch_t<0, 0, EPI_STORE>(a, st);
    case EPI_RELU_BWD: return launch_t<0, 0, EPI_RELU_BWD>(a, st);
    case EPI_SWIGLU_BWD: return launch_t<0, 0, EPI_SWIGLU_BWD>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace moe
