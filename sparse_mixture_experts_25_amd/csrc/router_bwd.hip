// Router weight and input gradients on the matrix cores (bf16 activations).
//
// [SW] = "Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散"
// (ta-paperlens.web.app), eq. (1): h = W_r x, so for the logit gradient
// g = dL/dh the router weight gradient is g^T x (summed over tokens) and the
// router's share of the input gradient is g W_r.
//
// Both products are fp32 results. The fp32 operands are split exactly into
// three bf16 terms, v = hi + mid + lo (hi = bf16(v), mid = bf16(v - hi),
// lo = bf16(v - hi - mid); each subtraction is exact, and the three terms
// carry the full 24-bit significand). A bf16 x bf16 product is exact in fp32,
// so the grouped matmul kernel (fp32 accumulation) gives fp32-accurate results:
//   dW_r[e][j] = sum_t (g_hi + g_mid + g_lo)[t][e] * x[t][j]   (x is bf16: 3 bands)
//   dx_r[t][j] = sum_e g[t][e] * W[e][j] with the cross terms hi.hi, hi.mid
//                and mid.hi; the dropped ones (hi.lo, mid.mid, lo.hi and
//                smaller) are at most about 2^-16 of each product. dx_r only
//                enters the input gradient, which is rounded to bf16 (2^-9).
// Each product is one contraction over split operands of width 3E (rounded up
// to 8): dW_r runs on the weight-gradient (ragged-K) path over fixed token
// chunks with fp32 partials summed in a fixed order; dx_r runs on the
// ragged-M path as a single group. No atomics.
#include "internal.h"
#include "mfma_tile.h"

namespace moe {

namespace {


// Split operands, all of width Kp = router_dx_k(E):
//   gx[t]  = [g_hi | g_hi | g_mid | 0 ...]      dx_r:   gx[t] . wsp[:, j]
//   wsp    = [W_hi ; W_mid ; W_hi ; 0 ...]              = hi.hi + hi.mid + mid.hi
//   gw[t]  = [g_hi | g_mid | g_lo | 0 ...]      dW_r:   sum_t gw[t][p E + e] x[t][j],
//                                                       summed over the three bands p
// One thread per 8 elements; the weight threads also write the row ranges
// (split_router_weights). bf16 layers with the plain gates get all of it from
// the dlogits kernel instead.
__global__ __launch_bounds__(256) void router_split_kernel(const float* __restrict__ g, const float* __restrict__ w,
                                                           int T, int E, int d, int kp, int nsw, int chunk,
                                                           uint16_t* __restrict__ gx, uint16_t* __restrict__ gw,
                                                           uint16_t* __restrict__ wsp, int32_t* __restrict__ offs) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t ng = (int64_t)T * (kp / 8);
  if (u < ng) {
    const int t = (int)(u / (kp / 8)), c0 = (int)(u % (kp / 8)) * 8;
    u128 ox, ow;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t hx[2], hw[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = c0 + 2 * i + q;
        const int e = c % E, band = c / E;
        hx[q] = hw[q] = 0;
        if (band < 3) {
          const Split3 sp = split3(g[(int64_t)t * E + e]);
          hx[q] = band == 2 ? sp.m : sp.h;
          hw[q] = band == 0 ? sp.h : band == 1 ? sp.m : sp.l;
        }
      }
      ox.w[i] = (uint32_t)hx[0] | ((uint32_t)hx[1] << 16);
      ow.w[i] = (uint32_t)hw[0] | ((uint32_t)hw[1] << 16);
    }
    st128(gx + (int64_t)t * kp + c0, ox);
    st128(gw + (int64_t)t * kp + c0, ow);
    return;
  }
  split_router_weights(u - ng, w, E, d, kp, wsp, T, nsw, chunk, offs);
}

// dW_r[e][j] = sum over chunks c and bands p of part[c][p E + e][j], in that
// fixed order.
__global__ __launch_bounds__(256) void router_dw_sum_kernel(const float* __restrict__ part, int nsw, int E, int d,
                                                            int kp, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)E * d) return;
  const int64_t e = i / d, j = i % d;
  float s = 0.0f;
  for (int c = 0; c < nsw; ++c)
#pragma unroll
    for (int p = 0; p < 3; ++p) s += part[((int64_t)c * kp + p * E + e) * d + j];
  out[i] = s;
}

}  // namespace

// Token chunks of dW_r. Every chunk writes a kp x d fp32 partial that the
// sum kernel reads back, so chunks are as few as keep the CUs busy:
//  - large products (at least 512 workgroups' worth of 256x256 tiles over
//    256-token chunks): about 512 workgroups of 256x256 tiles, partials capped
//    at 128 MB, chunks of at least 2048 tokens (fine-grained top-8 shape: 16
//    chunks; DeepSeek-V3 shape: 6);
//  - small products: 128x128 tiles (the matmul picks them when 256x256 tiles
//    would leave CUs idle), about 256 workgroups, chunks of at least 1024 tokens.
int router_dw_splits(int T, int E, int d) {
  const int64_t kp = router_dx_k(E);
  const int64_t big_tiles = ((kp + 255) / 256) * (((int64_t)d + 255) / 256);
  int64_t ns;
  if (big_tiles * (((int64_t)T + 255) / 256) >= 512) {
    ns = (512 + big_tiles - 1) / big_tiles;
    const int64_t mem = (int64_t(128) << 20) / (kp * (int64_t)d * 4 > 0 ? kp * (int64_t)d * 4 : 1);
    if (ns > mem) ns = mem;
    const int64_t by_t = (int64_t)T / 2048;
    if (ns > by_t) ns = by_t;
  } else {
    const int64_t tiles = ((kp + 127) / 128) * (((int64_t)d + 127) / 128);
    ns = (256 + tiles - 1) / tiles;
    const int64_t by_t = (int64_t)T / 1024;
    if (ns > by_t) ns = by_t;
  }
  return (int)(ns < 1 ? 1 : ns);
}

// Split operands (both layouts), dW_r on the weight-gradient matmul (one
// group per token chunk, fp32 partials), then the fixed-order sum.
hipError_t launch_router_dw_gemm(const RouterGradArgs& a, hipStream_t st) {
  const int64_t ed = (int64_t)a.E * a.d;
  if (a.T == 0) {
    hipLaunchKernelGGL(router_dw_sum_kernel, dim3((unsigned)((ed + 255) / 256)), dim3(256), 0, st, a.ws_partial, 0,
                       a.E, a.d, router_dx_k(a.E), a.dw_router);
    return hipGetLastError();
  }
  const int kp = router_dx_k(a.E);
  const int nsw = router_dw_splits(a.T, a.E, a.d);
  const int chunk = (a.T + nsw - 1) / nsw;
  hipError_t e;
  if (!a.split_done) {  // else the dlogits kernel wrote every split operand and the row ranges
    const int64_t nw = (int64_t)kp * (a.d / 8) > nsw + 1 ? (int64_t)kp * (a.d / 8) : nsw + 1;
    const int64_t nthreads = (int64_t)a.T * (kp / 8) + nw;
    hipLaunchKernelGGL(router_split_kernel, dim3((unsigned)((nthreads + 255) / 256)), dim3(256), 0, st, a.dlogits,
                       a.w_router, a.T, a.E, a.d, kp, nsw, chunk, a.gx, a.gw, a.wsplit, a.offs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  GemmArgs g{};
  g.kind = 1;
  g.epi = EPI_STORE_F32;
  g.M = kp;
  g.N = a.d;
  g.offsets = a.offs + 2;
  g.E = nsw;
  g.max_rows = a.T;
  g.order = nullptr;
  g.A = a.gw;
  g.lda = kp;
  g.B = a.x;
  g.ldb = a.d;
  g.C = a.ws_partial;
  g.ldc = a.d;
  g.strideC = (int64_t)kp * a.d;
  if ((e = launch_gemm_bf16(g, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(router_dw_sum_kernel, dim3((unsigned)((ed + 255) / 256)), dim3(256), 0, st, a.ws_partial, nsw,
                     a.E, a.d, kp, a.dw_router);
  return hipGetLastError();
}

// dx_r on the grouped matmul: one ragged-M group of T rows, K = Kp, N = d,
// B MN-contiguous. Either an fp32 dx_router, or (a.dx set) the layer's input
// gradient dx = dy + sum_kept dX_perm[slot] + dx_r (+ dx_shared) in the
// epilogue, in the order of the separate unpermute pass, so dx_r never goes to
// memory. Needs the split operands of launch_router_dw_gemm (same stream,
// launched before).
hipError_t launch_router_dx_gemm(const RouterGradArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int kp = router_dx_k(a.E);
  GemmArgs g{};
  g.kind = 0;
  g.epi = a.dx ? EPI_UNPERMUTE : EPI_STORE_F32;
  g.b_kcontig = 0;
  g.M = a.T;
  g.N = a.d;
  g.K = kp;
  g.offsets = a.offs;
  g.E = 1;
  g.max_rows = a.T;
  g.order = nullptr;
  g.A = a.gx;
  g.lda = kp;
  g.B = a.wsplit;
  g.ldb = a.d;
  g.C = a.dx ? a.dx : a.dx_router;
  g.ldc = a.d;
  if (a.dx) {
    g.X = a.dy;
    g.ldx = a.d;
    g.slot = a.slot;
    g.slot_k = a.k;
    g.Y = a.dX_perm;
    g.Y_sh = a.dX_sh;
  }
  return launch_gemm_bf16(g, st);
}

}  // namespace moe
