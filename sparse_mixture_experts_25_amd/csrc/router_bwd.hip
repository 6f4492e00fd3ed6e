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
// so summing the partial products with fp32 accumulation on
// v_mfma_f32_32x32x16_bf16 gives an fp32-accurate result:
//   dW_r[e][j] = sum_t (g_hi + g_mid + g_lo)[t][e] * x[t][j]   (x is bf16: 3 products)
//   dx_r[t][j] = sum_e g[t][e] * W[e][j] with the cross terms hi.hi, hi.mid
//                and mid.hi; the dropped ones (hi.lo, mid.mid, lo.hi and
//                smaller) are at most about 2^-16 of each product. dx_r only
//                enters the input gradient, which is rounded to bf16 (2^-9).
// Tiles are staged through LDS (fp32 loaded, split, written as bf16); the
// fragment reads are those of the expert matmuls. No atomics: dW_r is summed
// over fixed token chunks into partial buffers and then in a fixed order.
#include "internal.h"
#include "mfma_tile.h"

namespace moe {

namespace {

constexpr int kT = 64;  // workgroup tile (rows and columns)
constexpr int kK = 32;  // contraction step

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

// Split 8 fp32 values and store the three 16-byte bf16 vectors at offset o of
// the three part tiles.
__device__ __forceinline__ void split_store(const float* v, uint16_t* t0, uint16_t* t1, uint16_t* t2, int o) {
  u128 a, b, c;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const Split3 s0 = split3(v[2 * i]), s1 = split3(v[2 * i + 1]);
    a.w[i] = (uint32_t)s0.h | ((uint32_t)s1.h << 16);
    b.w[i] = (uint32_t)s0.m | ((uint32_t)s1.m << 16);
    c.w[i] = (uint32_t)s0.l | ((uint32_t)s1.l << 16);
  }
  st128(t0 + o, a);
  st128(t1 + o, b);
  st128(t2 + o, c);
}

// part[c][e][j] = sum over the tokens of chunk c of g[t][e] * x[t][j].
// Workgroup: 64 experts x 64 columns; four waves of 32 x 32.
__global__ __launch_bounds__(256) void router_dw_kernel(const float* __restrict__ g, const uint16_t* __restrict__ x,
                                                        int T, int E, int d, int chunk, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t As[3][kK * kT];  // [k = t][m = e], per split term
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kK * kT];     // [k = t][n = j]
  const int nN = (d + kT - 1) / kT;
  const int mb = blockIdx.x / nN, nb = blockIdx.x % nN;
  const int t0 = blockIdx.y * chunk, t1 = min(T, t0 + chunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int kr = tid >> 3, c = tid & 7;  // this thread's row and 8-wide chunk of both tiles
  floatx16 acc = {};
  // the next step's operands are loaded into registers during this step's
  // matrix work
  float v[8];
  u128 xv;
  auto load = [&](int k0) {
    const int t = k0 + kr;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = mb * kT + 8 * c + i;
      v[i] = (t < t1 && e < E) ? g[(int64_t)t * E + e] : 0.0f;
    }
    const int j = nb * kT + 8 * c;
    xv = (t < t1 && j < d) ? ld128(x + (int64_t)t * d + j) : zero128();
  };
  if (t0 < t1) load(t0);
  for (int k0 = t0; k0 < t1; k0 += kK) {
    __syncthreads();  // the previous step's fragments are read
    split_store(v, As[0], As[1], As[2], mn_off<kT>(kr, c));
    st128(Bs + mn_off<kT>(kr, c), xv);
    __syncthreads();
    if (k0 + kK < t1) load(k0 + kK);
#pragma unroll
    for (int s = 0; s < kK / 16; ++s) {
      const bf16x8 b = frag_mn<kT>(Bs, wn * 32, s, lane);
#pragma unroll
      for (int p = 0; p < 3; ++p)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_mn<kT>(As[p], wm * 32, s, lane), b, acc, 0, 0, 0);
    }
  }
  float* out = part + (int64_t)blockIdx.y * E * d;
  const int n = nb * kT + wn * 32 + (lane & 31);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int m = mb * kT + wm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    if (m < E && n < d) out[(int64_t)m * d + n] = acc[e];
  }
}

// dxr[t][j] = sum_e g[t][e] * W[e][j]. Workgroup: 64 tokens x 64 columns.
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ g, const float* __restrict__ w,
                                                        int T, int E, int d, float* __restrict__ dxr) {
  __shared__ __attribute__((aligned(16))) uint16_t As[3][kT * kK];  // [m = t][k = e] (K-contiguous)
  __shared__ __attribute__((aligned(16))) uint16_t Bs[3][kK * kT];  // [k = e][n = j] (lo terms unused)
  const int nN = (d + kT - 1) / kT;
  const int mb = blockIdx.x / nN, nb = blockIdx.x % nN;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int ar = tid >> 2, ac = tid & 3;  // A: row (token) and 8-wide e chunk
  const int br = tid >> 3, bc = tid & 7;  // B: row (expert) and 8-wide column chunk
  floatx16 acc = {};
  float va[8], vb[8];
  auto load = [&](int k0) {
    const int t = mb * kT + ar;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = k0 + 8 * ac + i;
      va[i] = (t < T && e < E) ? g[(int64_t)t * E + e] : 0.0f;
    }
    const int e = k0 + br, j = nb * kT + 8 * bc;
    if (e < E && j < d) {
      const float4 p = *reinterpret_cast<const float4*>(w + (int64_t)e * d + j);
      const float4 q = *reinterpret_cast<const float4*>(w + (int64_t)e * d + j + 4);
      vb[0] = p.x; vb[1] = p.y; vb[2] = p.z; vb[3] = p.w;
      vb[4] = q.x; vb[5] = q.y; vb[6] = q.z; vb[7] = q.w;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) vb[i] = 0.0f;
    }
  };
  if (E > 0) load(0);
  for (int k0 = 0; k0 < E; k0 += kK) {
    __syncthreads();
    split_store(va, As[0], As[1], As[2], kc_off<kK>(ar, ac));
    split_store(vb, Bs[0], Bs[1], Bs[2], mn_off<kT>(br, bc));
    __syncthreads();
    if (k0 + kK < E) load(k0 + kK);
#pragma unroll
    for (int s = 0; s < kK / 16; ++s) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        fa[p] = frag_kc<kK>(As[p], wm * 32, s, lane);
        fb[p] = frag_mn<kT>(Bs[p], wn * 32, s, lane);
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0], fb[0], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[0], fb[1], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[1], fb[0], acc, 0, 0, 0);
    }
  }
  const int n = nb * kT + wn * 32 + (lane & 31);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int m = mb * kT + wm * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
    if (m < T && n < d) dxr[(int64_t)m * d + n] = acc[e];
  }
}

// Operands of dx_r as one contraction of length Kp = router_dx_k(E):
//   gx[t]  = [g_hi | g_hi | g_mid | 0 ...]      (bf16 [T][Kp])
//   wsp    = [W_hi ; W_mid ; W_hi ; 0 ...]      (bf16 [Kp][d])
// so gx[t] . wsp[:, j] = hi.hi + hi.mid + mid.hi of g[t] . W[:, j]. One
// thread per 8 output elements; also writes the single group's row range.
__global__ __launch_bounds__(256) void router_dx_split_kernel(const float* __restrict__ g, const float* __restrict__ w,
                                                              int T, int E, int d, int kp, uint16_t* __restrict__ gx,
                                                              uint16_t* __restrict__ wsp, int32_t* __restrict__ offs2) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t ng = (int64_t)T * (kp / 8);
  if (u == 0) {
    offs2[0] = 0;
    offs2[1] = T;
  }
  if (u < ng) {
    const int t = (int)(u / (kp / 8)), c0 = (int)(u % (kp / 8)) * 8;
    u128 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t h[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int c = c0 + 2 * i + q;
        const int e = c % E, part = c / E;
        uint16_t v = 0;
        if (part < 3) {
          const Split3 sp = split3(g[(int64_t)t * E + e]);
          v = part == 2 ? sp.m : sp.h;
        }
        h[q] = v;
      }
      o.w[i] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
    }
    st128(gx + (int64_t)t * kp + c0, o);
    return;
  }
  const int64_t v = u - ng;
  if (v >= (int64_t)kp * (d / 8)) return;
  const int r = (int)(v / (d / 8)), j0 = (int)(v % (d / 8)) * 8;
  const int e = r % E, part = r / E;
  u128 o = zero128();
  if (part < 3) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const Split3 a = split3(w[(int64_t)e * d + j0 + 2 * i]), b = split3(w[(int64_t)e * d + j0 + 2 * i + 1]);
      const uint16_t x0 = part == 1 ? a.m : a.h, x1 = part == 1 ? b.m : b.h;
      o.w[i] = (uint32_t)x0 | ((uint32_t)x1 << 16);
    }
  }
  st128(wsp + (int64_t)r * d + j0, o);
}

}  // namespace

// dx_r on the grouped matmul: one ragged-M group of T rows, K = Kp, N = d,
// B MN-contiguous, fp32 output.
hipError_t launch_router_dx_gemm(const RouterGradArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  const int kp = router_dx_k(a.E);
  const int64_t n = (int64_t)a.T * (kp / 8) + (int64_t)kp * (a.d / 8);
  hipLaunchKernelGGL(router_dx_split_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.dlogits,
                     a.w_router, a.T, a.E, a.d, kp, a.gx, a.wsplit, a.offs2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  GemmArgs g{};
  g.kind = 0;
  g.epi = EPI_STORE_F32;
  g.b_kcontig = 0;
  g.M = a.T;
  g.N = a.d;
  g.K = kp;
  g.offsets = a.offs2;
  g.E = 1;
  g.shared_rows = 0;
  g.has_shared = 0;
  g.max_rows = a.T;
  g.order = nullptr;
  g.A = a.gx;
  g.lda = kp;
  g.B = a.wsplit;
  g.ldb = a.d;
  g.strideB = 0;
  g.C = a.dx_router;
  g.ldc = a.d;
  return launch_gemm_bf16(g, st);
}

hipError_t launch_router_dw_mfma(const float* g, const uint16_t* x, int T, int E, int d, int chunk, int nsplit,
                                 float* part, hipStream_t st) {
  const int tiles = ((E + kT - 1) / kT) * ((d + kT - 1) / kT);
  if (tiles == 0 || nsplit == 0) return hipSuccess;
  hipLaunchKernelGGL(router_dw_kernel, dim3(tiles, nsplit), dim3(256), 0, st, g, x, T, E, d, chunk, part);
  return hipGetLastError();
}

hipError_t launch_router_dx_mfma(const float* g, const float* w, int T, int E, int d, float* dxr, hipStream_t st) {
  const int tiles = ((T + kT - 1) / kT) * ((d + kT - 1) / kT);
  if (tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(router_dx_kernel, dim3(tiles), dim3(256), 0, st, g, w, T, E, d, dxr);
  return hipGetLastError();
}

}  // namespace moe
