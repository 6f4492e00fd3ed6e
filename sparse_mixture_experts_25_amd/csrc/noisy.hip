// Noisy top-k gating: importance and load losses and the logit gradient.
//
// [WIKI] = "Mixture-of-Experts" (notes.yuuk.io), findings on Shazeer et al.
// 2017: top-k gating with noisy softmax, trained with an importance loss
// (dispersion of each expert's summed softmax weight) and a load loss
// (dispersion of a smoothed load estimate), total loss = main + alpha
// (importance + load). Written out as that paper defines them:
//   H = h + eps * softplus(n) (clean logits h, noise logits n = the second E
//   rows of the router, eps an input); gates G = softmax over the top-k of H;
//   Importance_e = sum_t G[t, e]; Load_e = sum_t Phi((h[t, e] - r[t, e]) /
//   softplus(n[t, e])) with r the k-th largest H of the token leaving e out
//   (the (k+1)-th key when e is selected, the k-th otherwise);
//   aux = alpha (CV^2(Importance) + CV^2(Load)), CV^2 = variance / mean^2.
// Kernels:
//   noisy_stats_kernel   32 tokens per workgroup (one wave per 8 tokens, lane =
//                        expert): per-block sums of G and of the load terms,
//                        the four waves combined in a fixed order
//   noisy_final_kernel   one workgroup: Importance, Load, the loss, and the
//                        per-expert gradient coefficients alpha dCV^2/dv_e
//   noisy_dlogits_kernel one wave per token: [dL/dh | dL/dn] from the gate
//                        gradient, the importance coefficients (through the
//                        softmax-over-top-k Jacobian) and the load terms (to
//                        the expert and to its rival)
// Every sum runs in a fixed order; there are no atomics.
#include "common.h"
#include "gate_math.h"
#include "internal.h"

// H is one fp32 multiply and one fp32 add, as in the routing that selected on it
#pragma clang fp contract(off)

namespace moe {

namespace {

constexpr int kNzTok = 32;  // tokens per stats block
constexpr int kNzFin = 1024;

__device__ __forceinline__ float sigmoid_f(float v) { return 1.0f / (1.0f + __expf(-v)); }

// One token's keys H and the top-(k+1) cut: c_k / i_k (k-th selected) and
// c_k1 / i_k1 (first unselected), ordering by (H desc, index asc).
template <int QE>
struct TokenCut {
  float h[QE], n[QE], sp[QE], ep[QE], H[QE];
  float ck, ck1;
  int ik, ik1;
  __device__ void load(const float* __restrict__ logits2, const float* __restrict__ noise, int64_t t, int E, int k,
                       int lane) {
#pragma unroll
    for (int q = 0; q < QE; ++q) {
      const int e = lane + 64 * q;
      if (e < E) {
        h[q] = logits2[t * 2 * E + e];
        n[q] = logits2[t * 2 * E + E + e];
        ep[q] = noise[t * E + e];
        sp[q] = softplus_c(n[q]);
        const float prod = ep[q] * sp[q];
        H[q] = h[q] + prod;
      } else {
        h[q] = n[q] = sp[q] = ep[q] = 0.0f;
        H[q] = -__builtin_inff();
      }
    }
    uint32_t taken = 0;
    ck = ck1 = 0.0f;
    ik = ik1 = 0;
    const int rounds = k < E ? k + 1 : k;
    for (int r = 0; r < rounds; ++r) {
      float bk = -__builtin_inff();
      int be = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < QE; ++q) {
        const int e = lane + 64 * q;
        if (e < E && !(taken & (1u << q)) && (H[q] > bk || be == 0x7fffffff)) {
          bk = H[q];
          be = e;
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        const float ok = __shfl_xor(bk, o, 64);
        const int oe = __shfl_xor(be, o, 64);
        if (ok > bk || (ok == bk && oe < be)) {
          bk = ok;
          be = oe;
        }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      if (r == k - 1) {
        ck = bk;
        ik = be;
      }
      if (r == k) {
        ck1 = bk;
        ik1 = be;
      }
    }
  }
  __device__ bool selected(int q, int e) const { return H[q] > ck || (H[q] == ck && e <= ik); }
};

template <int QE>
__global__ __launch_bounds__(256) void noisy_stats_kernel(const float* __restrict__ logits2,
                                                          const float* __restrict__ noise,
                                                          const int32_t* __restrict__ topk_idx,
                                                          const float* __restrict__ topk_w, int T, int E, int k,
                                                          float* __restrict__ partG, float* __restrict__ partP) {
  __shared__ float sG[4][QE * 64], sP[4][QE * 64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float accG[QE], accP[QE];
#pragma unroll
  for (int q = 0; q < QE; ++q) accG[q] = accP[q] = 0.0f;
  for (int i = 0; i < kNzTok / 4; ++i) {
    const int64_t t = (int64_t)blockIdx.x * kNzTok + wave * (kNzTok / 4) + i;
    if (t >= T) break;
    for (int r = 0; r < k; ++r) {
      const int er = topk_idx[t * k + r];
      const float wr = topk_w[t * k + r];
#pragma unroll
      for (int q = 0; q < QE; ++q)
        if (er == lane + 64 * q) accG[q] += wr;
    }
    if (k >= E) continue;  // every expert always selected: no load term
    TokenCut<QE> c;
    c.load(logits2, noise, t, E, k, lane);
#pragma unroll
    for (int q = 0; q < QE; ++q) {
      const int e = lane + 64 * q;
      if (e >= E) continue;
      const float rival = c.selected(q, e) ? c.ck1 : c.ck;
      const float d = c.h[q] - rival;
      const float P = c.sp[q] > 0.0f ? 0.5f * erfcf(-(d / c.sp[q]) * 0.70710678118654752f)
                                     : (d > 0.0f ? 1.0f : (d < 0.0f ? 0.0f : 0.5f));
      accP[q] += P;
    }
  }
#pragma unroll
  for (int q = 0; q < QE; ++q) {
    sG[wave][q * 64 + lane] = accG[q];
    sP[wave][q * 64 + lane] = accP[q];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    partG[(int64_t)blockIdx.x * E + e] = ((sG[0][e] + sG[1][e]) + sG[2][e]) + sG[3][e];
    partP[(int64_t)blockIdx.x * E + e] = ((sP[0][e] + sP[1][e]) + sP[2][e]) + sP[3][e];
  }
}

// Block partials -> Importance, Load; aux and the coefficients
// coef[e] = alpha dCV^2/dv_e = alpha 2 / (E mean^2) (v_e - mean - var / mean).
__global__ __launch_bounds__(kNzFin) void noisy_final_kernel(const float* __restrict__ partG,
                                                             const float* __restrict__ partP, int nblk, int T, int E,
                                                             int k, float alpha, float* __restrict__ gimp,
                                                             float* __restrict__ gload, float* __restrict__ aux_out) {
  __shared__ float s[2][kNzFin];
  __shared__ float v[2][512];
  __shared__ float stat[2][2];  // mean, var of importance and load
  const int tid = threadIdx.x;
  const int parts = kNzFin / E;
  if (tid < parts * E) {
    const int e = tid % E, p = tid / E;
    float a = 0.0f, b = 0.0f;
#pragma unroll 8
    for (int blk = p; blk < nblk; blk += parts) {
      a += partG[(int64_t)blk * E + e];
      b += partP[(int64_t)blk * E + e];
    }
    s[0][tid] = a;
    s[1][tid] = b;
  }
  __syncthreads();
  if (tid < E) {
    float a = 0.0f, b = 0.0f;
    for (int p = 0; p < parts; ++p) {
      a += s[0][p * E + tid];
      b += s[1][p * E + tid];
    }
    v[0][tid] = a;
    v[1][tid] = b;
  }
  __syncthreads();
  if (tid < 2) {  // two serial passes over E values each (E <= 256): mean, then variance
    float m = 0.0f;
    for (int e = 0; e < E; ++e) m += v[tid][e];
    m /= (float)E;
    float var = 0.0f;
    for (int e = 0; e < E; ++e) var += (v[tid][e] - m) * (v[tid][e] - m);
    stat[tid][0] = m;
    stat[tid][1] = var / (float)E;
  }
  __syncthreads();
  const bool load_on = k < E;
  if (tid < E) {
    for (int i = 0; i < 2; ++i) {
      const float m = stat[i][0], var = stat[i][1];
      float g = 0.0f;
      if (m != 0.0f && alpha != 0.0f && T > 0 && (i == 0 || load_on))
        g = alpha * 2.0f / ((float)E * m * m) * (v[i][tid] - m - var / m);
      (i == 0 ? gimp : gload)[tid] = g;
    }
  }
  if (tid == 0 && aux_out) {
    float a = 0.0f;
    if (alpha != 0.0f && T > 0) {
      if (stat[0][0] != 0.0f) a += stat[0][1] / (stat[0][0] * stat[0][0]);
      if (load_on && stat[1][0] != 0.0f) a += stat[1][1] / (stat[1][0] * stat[1][0]);
      a *= alpha;
    }
    aux_out[0] = a;
  }
}

template <int QE>
__global__ __launch_bounds__(256) void noisy_dlogits_kernel(const float* __restrict__ logits2,
                                                            const float* __restrict__ noise,
                                                            const int32_t* __restrict__ topk_idx,
                                                            const float* __restrict__ topk_w,
                                                            const float* __restrict__ dg,
                                                            const float* __restrict__ gimp,
                                                            const float* __restrict__ gload, int T, int E, int k,
                                                            float* __restrict__ dl2) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  TokenCut<QE> c;
  c.load(logits2, noise, t, E, k, lane);
  // gate path: softmax over the top-k of H, with the importance coefficients
  float sdot = 0.0f;
  for (int r = 0; r < k; ++r) {
    const int er = topk_idx[t * k + r];
    sdot += topk_w[t * k + r] * (dg[t * k + r] + gimp[er]);
  }
  float dh[QE], dn[QE];
#pragma unroll
  for (int q = 0; q < QE; ++q) dh[q] = dn[q] = 0.0f;
  for (int r = 0; r < k; ++r) {
    const int er = topk_idx[t * k + r];
    const float v = topk_w[t * k + r] * ((dg[t * k + r] + gimp[er]) - sdot);
#pragma unroll
    for (int q = 0; q < QE; ++q)
      if (er == lane + 64 * q) dh[q] += v;
  }
#pragma unroll
  for (int q = 0; q < QE; ++q) dn[q] = dh[q] * c.ep[q] * sigmoid_f(c.n[q]);
  // load path: to the expert, and (summed per rival) to its rival
  if (k < E) {
    float csel = 0.0f, cun = 0.0f;
#pragma unroll
    for (int q = 0; q < QE; ++q) {
      const int e = lane + 64 * q;
      if (e >= E || !(c.sp[q] > 0.0f)) continue;
      const bool sel = c.selected(q, e);
      const float z = (c.h[q] - (sel ? c.ck1 : c.ck)) / c.sp[q];
      const float pdf = __expf(-0.5f * z * z) * 0.39894228040143268f;
      const float co = gload[e] * pdf / c.sp[q];
      dh[q] += co;
      dn[q] += -co * z * sigmoid_f(c.n[q]);
      if (sel) csel += co;
      else cun += co;
    }
    csel = wave_sum(csel);
    cun = wave_sum(cun);
#pragma unroll
    for (int q = 0; q < QE; ++q) {
      const int e = lane + 64 * q;
      const float s = (e == c.ik1 ? csel : 0.0f) + (e == c.ik ? cun : 0.0f);
      dh[q] -= s;
      dn[q] -= s * c.ep[q] * sigmoid_f(c.n[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < QE; ++q) {
    const int e = lane + 64 * q;
    if (e < E) {
      dl2[t * 2 * E + e] = dh[q];
      dl2[t * 2 * E + E + e] = dn[q];
    }
  }
}

}  // namespace

int noisy_num_blocks(int T) { return (T + kNzTok - 1) / kNzTok; }

size_t noisy_workspace_bytes(int T, int E) {
  return ((size_t)noisy_num_blocks(T) * E * 2 + (size_t)E * 2 + 64) * sizeof(float);
}

// Stats and final pass; the coefficients land at the end of ws (gimp, gload).
hipError_t launch_noisy_stats(const NoisyArgs& a, float* aux_out, hipStream_t st) {
  const int nblk = noisy_num_blocks(a.T);
  float* partG = a.ws;
  float* partP = partG + (size_t)nblk * a.E;
  float* gimp = partP + (size_t)nblk * a.E;
  float* gload = gimp + a.E;
  const int qe = (a.E + 63) / 64;
  if (nblk > 0) {
#define MOE_NZ_STATS(Q)                                                                                           \
  hipLaunchKernelGGL(noisy_stats_kernel<Q>, dim3(nblk), dim3(256), 0, st, a.logits2, a.noise, a.topk_idx, a.topk_w, \
                     a.T, a.E, a.k, partG, partP)
    if (qe <= 1) MOE_NZ_STATS(1);
    else if (qe <= 2) MOE_NZ_STATS(2);
    else MOE_NZ_STATS(4);
#undef MOE_NZ_STATS
  }
  hipLaunchKernelGGL(noisy_final_kernel, dim3(1), dim3(kNzFin), 0, st, partG, partP, nblk, a.T, a.E, a.k, a.alpha,
                     gimp, gload, aux_out);
  return hipGetLastError();
}

hipError_t launch_noisy_dlogits(const NoisyArgs& a, const float* dg, float* dl2, hipStream_t st) {
  hipError_t e = launch_noisy_stats(a, nullptr, st);
  if (e != hipSuccess || a.T == 0) return e;
  const int nblk = noisy_num_blocks(a.T);
  const float* gimp = a.ws + (size_t)nblk * a.E * 2;
  const float* gload = gimp + a.E;
  const int qe = (a.E + 63) / 64;
#define MOE_NZ_DL(Q)                                                                                              \
  hipLaunchKernelGGL(noisy_dlogits_kernel<Q>, dim3((a.T + 3) / 4), dim3(256), 0, st, a.logits2, a.noise, a.topk_idx, \
                     a.topk_w, dg, gimp, gload, a.T, a.E, a.k, dl2)
  if (qe <= 1) MOE_NZ_DL(1);
  else if (qe <= 2) MOE_NZ_DL(2);
  else MOE_NZ_DL(4);
#undef MOE_NZ_DL
  return hipGetLastError();
}

}  // namespace moe
