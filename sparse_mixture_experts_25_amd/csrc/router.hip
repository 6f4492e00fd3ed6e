// Router forward: fp32 logits, gate and top-k in one kernel.
//
// [SW] = "Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散"
// (ta-paperlens.web.app), eq. (1) and the section on routing; [WIKI] =
// "Mixture-of-Experts" (notes.yuuk.io), bullets on sigmoid gating with a
// per-expert bias that only steers the selection.
//
// Each workgroup owns 32 tokens and all E experts. The logits are a SIMT fp32
// register-tiled product: every thread owns 4 tokens x EPT experts and walks
// the d_model axis in ascending order with one fused multiply-add per term, so
// each logit is the fixed-order fp32 sum the routing decision is defined on
// (no split of the sum, no matrix cores, no reassociation). The x chunk and the
// router weight chunk are staged through LDS, transposed so that the per-step
// reads are conflict-free. The gate then runs one wave per token.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kTT = 32;   // tokens per workgroup
constexpr int kKC = 32;   // d_model chunk staged in LDS

#pragma clang fp contract(off)
// Fixed-operation fp32 exponential: Cody-Waite range reduction (Cody & Waite,
// "Software Manual for the Elementary Functions", 1980) with ln2 split in a
// 15-bit head and an fp32 tail, then the degree-7 Taylor polynomial of e^r in
// Horner form with fused multiply-adds, then scaling by 2^n built from the
// exponent bits. Inputs above 86 give +inf and below -86 give 0, so no result
// is subnormal. Every operation is a correctly rounded IEEE fp32 operation.
__device__ __forceinline__ float exp_c(float x) {
  if (x > 86.0f) return __builtin_inff();
  if (x < -86.0f) return 0.0f;
  const float log2e = 1.44269504088896341f;
  const float ln2_hi = 0.693145751953125f;
  const float ln2_lo = 1.42860682030941723e-6f;
  float n = __builtin_rintf(x * log2e);
  float r = __builtin_fmaf(-n, ln2_hi, x);
  r = __builtin_fmaf(-n, ln2_lo, r);
  float p = 1.98412698412698413e-4f;             // 1/7!
  p = __builtin_fmaf(p, r, 1.38888888888888889e-3f);  // 1/6!
  p = __builtin_fmaf(p, r, 8.33333333333333333e-3f);  // 1/5!
  p = __builtin_fmaf(p, r, 4.16666666666666667e-2f);  // 1/4!
  p = __builtin_fmaf(p, r, 1.66666666666666667e-1f);  // 1/3!
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  int ni = (int)n;
  float scale = __uint_as_float((uint32_t)(ni + 127) << 23);
  return p * scale;
}

__device__ __forceinline__ float sigmoid_c(float h) {
  float e = exp_c(-h);
  float den = 1.0f + e;
  return 1.0f / den;
}
#pragma clang fp contract(on)

template <typename TX, int EPT>
__global__ __launch_bounds__(256) void router_fwd_kernel(
    const TX* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ offset,
    const float* __restrict__ sel_bias, float* __restrict__ probs, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int T, int d, int E, int k, int gate, int renorm) {
  // Ws[j][e] (router weight chunk, transposed) and later Ls[t][e] (logits).
  extern __shared__ float smem[];
  const int Ep = E + 1;
  float* Ws = smem;                       // kKC * Ep
  float* Xs = smem + kKC * Ep;            // kKC * (kTT + 4)
  constexpr int XP = kTT + 4;

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTT;
  const int tg = tid >> 5;   // token group: tokens tg*4 .. tg*4+3
  const int el = tid & 31;   // expert lane: experts el + 32*j

  float acc[4][EPT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[i][j] = 0.0f;

  for (int k0 = 0; k0 < d; k0 += kKC) {
    const int kc = min(kKC, d - k0);
    __syncthreads();
    // router weight chunk: E rows x kKC columns, read along the row (4 floats),
    // stored transposed
    for (int u = tid; u < E * (kKC / 4); u += 256) {
      const int e = u / (kKC / 4);
      const int j4 = (u % (kKC / 4)) * 4;
      float v[4] = {0.f, 0.f, 0.f, 0.f};
      if (j4 < kc) {
        const float4 q = *reinterpret_cast<const float4*>(wr + (int64_t)e * d + k0 + j4);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Ws[(j4 + i) * Ep + e] = v[i];
    }
    // token chunk: kTT rows x kKC columns
    for (int u = tid; u < kTT * kKC; u += 256) {
      const int t = u / kKC, j = u % kKC;
      float v = 0.0f;
      if (t0 + t < T && j < kc) v = Elem<TX>::load(x, (int64_t)(t0 + t) * d + k0 + j);
      Xs[j * XP + t] = v;
    }
    __syncthreads();
    for (int j = 0; j < kc; ++j) {
      const float4 xv = *reinterpret_cast<const float4*>(&Xs[j * XP + tg * 4]);
      const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int jj = 0; jj < EPT; ++jj) {
        const int e = el + 32 * jj;
        const float w = (e < E) ? Ws[j * Ep + e] : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][jj] = __builtin_fmaf(xs[i], w, acc[i][jj]);
      }
    }
  }
  __syncthreads();
  float* Ls = smem;  // kTT * Ep
#pragma unroll
  for (int jj = 0; jj < EPT; ++jj) {
    const int e = el + 32 * jj;
    if (e < E) {
      const float off = offset ? offset[e] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) Ls[(tg * 4 + i) * Ep + e] = offset ? acc[i][jj] + off : acc[i][jj];
    }
  }
  __syncthreads();

  // gate + top-k: one wave per token
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int Q = (EPT * 32 + 63) / 64;  // experts per lane: e = lane + 64*q
  for (int t = wave; t < kTT; t += 4) {
    const int tt = t0 + t;
    if (tt >= T) break;
    float p[Q], key[Q];
    if (gate == MOE_GATE_SOFTMAX) {
      float m = -__builtin_inff();
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int e = lane + 64 * q;
        key[q] = (e < E) ? Ls[t * Ep + e] : -__builtin_inff();
        m = fmaxf(m, key[q]);
      }
      m = wave_max(m);
      float s = 0.0f;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int e = lane + 64 * q;
        p[q] = (e < E) ? expf(key[q] - m) : 0.0f;
        s += p[q];
      }
      s = wave_sum(s);
      const float inv = 1.0f / s;
#pragma unroll
      for (int q = 0; q < Q; ++q) p[q] *= inv;
    } else {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int e = lane + 64 * q;
        if (e < E) {
          p[q] = sigmoid_c(Ls[t * Ep + e]);
          key[q] = sel_bias ? p[q] + sel_bias[e] : p[q];
        } else {
          p[q] = 0.0f;
          key[q] = -__builtin_inff();
        }
      }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int e = lane + 64 * q;
      if (e < E) probs[(int64_t)tt * E + e] = p[q];
    }
    // top-k: k rounds of a wave argmax on (key desc, index asc)
    uint32_t taken = 0;
    int my_idx = 0;
    float my_p = 0.0f, psum = 0.0f;
    for (int r = 0; r < k; ++r) {
      float bk = -__builtin_inff();
      int be = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int e = lane + 64 * q;
        if (e < E && !(taken & (1u << q)) && (key[q] > bk || be == 0x7fffffff)) {
          bk = key[q];
          be = e;
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        const float ok = __shfl_xor(bk, o, kWave);
        const int oe = __shfl_xor(be, o, kWave);
        if (ok > bk || (ok == bk && oe < be)) {
          bk = ok;
          be = oe;
        }
      }
      // be is now wave-uniform
      const int qw = be >> 6;
      float pv = 0.0f;
#pragma unroll
      for (int q = 0; q < Q; ++q)
        if (q == qw) pv = p[q];
      pv = __shfl(pv, be & 63, kWave);
      if ((be & 63) == lane) taken |= 1u << qw;
      if (lane == r) {
        my_idx = be;
        my_p = pv;
      }
      psum += pv;
    }
    if (lane < k) {
      topk_idx[(int64_t)tt * k + lane] = my_idx;
      topk_w[(int64_t)tt * k + lane] = renorm ? my_p / psum : my_p;
    }
  }
}

template <typename TX, int EPT>
hipError_t launch_router_t(const RouterArgs& a, hipStream_t st) {
  const int Ep = a.E + 1;
  const size_t lds = (size_t)(kKC * Ep + kKC * (kTT + 4)) * sizeof(float);
  const int blocks = (a.T + kTT - 1) / kTT;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)router_fwd_kernel<TX, EPT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((router_fwd_kernel<TX, EPT>), dim3(blocks), dim3(256), lds, st,
                     (const TX*)a.x, a.w_router, a.logit_offset, a.sel_bias, a.probs, a.topk_idx,
                     a.topk_w, a.T, a.d, a.E, a.k, a.gate, a.renorm);
  return hipGetLastError();
}

template <typename TX>
hipError_t launch_router_e(const RouterArgs& a, hipStream_t st) {
  const int ept = (a.E + 31) / 32;
  if (ept <= 1) return launch_router_t<TX, 1>(a, st);
  if (ept <= 2) return launch_router_t<TX, 2>(a, st);
  if (ept <= 4) return launch_router_t<TX, 4>(a, st);
  if (ept <= 8) return launch_router_t<TX, 8>(a, st);
  return launch_router_t<TX, 16>(a, st);
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t st) {
  if (a.dtype == MOE_DT_BF16) return launch_router_e<uint16_t>(a, st);
  return launch_router_e<float>(a, st);
}

}  // namespace moe
