// Router forward: fp32 logits, gate and top-k in one kernel.
//
// [SW] = "Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散"
// (ta-paperlens.web.app), eq. (1) and the section on routing; [WIKI] =
// "Mixture-of-Experts" (notes.yuuk.io), bullets on sigmoid gating with a
// per-expert bias that only steers the selection.
//
// Each workgroup owns TT (16 or 32) tokens and all E experts. The logits are a
// SIMT fp32 register-tiled product: every thread owns TT/8 tokens x EPT experts
// and walks the d_model axis in ascending order with one fused multiply-add per
// term, so each logit is the fixed-order fp32 sum the routing decision is
// defined on (no split of the sum, no matrix cores, no reassociation). The x
// chunk and the router weight chunk are staged through two LDS stages,
// transposed so that the per-step reads are conflict-free; the next chunk is
// fetched into registers while the current one is consumed. The gate then runs
// one wave per token.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

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

template <typename TX, int EPT, int TT>
__global__ __launch_bounds__(256) void router_fwd_kernel(
    const TX* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ offset,
    const float* __restrict__ sel_bias, float* __restrict__ probs, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int T, int d, int E, int k, int gate, int renorm) {
  // Two LDS stages, each Ws[j][e] (router weight chunk, transposed) + Xs[j][t];
  // after the loop Ls[t][e] (logits) reuses stage 0.
  constexpr int TPT = TT / 8;         // tokens per thread
  constexpr int XP = TT + 4;
  constexpr int WU = (EPT * 32) * (kKC / 4) / 256;  // float4 units of W per thread (E rounded up)
  constexpr int XU = TT * kKC / 256;                // x elements per thread
  extern __shared__ float smem[];
  const int Ep = E + 1;
  const int stage_floats = kKC * Ep + kKC * XP;

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TT;
  const int tg = tid >> 5;   // token group: tokens tg*TPT .. tg*TPT+TPT-1
  const int el = tid & 31;   // expert lane: experts el + 32*j

  float acc[TPT][EPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int j = 0; j < EPT; ++j) acc[i][j] = 0.0f;

  float4 wreg[WU];
  float xreg[XU];
  auto fetch = [&](int k0) {
    const int kc = min(kKC, d - k0);
#pragma unroll
    for (int i = 0; i < WU; ++i) {
      const int u = tid + i * 256;
      const int e = u / (kKC / 4);
      const int j4 = (u % (kKC / 4)) * 4;
      wreg[i] = (e < E && j4 < kc) ? *reinterpret_cast<const float4*>(wr + (int64_t)e * d + k0 + j4)
                                   : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const int u = tid + i * 256;
      const int t = u / kKC, j = u % kKC;
      xreg[i] = (t0 + t < T && j < kc) ? Elem<TX>::load(x, (int64_t)(t0 + t) * d + k0 + j) : 0.0f;
    }
  };
  auto stash = [&](float* st) {
    float* Ws = st;
    float* Xs = st + kKC * Ep;
#pragma unroll
    for (int i = 0; i < WU; ++i) {
      const int u = tid + i * 256;
      const int e = u / (kKC / 4);
      const int j4 = (u % (kKC / 4)) * 4;
      if (e < E) {
        Ws[(j4 + 0) * Ep + e] = wreg[i].x;
        Ws[(j4 + 1) * Ep + e] = wreg[i].y;
        Ws[(j4 + 2) * Ep + e] = wreg[i].z;
        Ws[(j4 + 3) * Ep + e] = wreg[i].w;
      }
    }
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const int u = tid + i * 256;
      Xs[(u % kKC) * XP + u / kKC] = xreg[i];
    }
  };

  const int nch = (d + kKC - 1) / kKC;
  fetch(0);
  stash(smem);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    float* st = smem + (c & 1) * stage_floats;
    if (c + 1 < nch) fetch((c + 1) * kKC);  // in flight during this chunk's FMAs
    const float* Ws = st;
    const float* Xs = st + kKC * Ep;
    const int kc = min(kKC, d - c * kKC);
    for (int j = 0; j < kc; ++j) {
      float xs[TPT];
#pragma unroll
      for (int i = 0; i < TPT; ++i) xs[i] = Xs[j * XP + tg * TPT + i];
#pragma unroll
      for (int jj = 0; jj < EPT; ++jj) {
        const int e = el + 32 * jj;
        const float w = (e < E) ? Ws[j * Ep + e] : 0.0f;
#pragma unroll
        for (int i = 0; i < TPT; ++i) acc[i][jj] = __builtin_fmaf(xs[i], w, acc[i][jj]);
      }
    }
    if (c + 1 < nch) stash(smem + ((c + 1) & 1) * stage_floats);
    __syncthreads();
  }
  float* Ls = smem;  // TT * Ep
#pragma unroll
  for (int jj = 0; jj < EPT; ++jj) {
    const int e = el + 32 * jj;
    if (e < E) {
      const float off = offset ? offset[e] : 0.0f;
#pragma unroll
      for (int i = 0; i < TPT; ++i) Ls[(tg * TPT + i) * Ep + e] = offset ? acc[i][jj] + off : acc[i][jj];
    }
  }
  __syncthreads();

  // gate + top-k: one wave per token
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int Q = (EPT * 32 + 63) / 64;  // experts per lane: e = lane + 64*q
  for (int t = wave; t < TT; t += 4) {
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

template <typename TX, int EPT, int TT>
hipError_t launch_router_t(const RouterArgs& a, hipStream_t st) {
  const int Ep = a.E + 1;
  const size_t lds = 2 * (size_t)(kKC * Ep + kKC * (TT + 4)) * sizeof(float);
  const int blocks = (a.T + TT - 1) / TT;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute((const void*)router_fwd_kernel<TX, EPT, TT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((router_fwd_kernel<TX, EPT, TT>), dim3(blocks), dim3(256), lds, st, (const TX*)a.x,
                     a.w_router, a.logit_offset, a.sel_bias, a.probs, a.topk_idx, a.topk_w, a.T, a.d, a.E, a.k,
                     a.gate, a.renorm);
  return hipGetLastError();
}

// 32 tokens per workgroup when that still gives at least two workgroups per CU
// of a 256-CU part, else 16 (more workgroups in flight for smaller batches).
template <typename TX, int EPT>
hipError_t launch_router_tt(const RouterArgs& a, hipStream_t st) {
  if ((a.T + 31) / 32 >= 512) return launch_router_t<TX, EPT, 32>(a, st);
  return launch_router_t<TX, EPT, 16>(a, st);
}

template <typename TX>
hipError_t launch_router_e(const RouterArgs& a, hipStream_t st) {
  const int ept = (a.E + 31) / 32;
  if (ept <= 1) return launch_router_tt<TX, 1>(a, st);
  if (ept <= 2) return launch_router_tt<TX, 2>(a, st);
  if (ept <= 4) return launch_router_tt<TX, 4>(a, st);
  if (ept <= 8) return launch_router_tt<TX, 8>(a, st);
  return launch_router_tt<TX, 16>(a, st);
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, hipStream_t st) {
  if (a.dtype == MOE_DT_BF16) return launch_router_e<uint16_t>(a, st);
  return launch_router_e<float>(a, st);
}

}  // namespace moe
