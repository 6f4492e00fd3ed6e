// Router forward: fp32 logits, gate and top-k in one kernel.
//
// [SW] = "Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散"
// (ta-paperlens.web.app), eq. (1) and the section on routing; [WIKI] =
// "Mixture-of-Experts" (notes.yuuk.io), bullets on sigmoid gating with a
// per-expert bias that only steers the selection, and the finding on the
// sigmoid giving way to the square root of softplus.
//
// The logit h[t,e] is the fp32 sum over j = 0..d-1 in ascending order of one
// fused multiply-add per term, starting from +0, so each lane owns whole dot
// products (no split of the sum, no matrix cores, no reassociation).
//
// Work split (two kernels). Logits: a wave owns 64 tokens (one per lane) and
// four experts. For a given j the router weight of an expert is the same for
// all 64 lanes, so the weights are read with scalar loads into SGPRs and enter
// each v_fma_f32 as its scalar operand; each lane streams its own x row with
// vector loads. The logits go to the probabilities buffer. Gate and top-k
// then run one wave per token on that row.
#include "common.h"
#include "gate_math.h"
#include "internal.h"

namespace moe {

namespace {

// Gate and top-k of one token whose logits h[q] (expert lane + 64 q) sit in
// the registers of the wave.
template <int QE>
__device__ __forceinline__ void gate_topk(const float* h, const float* __restrict__ sel_bias, int lane, int E,
                                          int k, int gate, int renorm, int64_t tt, float* __restrict__ probs,
                                          int32_t* __restrict__ topk_idx, float* __restrict__ topk_w) {
  float p[QE], key[QE];
  if (gate == MOE_GATE_SOFTMAX) {
    float m = -__builtin_inff();
#pragma unroll
    for (int q = 0; q < QE; ++q) {
      const int e = lane + 64 * q;
      key[q] = (e < E) ? h[q] : -__builtin_inff();
      m = fmaxf(m, key[q]);
    }
    m = wave_max(m);
    float s = 0.0f;
#pragma unroll
    for (int q = 0; q < QE; ++q) {
      const int e = lane + 64 * q;
      p[q] = (e < E) ? expf(key[q] - m) : 0.0f;
      s += p[q];
    }
    s = wave_sum(s);
    const float inv = 1.0f / s;
#pragma unroll
    for (int q = 0; q < QE; ++q) p[q] *= inv;
  } else {
#pragma unroll
    for (int q = 0; q < QE; ++q) {
      const int e = lane + 64 * q;
      if (e < E) {
        p[q] = gate == MOE_GATE_SIGMOID_BIAS ? sigmoid_c(h[q]) : sqrt_softplus_c(h[q]);
        key[q] = sel_bias ? p[q] + sel_bias[e] : p[q];
      } else {
        p[q] = 0.0f;
        key[q] = -__builtin_inff();
      }
    }
  }
#pragma unroll
  for (int q = 0; q < QE; ++q) {
    const int e = lane + 64 * q;
    if (e < E) probs[tt * E + e] = p[q];
  }
  // top-k: k rounds of a wave argmax on (key desc, index asc)
  uint32_t taken = 0;
  int my_idx = 0;
  float my_p = 0.0f, psum = 0.0f;
  for (int r = 0; r < k; ++r) {
    float bk = -__builtin_inff();
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < QE; ++q) {
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
    for (int q = 0; q < QE; ++q)
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
    topk_idx[tt * k + lane] = my_idx;
    topk_w[tt * k + lane] = renorm ? my_p / psum : my_p;
  }
}

// 8 consecutive x values of one token as fp32 (16 bytes of bf16, or two
// 16-byte fp32 loads).
template <typename TX>
struct X8;
template <>
struct X8<uint16_t> {
  uint4 r;
  __device__ void load(const uint16_t* p) { r = *reinterpret_cast<const uint4*>(p); }
  __device__ float get(int i) const {
    const uint32_t w = i < 2 ? r.x : i < 4 ? r.y : i < 6 ? r.z : r.w;
    return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct X8<float> {
  float4 a, b;
  __device__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ float get(int i) const {
    return i == 0 ? a.x : i == 1 ? a.y : i == 2 ? a.z : i == 3 ? a.w : i == 4 ? b.x : i == 5 ? b.y : i == 6 ? b.z : b.w;
  }
};

// Eight router weights of one expert (wave-uniform address, read into SGPRs).
struct W8 {
  float v[8];
  __device__ void load(const float* p) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

constexpr int kEW = 4;   // experts per wave
constexpr int kWaves = 4;

// Logits: lane = token (64 per wave), the wave's kEW experts are uniform. Each
// lane streams its own x row (vector loads, two 8-wide blocks ahead); the
// weights of the wave's experts come through scalar loads one block ahead.
// Writes h (without the offset) to out[T, E].
template <typename TX>
__global__ __launch_bounds__(256) void router_logits_kernel(const TX* __restrict__ x, const float* __restrict__ wr,
                                                            float* __restrict__ out, int T, int d, int E) {
  // 1-D grid, XCD-aware: workgroups go to the 8 XCDs round-robin, and each
  // XCD takes a contiguous range of (token tile, expert group) pairs with the
  // expert group fastest, so all expert groups of a 64-token x tile run on one
  // XCD back to back and the tile is read from HBM once.
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int neg = (E + kEW * kWaves - 1) / (kEW * kWaves);
  const int64_t total = (int64_t)((T + 63) / 64) * neg;
  const int64_t per = (total + 7) / 8;
  if ((int64_t)blockIdx.x / 8 >= per) return;
  const int64_t L = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (L >= total) return;
  const int t = (int)(L / neg) * 64 + lane;
  const int e0 = ((int)(L % neg) * kWaves + wave) * kEW;
  if (e0 >= E) return;
  const TX* xr = x + (int64_t)min(t, T - 1) * d;
  const float* wbase = wr + (int64_t)e0 * d;  // rows e0 .. e0 + kEW - 1 (clamped below)
  const int64_t wstep[kEW] = {0, (int64_t)min(1, E - 1 - e0) * d, (int64_t)min(2, E - 1 - e0) * d,
                              (int64_t)min(3, E - 1 - e0) * d};

  float acc[kEW];
#pragma unroll
  for (int i = 0; i < kEW; ++i) acc[i] = 0.0f;

  // Blocks of 8 along d with ping-pong weight buffers (4 experts x 8 values =
  // 32 SGPRs each). Scalar loads may complete out of order, so the only wait
  // for them is lgkmcnt(0), placed by the compiler before the first use: each
  // block starts with its first multiply-adds (waiting for its own weights,
  // issued one block earlier) and only then issues the next block's scalar
  // loads, which stay in flight during the other 28 multiply-adds of the block
  // (4-deep blocks left 12, and the waves waited on the weights). x is read 8
  // values at a time, one 16-byte vector load per lane, two blocks ahead.
  const int nb = d / 8;
  W8 w0[kEW], w1[kEW];
  auto loadw = [&](W8* w, int blk) {
#pragma unroll
    for (int i = 0; i < kEW; ++i) w[i].load(wbase + wstep[i] + 8 * blk);
  };
  auto fma_j = [&](float xv, const W8* wc, int j) {
#pragma unroll
    for (int i = 0; i < kEW; ++i) acc[i] = __builtin_fmaf(xv, wc[i].v[j], acc[i]);
  };
  auto block = [&](const X8<TX>& xc, const W8* wc, W8* wn, int nxt) {
    fma_j(xc.get(0), wc, 0);
    __builtin_amdgcn_sched_barrier(0);
    if (nxt < nb) loadw(wn, nxt);
#pragma unroll
    for (int j = 1; j < 8; ++j) fma_j(xc.get(j), wc, j);
  };
  X8<TX> x0, x1;
  x0.load(xr);
  if (nb > 1) x1.load(xr + 8);
  loadw(w0, 0);
  // d is a multiple of 8: one block per 8 values of x, in ascending order
  for (int b = 0; b < nb; b += 2) {
    block(x0, w0, w1, b + 1);
    if (b + 2 < nb) x0.load(xr + 8 * (b + 2));
    if (b + 1 >= nb) break;
    block(x1, w1, w0, b + 2);
    if (b + 3 < nb) x1.load(xr + 8 * (b + 3));
  }
  if (t < T) {
    float* o = out + (int64_t)t * E + e0;
    if (e0 + kEW <= E && (E & 3) == 0) {  // 16-byte aligned row segment
      *reinterpret_cast<float4*>(o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
#pragma unroll
      for (int i = 0; i < kEW; ++i)
        if (e0 + i < E) o[i] = acc[i];
    }
  }
}

// Gate and top-k, one wave per token: reads the logits from probs, adds the
// offset (one fp32 add), overwrites probs with the gate values.
template <int QE>
__global__ __launch_bounds__(256) void router_gate_kernel(const float* __restrict__ offset,
                                                          const float* __restrict__ sel_bias, float* probs,
                                                          int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                          int T, int E, int k, int gate, int renorm) {
  const int lane = threadIdx.x & 63;
  const int64_t tt = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tt >= T) return;
  float h[QE];
#pragma unroll
  for (int q = 0; q < QE; ++q) {
    const int e = lane + 64 * q;
    h[q] = 0.0f;
    if (e < E) {
      h[q] = probs[tt * E + e];
      if (offset) h[q] = h[q] + offset[e];
    }
  }
  gate_topk<QE>(h, sel_bias, lane, E, k, gate, renorm, tt, probs, topk_idx, topk_w);
}

// Noisy top-k gate (one wave per token): H = h + eps * softplus_c(n) from the
// stacked clean|noise logits (one fp32 multiply and one fp32 add; no
// contraction), then the softmax gate on H, renormalised over the k selected.
#pragma clang fp contract(off)
template <int QE>
__global__ __launch_bounds__(256) void noisy_gate_kernel(const float* __restrict__ logits2,
                                                         const float* __restrict__ noise, float* __restrict__ probs,
                                                         int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                                         int T, int E, int k) {
  const int lane = threadIdx.x & 63;
  const int64_t tt = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (tt >= T) return;
  float H[QE];
#pragma unroll
  for (int q = 0; q < QE; ++q) {
    const int e = lane + 64 * q;
    H[q] = 0.0f;
    if (e < E) {
      const float sp = softplus_c(logits2[tt * 2 * E + E + e]);
      const float prod = noise[tt * E + e] * sp;
      H[q] = logits2[tt * 2 * E + e] + prod;
    }
  }
  gate_topk<QE>(H, nullptr, lane, E, k, MOE_GATE_SOFTMAX, 1, tt, probs, topk_idx, topk_w);
}
#pragma clang fp contract(on)

// Register-tiled variant for wide d_model, where streaming x once per
// workgroup matters more than occupancy. A workgroup owns TT = TG * TPT tokens
// and every expert; thread (tg, eg) owns tokens tg*TPT .. +TPT-1 and experts
// 4*(eg + EG*h) + 0..3 (h < NE4), one dot product per (token, expert) walked
// in ascending j as above. The x chunk (Xs[j][t]) and the router weight chunk
// (Ws[j][e]) are staged through two LDS stages, transposed so that a thread's
// TPT tokens and each of its 4-expert groups are one 16-byte LDS read; the
// next chunk is fetched into registers while the current one is consumed.
// The logits then go through LDS to one wave per token for the gate.
template <typename TX>
struct XV;
template <>
struct XV<uint16_t> {  // 8 bf16 per 16 bytes
  static constexpr int N = 8;
  __device__ static void load(const uint16_t* p, float* v) {
    const uint4 r = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct XV<float> {  // 4 fp32 per 16 bytes
  static constexpr int N = 4;
  __device__ static void load(const float* p, float* v) {
    const float4 r = *reinterpret_cast<const float4*>(p);
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
  }
};

template <typename TX, int TPT, int NE4, int EG>
__global__ __launch_bounds__(256) void router_tile_kernel(
    const TX* __restrict__ x, const float* __restrict__ wr, const float* __restrict__ offset,
    const float* __restrict__ sel_bias, float* __restrict__ probs, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_w, int T, int d, int E, int k, int gate, int renorm) {
  constexpr int TG = 256 / EG;
  constexpr int TT = TG * TPT;
  constexpr int EPT = 4 * NE4;
  constexpr int EMAX = 4 * EG * NE4;
  constexpr int KC = 32;
  constexpr int XP = TT + 4;    // x row (16-byte aligned)
  constexpr int EP = EMAX + 4;  // weight row (16-byte aligned)
  constexpr int STAGE = KC * (EP + XP);
  constexpr int NX = XV<TX>::N;
  constexpr int XUNITS = TT * KC / NX;     // 16-byte x loads of a chunk
  constexpr int XU = (XUNITS + 255) / 256;  // per thread
  constexpr int WU = EMAX * KC / 4 / 256;   // float4 weight loads per thread
  static_assert(WU >= 1, "tile too small");
  extern __shared__ float smem[];

  const int tid = threadIdx.x;
  const int eg = tid % EG, tg = tid / EG;
  const int t0 = blockIdx.x * TT;

  float acc[TPT][EPT];
#pragma unroll
  for (int i = 0; i < TPT; ++i)
#pragma unroll
    for (int c = 0; c < EPT; ++c) acc[i][c] = 0.0f;

  float xreg[XU][NX];
  float4 wreg[WU];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const int u = tid + 256 * i;
      const int t = u / (KC / NX), j = (u % (KC / NX)) * NX;
      if (u < XUNITS && k0 + j < d) {
        XV<TX>::load(x + (int64_t)min(t0 + t, T - 1) * d + k0 + j, xreg[i]);
      } else {
#pragma unroll
        for (int c = 0; c < NX; ++c) xreg[i][c] = 0.0f;
      }
    }
#pragma unroll
    for (int i = 0; i < WU; ++i) {
      const int v = tid + 256 * i;
      const int e = v / (KC / 4), j4 = (v % (KC / 4)) * 4;
      wreg[i] = (e < E && k0 + j4 < d) ? *reinterpret_cast<const float4*>(wr + (int64_t)e * d + k0 + j4)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto stash = [&](float* st) {
    float* Ws = st;
    float* Xs = st + KC * EP;
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const int u = tid + 256 * i;
      const int t = u / (KC / NX), j = (u % (KC / NX)) * NX;
      if (u < XUNITS) {
#pragma unroll
        for (int c = 0; c < NX; ++c) Xs[(j + c) * XP + t] = xreg[i][c];
      }
    }
#pragma unroll
    for (int i = 0; i < WU; ++i) {
      const int v = tid + 256 * i;
      const int e = v / (KC / 4), j4 = (v % (KC / 4)) * 4;
      Ws[(j4 + 0) * EP + e] = wreg[i].x;
      Ws[(j4 + 1) * EP + e] = wreg[i].y;
      Ws[(j4 + 2) * EP + e] = wreg[i].z;
      Ws[(j4 + 3) * EP + e] = wreg[i].w;
    }
  };

  const int nch = (d + KC - 1) / KC;
  fetch(0);
  stash(smem);
  __syncthreads();
  for (int ch = 0; ch < nch; ++ch) {
    const float* Ws = smem + (ch & 1) * STAGE;
    const float* Xs = Ws + KC * EP;
    if (ch + 1 < nch) fetch((ch + 1) * KC);  // in flight during this chunk's multiply-adds
    const int kc = min(KC, d - ch * KC);
    // this thread's x values and router weights of step j of the chunk
    auto read_step = [&](int j, float* xs, float* ws) {
#pragma unroll
      for (int i = 0; i < TPT / 4; ++i) {
        const float4 v = *reinterpret_cast<const float4*>(Xs + j * XP + tg * TPT + 4 * i);
        xs[4 * i] = v.x; xs[4 * i + 1] = v.y; xs[4 * i + 2] = v.z; xs[4 * i + 3] = v.w;
      }
#pragma unroll
      for (int h = 0; h < NE4; ++h) {
        const float4 v = *reinterpret_cast<const float4*>(Ws + j * EP + 4 * (eg + EG * h));
        ws[4 * h] = v.x; ws[4 * h + 1] = v.y; ws[4 * h + 2] = v.z; ws[4 * h + 3] = v.w;
      }
    };
    auto fma_step = [&](const float* xs, const float* ws) {
#pragma unroll
      for (int i = 0; i < TPT; ++i)
#pragma unroll
        for (int c = 0; c < EPT; ++c) acc[i][c] = __builtin_fmaf(xs[i], ws[c], acc[i][c]);
    };
    if (kc == KC) {
      // A full chunk: the LDS reads of step j + 1 are issued before the
      // multiply-adds of step j, which hide their latency. Each logit still
      // takes its multiply-adds in ascending j.
      float xs[2][TPT], ws[2][EPT];
      read_step(0, xs[0], ws[0]);
#pragma unroll
      for (int j = 0; j + 1 < KC; ++j) {
        read_step(j + 1, xs[(j + 1) & 1], ws[(j + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the multiply-adds
        fma_step(xs[j & 1], ws[j & 1]);
      }
      fma_step(xs[(KC - 1) & 1], ws[(KC - 1) & 1]);
    } else {
      for (int j = 0; j < kc; ++j) {
        float xs[TPT], ws[EPT];
        read_step(j, xs, ws);
        fma_step(xs, ws);
      }
    }
    if (ch + 1 < nch) stash(smem + ((ch + 1) & 1) * STAGE);
    __syncthreads();
  }

  // logits (+ offset, one fp32 add) to LDS, then the gate, one wave per token
  float* Ls = smem;  // [TT][E + 1]
  const int LP = E + 1;
#pragma unroll
  for (int h = 0; h < NE4; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int e = 4 * (eg + EG * h) + c;
      if (e < E) {
        const float off = offset ? offset[e] : 0.0f;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
          const float v = acc[i][4 * h + c];
          Ls[(tg * TPT + i) * LP + e] = offset ? v + off : v;
        }
      }
    }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  constexpr int QE = EMAX / 64;
  for (int t = wave; t < TT; t += 4) {
    const int tt = t0 + t;
    if (tt >= T) break;
    float h[QE];
#pragma unroll
    for (int q = 0; q < QE; ++q) {
      const int e = lane + 64 * q;
      h[q] = (e < E) ? Ls[t * LP + e] : 0.0f;
    }
    if (gate == kGateLogitsOnly) {
#pragma unroll
      for (int q = 0; q < QE; ++q)
        if (lane + 64 * q < E) probs[(int64_t)tt * E + lane + 64 * q] = h[q];
      continue;
    }
    gate_topk<QE>(h, sel_bias, lane, E, k, gate, renorm, tt, probs, topk_idx, topk_w);
  }
}

template <typename TX, int TPT, int NE4>
hipError_t launch_router_tile(const RouterArgs& a, hipStream_t st) {
  constexpr int EG = 32;
  constexpr int TT = (256 / EG) * TPT;
  constexpr int KC = 32;
  const size_t stage = (size_t)KC * ((4 * EG * NE4 + 4) + (TT + 4));
  const size_t logits = (size_t)TT * (a.E + 1);
  const size_t lds = (2 * stage > logits ? 2 * stage : logits) * sizeof(float);
  const hipError_t e = hipFuncSetAttribute((const void*)router_tile_kernel<TX, TPT, NE4, EG>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((router_tile_kernel<TX, TPT, NE4, EG>), dim3((a.T + TT - 1) / TT), dim3(256), lds, st,
                     (const TX*)a.x, a.w_router, a.logit_offset, a.sel_bias, a.probs, a.topk_idx, a.topk_w, a.T,
                     a.d, a.E, a.k, a.gate, a.renorm);
  return hipGetLastError();
}

template <typename TX>
hipError_t launch_router_t(const RouterArgs& a, hipStream_t st) {
  const int64_t total = (int64_t)((a.T + 63) / 64) * ((a.E + kEW * kWaves - 1) / (kEW * kWaves));
  const dim3 g1((unsigned)((total + 7) / 8 * 8));
  hipLaunchKernelGGL(router_logits_kernel<TX>, g1, dim3(256), 0, st, (const TX*)a.x, a.w_router, a.probs, a.T,
                     a.d, a.E);
  const int qe = (a.E + 63) / 64;
  const dim3 g2((a.T + 3) / 4);
#define MOE_GATE_LAUNCH(Q)                                                                                   \
  hipLaunchKernelGGL(router_gate_kernel<Q>, g2, dim3(256), 0, st, a.logit_offset, a.sel_bias, a.probs,      \
                     a.topk_idx, a.topk_w, a.T, a.E, a.k, a.gate, a.renorm)
  if (qe <= 1) MOE_GATE_LAUNCH(1);
  else if (qe <= 2) MOE_GATE_LAUNCH(2);
  else if (qe <= 4) MOE_GATE_LAUNCH(4);
  else MOE_GATE_LAUNCH(8);
#undef MOE_GATE_LAUNCH
  return hipGetLastError();
}

}  // namespace

// Narrow d_model: the scalar-operand logits kernel (more waves in flight; x
// rows are short). Wide d_model: the register-tiled kernel, which streams x
// once per 32 or 64 tokens and reuses each LDS read over 4-8 tokens. With 129
// to 256 experts, 8 tokens per thread (158 VGPRs, 84 KB of LDS: one
// workgroup and one wave per SIMD) left the multiply-adds waiting on LDS; 4
// tokens per thread (two workgroups per CU) is faster at any batch size.
template <typename TX>
hipError_t launch_router_wide(const RouterArgs& a, hipStream_t st) {
  const bool big = (a.T + 63) / 64 >= 256;  // 64-token tiles still cover every CU
  if (a.E <= 128) return big ? launch_router_tile<TX, 8, 1>(a, st) : launch_router_tile<TX, 4, 1>(a, st);
  if (a.E <= 256) return launch_router_tile<TX, 4, 2>(a, st);
  return launch_router_tile<TX, 4, 4>(a, st);
}

namespace {

// Selection-bias step ([WIKI], Quantile Balancing finding, restating
// DeepSeek-V3's rule): b_j += gamma * sign(mean load - l_j) with l_j =
// counts[j]. sign(sum_i l_i / E - l_j) = sign(sum_i l_i - E l_j) is decided in
// 64-bit integers, so the step is exact; the add is one fp32 add. One
// workgroup: the count total is a fixed tree over LDS.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ counts, int E, float gamma,
                                                          float* __restrict__ bias) {
  __shared__ int64_t red[256];
  int64_t s = 0;
  for (int i = threadIdx.x; i < E; i += 256) s += counts[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  const int64_t total = red[0];
  for (int j = threadIdx.x; j < E; j += 256) {
    const int64_t diff = total - (int64_t)E * counts[j];
    const float b = bias[j];
    bias[j] = diff > 0 ? b + gamma : diff < 0 ? b - gamma : b;
  }
}

}  // namespace

hipError_t launch_bias_update(const int32_t* counts, int E, float gamma, float* bias, hipStream_t st) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(256), 0, st, counts, E, gamma, bias);
  return hipGetLastError();
}

hipError_t launch_router_logits(const RouterArgs& a, hipStream_t st, bool* offset_applied) {
  if (a.d <= 1024) {
    *offset_applied = false;
    const int64_t total = (int64_t)((a.T + 63) / 64) * ((a.E + kEW * kWaves - 1) / (kEW * kWaves));
    const dim3 g1((unsigned)((total + 7) / 8 * 8));
    if (a.dtype == MOE_DT_BF16)
      hipLaunchKernelGGL(router_logits_kernel<uint16_t>, g1, dim3(256), 0, st, (const uint16_t*)a.x, a.w_router,
                         a.probs, a.T, a.d, a.E);
    else
      hipLaunchKernelGGL(router_logits_kernel<float>, g1, dim3(256), 0, st, (const float*)a.x, a.w_router,
                         a.probs, a.T, a.d, a.E);
    return hipGetLastError();
  }
  *offset_applied = true;
  RouterArgs b = a;
  b.gate = kGateLogitsOnly;
  if (a.dtype == MOE_DT_BF16) return launch_router_wide<uint16_t>(b, st);
  return launch_router_wide<float>(b, st);
}

// Noisy top-k routing: the logits kernels over the stacked 2E-row router into
// logits2 [T, 2E], then the noisy gate.
hipError_t launch_route_noisy(const RouterArgs& a, const float* noise, float* logits2, hipStream_t st) {
  RouterArgs r = a;
  r.E = 2 * a.E;
  r.probs = logits2;
  r.logit_offset = nullptr;
  bool applied = false;
  hipError_t e = launch_router_logits(r, st, &applied);
  if (e != hipSuccess) return e;
  const int qe = (a.E + 63) / 64;
  const dim3 g((a.T + 3) / 4);
#define MOE_NOISY_LAUNCH(Q)                                                                                  \
  hipLaunchKernelGGL(noisy_gate_kernel<Q>, g, dim3(256), 0, st, logits2, noise, a.probs, a.topk_idx, a.topk_w, \
                     a.T, a.E, a.k)
  if (qe <= 1) MOE_NOISY_LAUNCH(1);
  else if (qe <= 2) MOE_NOISY_LAUNCH(2);
  else MOE_NOISY_LAUNCH(4);
#undef MOE_NOISY_LAUNCH
  return hipGetLastError();
}

hipError_t launch_router(const RouterArgs& a, hipStream_t st) {
  if (a.d <= 1024) {
    if (a.dtype == MOE_DT_BF16) return launch_router_t<uint16_t>(a, st);
    return launch_router_t<float>(a, st);
  }
  if (a.dtype == MOE_DT_BF16) return launch_router_wide<uint16_t>(a, st);
  return launch_router_wide<float>(a, st);
}

}  // namespace moe
