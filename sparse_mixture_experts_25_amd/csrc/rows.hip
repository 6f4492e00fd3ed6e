// Row-streaming kernels of the layer: combine, aux loss, and the backward
// pieces around the expert matmuls (combine backward, router gradient,
// unpermute backward).
//
// [SW] = "Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散"
// (ta-paperlens.web.app): eq. (2) (gate-weighted sum over the selected
// experts; the router is trained through the gate), the capacity section
// (dropped tokens pass through on the residual), eq. (4) and the numpy sketch
// after it (aux loss; f is a count, P a mean probability).
// [WIKI] = "Mixture-of-Experts" (notes.yuuk.io): sigmoid gate with a bias used
// only for selection; shared expert.
//
// All of these are HBM-bound gathers/scatters of whole rows: one wave per
// token row, 16-byte vectors, fp32 accumulation, and no atomics, so every
// result is reproducible bit for bit.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

// Wide token tables (expert-choice routing has one column per expert, k = E,
// with only a few kept) are first compacted per token: the kept columns, in
// column order, go to a per-wave LDS list, so the row loop touches only them.
constexpr int kWideK = 8;       // tables wider than this take the compacted path
constexpr int kListMax = 512;   // most table columns a token can have

// Hand LDS written by some lanes of a wave to the other lanes of that wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Kept columns (slot >= 0) of one token's k columns, in column order: slot to
// ls[], column to lr[]. Returns their number (wave-uniform).
__device__ __forceinline__ int kept_columns(const int32_t* __restrict__ srow, int k, int lane, int32_t* ls,
                                            int32_t* lr) {
  int n = 0;
  for (int r0 = 0; r0 < k; r0 += 64) {
    const int r = r0 + lane;
    const int s = r < k ? srow[r] : -1;
    const uint64_t m = __ballot(s >= 0);
    if (s >= 0) {
      const int pos = n + (int)__popcll(m & ((1ull << lane) - 1ull));
      ls[pos] = s;
      lr[pos] = r;
    }
    n += (int)__popcll(m);
  }
  wave_lds_sync();
  return n;
}

// Narrow token tables (k <= KM <= 8): one token per wave. The token's slots
// and weights are read once (wave-uniform); for each 16-byte vector of the row
// the loads of all k rows are issued before any of them is summed, so a lane
// has k + 1 loads in flight. A dropped column (slot < 0) loads the token's own
// row of the first operand instead (always valid memory) and is not summed.
// The expert-group ranking of the weight-gradient launches, folded into the
// combine backward launch as its first workgroup (one dependent launch fewer;
// first, so that it runs beside the row work instead of after it).
struct GroupRank {
  const int32_t* offsets;
  int E, shared_rows, has_shared;
  int32_t* order;  // null: no extra workgroup
  // workgroups before the row work
  __device__ int skip() const { return order ? 1 : 0; }
  // true in the extra workgroup, after it has done the ranking
  __device__ bool run() const {
    if (!order || blockIdx.x != 0) return false;
    __shared__ int rows_s[1025];
    rank_groups_by_rows(offsets, E, shared_rows, has_shared, order, rows_s, 256);
    return true;
  }
};

template <int KM>
struct TokenCols {
  int s[KM];
  float w[KM];
  __device__ void load(const int32_t* __restrict__ slot, const float* __restrict__ topk_w, int64_t t, int k) {
#pragma unroll
    for (int r = 0; r < KM; ++r) {
      s[r] = r < k ? slot[t * k + r] : -1;
      w[r] = r < k && topk_w ? topk_w[t * k + r] : 0.0f;
    }
  }
};

// combine for k <= KM: y[t] = x[t] + sum_kept w y_perm[s] (+ y_shared[t]), ascending r
template <typename TX, int KM>
__global__ __launch_bounds__(256) void combine_narrow_kernel(const TX* __restrict__ x, const TX* __restrict__ y_perm,
                                                             const int32_t* __restrict__ slot,
                                                             const float* __restrict__ topk_w,
                                                             const TX* __restrict__ y_shared, TX* __restrict__ y,
                                                             int T, int d, int k) {
  constexpr int V = Elem<TX>::kVec;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wave);  // wave-uniform: scalar table reads
  if (t >= T) return;
  TokenCols<KM> c;
  c.load(slot, topk_w, t, k);
  const TX* xr = x + (int64_t)t * d;
  const TX* rows[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) rows[r] = c.s[r] >= 0 ? y_perm + (int64_t)c.s[r] * d : xr;
  // Two vectors per lane and iteration (2 KB of each row per wave), all their
  // loads issued before either is summed; a missing shared expert loads x again.
  // The gathered rows (read once) and y (written once) bypass the caches.
  const TX* ysr = y_shared ? y_shared + (int64_t)t * d : xr;
  struct In { u128 raw[KM], xv, sv; };
  auto load = [&](int v, In& in) {
#pragma unroll
    for (int r = 0; r < KM; ++r) in.raw[r] = ld128_nt(rows[r] + v * V);
    in.xv = ld128(xr + v * V);
    in.sv = ld128(ysr + v * V);
  };
  auto finish = [&](int v, const In& in) {
    float acc[V], tmp[V];
    Elem<TX>::unpack(in.xv, acc);
#pragma unroll
    for (int r = 0; r < KM; ++r) {
      if (c.s[r] < 0) continue;
      Elem<TX>::unpack(in.raw[r], tmp);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = __builtin_fmaf(c.w[r], tmp[e], acc[e]);
    }
    if (y_shared) {
      Elem<TX>::unpack(in.sv, tmp);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += tmp[e];
    }
    st128_nt(y + (int64_t)t * d + v * V, Elem<TX>::pack(acc));
  };
  const int nv = d / V;
  int v = lane;
  for (; v + 64 < nv; v += 128) {
    In a, b;
    load(v, a);
    load(v + 64, b);
    finish(v, a);
    finish(v + 64, b);
  }
  if (v < nv) {
    In a;
    load(v, a);
    finish(v, a);
  }
}

// combine backward for k <= KM: dO[s] = w dy[t] and dg[t,r] = <dy[t], y_perm[s]>
// for every kept column; dg = 0 for dropped ones. dy is read once per token.
template <typename TX, int KM>
__global__ __launch_bounds__(256) void combine_bwd_narrow_kernel(const TX* __restrict__ dy,
                                                                 const TX* __restrict__ y_perm,
                                                                 const int32_t* __restrict__ slot,
                                                                 const float* __restrict__ topk_w,
                                                                 TX* __restrict__ dO, float* __restrict__ dg, int T,
                                                                 int d, int k, GroupRank gr_job) {
  if (gr_job.run()) return;
  constexpr int V = Elem<TX>::kVec;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // wave-uniform: scalar table reads
  const int t = __builtin_amdgcn_readfirstlane(((int)blockIdx.x - gr_job.skip()) * 4 + wave);
  if (t >= T) return;
  TokenCols<KM> c;
  c.load(slot, topk_w, t, k);
  const TX* gr = dy + (int64_t)t * d;
  const TX* rows[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) rows[r] = c.s[r] >= 0 ? y_perm + (int64_t)c.s[r] * d : gr;
  float dot[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) dot[r] = 0.0f;
  // Two vectors per lane and iteration (2 KB of each row per wave), all their
  // loads issued before either is used; each lane's dot products still add its
  // vectors in ascending order. The gathered rows (read once) bypass the caches.
  struct In { u128 raw[KM], gv; };
  auto load = [&](int v, In& in) {
#pragma unroll
    for (int r = 0; r < KM; ++r) in.raw[r] = ld128_nt(rows[r] + v * V);
    in.gv = ld128(gr + v * V);
  };
  auto finish = [&](int v, const In& in) {
    float g[V], yv[V], o[V];
    Elem<TX>::unpack(in.gv, g);
#pragma unroll
    for (int r = 0; r < KM; ++r) {
      if (c.s[r] < 0) continue;
      Elem<TX>::unpack(in.raw[r], yv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        dot[r] = __builtin_fmaf(g[e], yv[e], dot[r]);
        o[e] = c.w[r] * g[e];
      }
      st128(dO + (int64_t)c.s[r] * d + v * V, Elem<TX>::pack(o));
    }
  };
  const int nv = d / V;
  int v = lane;
  for (; v + 64 < nv; v += 128) {
    In a, b;
    load(v, a);
    load(v + 64, b);
    finish(v, a);
    finish(v + 64, b);
  }
  if (v < nv) {
    In a;
    load(v, a);
    finish(v, a);
  }
#pragma unroll
  for (int r = 0; r < KM; ++r) {
    if (r >= k) break;
    const float sum = wave_sum(dot[r]);
    if (lane == 0) dg[(int64_t)t * k + r] = c.s[r] >= 0 ? sum : 0.0f;
  }
}

// unpermute backward for k <= KM: dx = dy + sum_kept dX_perm[s] (ascending r)
// (+ dx_router) (+ dx_shared)
template <typename TX, int KM>
__global__ __launch_bounds__(256) void unpermute_bwd_narrow_kernel(const TX* __restrict__ dy,
                                                                   const TX* __restrict__ dX_perm,
                                                                   const int32_t* __restrict__ slot,
                                                                   const float* __restrict__ dx_router,
                                                                   const TX* __restrict__ dx_shared,
                                                                   TX* __restrict__ dx, int T, int d, int k) {
  constexpr int V = Elem<TX>::kVec;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wave);  // wave-uniform: scalar table reads
  if (t >= T) return;
  TokenCols<KM> c;
  c.load(slot, nullptr, t, k);
  const TX* gr = dy + (int64_t)t * d;
  const TX* rows[KM];
#pragma unroll
  for (int r = 0; r < KM; ++r) rows[r] = c.s[r] >= 0 ? dX_perm + (int64_t)c.s[r] * d : gr;
  // every load of a vector is issued before any sum (a missing router or shared
  // term loads the token's dy row instead and is skipped); the sums keep the
  // order dy, kept rows by ascending r, router term, shared expert
  const float* prr = dx_router ? dx_router + (int64_t)t * d : nullptr;
  const TX* psh = dx_shared ? dx_shared + (int64_t)t * d : gr;
  // Two vectors per lane and iteration (2 KB of each row per wave), all their
  // loads issued before either is summed. Every input row (read once) and dx
  // (written once) bypass the caches.
  struct In { u128 raw[KM], rdy, rsh; float4 q[V / 4]; };
  auto load = [&](int v, In& in) {
#pragma unroll
    for (int r = 0; r < KM; ++r) in.raw[r] = ld128_nt(rows[r] + v * V);
    in.rdy = ld128_nt(gr + v * V);
    in.rsh = ld128_nt(psh + v * V);
#pragma unroll
    for (int e = 0; e < V / 4; ++e) {
      if (prr) {
        const u128 w = ld128_nt(prr + v * V + 4 * e);
        in.q[e] = make_float4(__uint_as_float(w.w[0]), __uint_as_float(w.w[1]), __uint_as_float(w.w[2]),
                              __uint_as_float(w.w[3]));
      } else {
        in.q[e] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto finish = [&](int v, const In& in) {
    const u128* raw = in.raw;
    const u128 rsh = in.rsh;
    const float4* q = in.q;
    float acc[V], tmp[V];
    Elem<TX>::unpack(in.rdy, acc);
#pragma unroll
    for (int r = 0; r < KM; ++r) {
      if (c.s[r] < 0) continue;
      Elem<TX>::unpack(raw[r], tmp);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += tmp[e];
    }
    if (prr) {
#pragma unroll
      for (int e = 0; e < V / 4; ++e) {
        acc[4 * e] += q[e].x; acc[4 * e + 1] += q[e].y; acc[4 * e + 2] += q[e].z; acc[4 * e + 3] += q[e].w;
      }
    }
    if (dx_shared) {
      Elem<TX>::unpack(rsh, tmp);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += tmp[e];
    }
    st128_nt(dx + (int64_t)t * d + v * V, Elem<TX>::pack(acc));
  };
  const int nv = d / V;
  int v = lane;
  for (; v + 64 < nv; v += 128) {
    In a, b;
    load(v, a);
    load(v + 64, b);
    finish(v, a);
    finish(v + 64, b);
  }
  if (v < nv) {
    In a;
    load(v, a);
    finish(v, a);
  }
}

// Wide tables (k > 8): y[t] = x[t] + sum_kept w[t,r] * y_perm[slot[t,r]]
// (+ y_shared[t]), kept columns (compacted first) in ascending r
template <typename TX>
__global__ __launch_bounds__(256) void combine_wide_kernel(const TX* __restrict__ x, const TX* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ topk_w,
                                                      const TX* __restrict__ y_shared, TX* __restrict__ y,
                                                      int T, int d, int k) {
  constexpr int V = Elem<TX>::kVec;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int nvec = d / V;
  __shared__ int32_t lsb[4][kListMax], lrb[4][kListMax];
  const int n = kept_columns(slot + (int64_t)t * k, k, lane, lsb[wave], lrb[wave]);
  const int32_t* ls = lsb[wave];
  const int32_t* lr = lrb[wave];
  for (int v = lane; v < nvec; v += 64) {
    float acc[V], tmp[V];
    Elem<TX>::unpack(ld128(x + (int64_t)t * d + v * V), acc);
    for (int i = 0; i < n; ++i) {
      const int r = lr[i];
      const int s = ls[i];
      const float w = topk_w[(int64_t)t * k + r];
      Elem<TX>::unpack(ld128(y_perm + (int64_t)s * d + v * V), tmp);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = __builtin_fmaf(w, tmp[e], acc[e]);
    }
    if (y_shared) {
      Elem<TX>::unpack(ld128(y_shared + (int64_t)t * d + v * V), tmp);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += tmp[e];
    }
    st128(y + (int64_t)t * d + v * V, Elem<TX>::pack(acc));
  }
}

constexpr int kAuxTok = 32;  // tokens per partial-sum block

__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ probs, int T, int E,
                                                          float* __restrict__ partial) {
  const int t0 = blockIdx.x * kAuxTok;
  const int t1 = min(T, t0 + kAuxTok);
  for (int e = threadIdx.x; e < E; e += 256) {
    float s = 0.0f;
#pragma unroll 8
    for (int t = t0; t < t1; ++t) s += probs[(int64_t)t * E + e];
    partial[(int64_t)blockIdx.x * E + e] = s;
  }
}

// aux = alpha * E * sum_e f_e P_e. Each expert's column of block partials is
// summed by `parts` threads (strided over the blocks), then the parts in order,
// then the experts by a fixed tree: many short sums instead of E long ones.
constexpr int kAuxFin = 1024;
__global__ __launch_bounds__(kAuxFin) void aux_final_kernel(const float* __restrict__ partial, int nblk,
                                                            const int32_t* __restrict__ counts, int T, int E,
                                                            int k, float alpha, float* __restrict__ out) {
  __shared__ float part_sum[kAuxFin];
  __shared__ float red[kAuxFin / 64];
  const int tid = threadIdx.x;
  const int parts = kAuxFin / E;  // >= 2 (E <= 512)
  if (tid < parts * E) {
    const int e = tid % E, p = tid / E;
    float s = 0.0f;
#pragma unroll 8
    for (int b = p; b < nblk; b += parts) s += partial[(int64_t)b * E + e];
    part_sum[tid] = s;
  }
  __syncthreads();
  float acc = 0.0f;
  if (tid < E) {
    float P = 0.0f;
    for (int p = 0; p < parts; ++p) P += part_sum[p * E + tid];
    P /= (float)T;
    const float f = (float)counts[tid] / ((float)T * (float)k);
    acc = f * P;
  }
  acc = wave_sum(acc);
  if ((tid & 63) == 0) red[tid >> 6] = acc;
  __syncthreads();
  if (tid == 0) {
    float s = 0.0f;
    for (int w = 0; w < kAuxFin / 64; ++w) s += red[w];
    out[0] = (T == 0 || alpha == 0.0f) ? 0.0f : alpha * (float)E * s;
  }
}

// dO[slot] = w * dy[t]; dg[t,r] = <dy[t], y_perm[slot]> (0 when dropped)
template <typename TX>
__global__ __launch_bounds__(256) void combine_bwd_wide_kernel(const TX* __restrict__ dy, const TX* __restrict__ y_perm,
                                                          const int32_t* __restrict__ slot,
                                                          const float* __restrict__ topk_w, TX* __restrict__ dO,
                                                          float* __restrict__ dg, int T, int d, int k,
                                                          GroupRank gr_job) {
  if (gr_job.run()) return;
  constexpr int V = Elem<TX>::kVec;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = ((int)blockIdx.x - gr_job.skip()) * 4 + wave;
  if (t >= T) return;
  const int nvec = d / V;
  __shared__ int32_t lsb[4][kListMax], lrb[4][kListMax];
  const int n = kept_columns(slot + (int64_t)t * k, k, lane, lsb[wave], lrb[wave]);
  const int32_t* ls = lsb[wave];
  const int32_t* lr = lrb[wave];
  for (int r = lane; r < k; r += 64)
    if (slot[(int64_t)t * k + r] < 0) dg[(int64_t)t * k + r] = 0.0f;
  for (int i = 0; i < n; ++i) {
    const int r = lr[i];
    const int s = ls[i];
    const float w = topk_w[(int64_t)t * k + r];
    float dot = 0.0f;
    for (int v = lane; v < nvec; v += 64) {
      float g[V], yv[V], o[V];
      Elem<TX>::unpack(ld128(dy + (int64_t)t * d + v * V), g);
      Elem<TX>::unpack(ld128(y_perm + (int64_t)s * d + v * V), yv);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        dot = __builtin_fmaf(g[e], yv[e], dot);
        o[e] = w * g[e];
      }
      st128(dO + (int64_t)s * d + v * V, Elem<TX>::pack(o));
    }
    dot = wave_sum(dot);
    if (lane == 0) dg[(int64_t)t * k + r] = dot;
  }
}

// Router logit gradient for one token per wave: gate path + aux path.
__global__ __launch_bounds__(256) void dlogits_kernel(const float* __restrict__ probs,
                                                      const int32_t* __restrict__ topk_idx,
                                                      const float* __restrict__ topk_w,
                                                      const float* __restrict__ dg,
                                                      const int32_t* __restrict__ counts,
                                                      float* __restrict__ dlogits, int T, int E, int k, int gate,
                                                      int renorm, float alpha, uint16_t* __restrict__ gx,
                                                      uint16_t* __restrict__ gw, int kp,
                                                      const float* __restrict__ w_router,
                                                      uint16_t* __restrict__ wsplit, int32_t* __restrict__ offs,
                                                      int d, int nsw, int chunk) {
  const int tok_blocks = (T + 3) / 4;
  if ((int)blockIdx.x >= tok_blocks) {  // the router-weight split (bf16 layers)
    split_router_weights((int64_t)(blockIdx.x - tok_blocks) * 256 + threadIdx.x, w_router, E, d, kp, wsplit, T, nsw,
                         chunk, offs);
    return;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // wave-uniform: the token's k indices, weights and gate gradients, and the
  // probabilities they select, are scalar loads
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + wave);
  if (t >= T) return;
  const float* p = probs + (int64_t)t * E;
  // without topk_idx (expert-choice tables) column r is expert r and k = E
  const int32_t* it = topk_idx ? topk_idx + (int64_t)t * k : nullptr;
  const float* wt = topk_w + (int64_t)t * k;
  const float* gt = dg + (int64_t)t * k;
  // token-level sums over the k selected
  float S = 0.0f, wdg = 0.0f, ssum = 0.0f;
  if (it) {
    for (int r = 0; r < k; ++r) {
      const float pe = p[it[r]];
      S += gt[r] * pe;
      wdg += wt[r] * gt[r];
      ssum += pe;
    }
  } else {
    for (int j = lane; j < E; j += 64) {
      S += gt[j] * p[j];
      wdg += wt[j] * gt[j];
      ssum += p[j];
    }
    S = wave_sum(S);
    wdg = wave_sum(wdg);
    ssum = wave_sum(ssum);
  }
  const float c = alpha * (float)E / (float)T;
  const float invTk = 1.0f / ((float)T * (float)k);
  // f_j = counts_j / (T k), rounded once (no contraction) and used both in
  // sum_j f_j p_j and in each f_j - that sum, so that with one expert (p = 1)
  // the softmax term is exactly zero
  auto frac = [&](int j) {
#pragma clang fp contract(off)
    return (float)counts[j] * invTk;
  };
  float fp = 0.0f;
  if (alpha != 0.0f) {
    for (int j = lane; j < E; j += 64) fp += frac(j) * p[j];
    fp = wave_sum(fp);
  }
  for (int j = lane; j < E; j += 64) {
    const float pj = p[j];
    int rsel = it ? -1 : j;
    if (it)
      for (int r = 0; r < k; ++r)
        if (it[r] == j) rsel = r;
    float v = 0.0f;
    if (gate == MOE_GATE_SOFTMAX) {
      if (!renorm) {
        v = (rsel >= 0 ? gt[rsel] * pj : 0.0f) - pj * S;
      } else if (rsel >= 0) {
        v = wt[rsel] * (gt[rsel] - wdg);
      }
      if (alpha != 0.0f) v += c * pj * (frac(j) - fp);
    } else {
      // derivative of the gate written with its value s: sigmoid s (1 - s);
      // sqrt(softplus) sigmoid(h) / (2 s) = (1 - e^(-s^2)) / (2 s), 0 at s = 0
      const float gd = gate == MOE_GATE_SIGMOID_BIAS ? pj * (1.0f - pj)
                       : pj > 0.0f                   ? -expm1f(-pj * pj) / (2.0f * pj)
                                                     : 0.0f;
      if (rsel >= 0) {
        const float ds = renorm ? (gt[rsel] - wdg) / ssum : gt[rsel];
        v = ds * gd;
      }
      if (alpha != 0.0f) v += c * frac(j) * gd;
    }
    if (dlogits) dlogits[(int64_t)t * E + j] = v;
    if (gx) {
      // gx[t] = [hi | hi | mid | 0 ...], gw[t] = [hi | mid | lo | 0 ...]
      const Split3 sp = split3(v);
      uint16_t* xr = gx + (int64_t)t * kp;
      uint16_t* wr = gw + (int64_t)t * kp;
      xr[j] = sp.h;
      xr[E + j] = sp.h;
      xr[2 * E + j] = sp.m;
      wr[j] = sp.h;
      wr[E + j] = sp.m;
      wr[2 * E + j] = sp.l;
    }
  }
  if (gx)
    for (int cp = 3 * E + lane; cp < kp; cp += 64) {
      gx[(int64_t)t * kp + cp] = 0;
      gw[(int64_t)t * kp + cp] = 0;
    }
}

// C[M,N] (+)= sum_k A[k,m] * B[k,n] over one chunk of k (fp32 SIMT, 64x64 tiles).
// A: fp32 [K][M] (row stride lda); B: TB [K][N]. Partial results per K chunk go
// to part[split][M][N]; a second kernel sums the chunks in a fixed order.
constexpr int kRG = 64, kRK = 16;
template <typename TB>
__global__ __launch_bounds__(256) void gemm_tn_split_kernel(const float* __restrict__ A, int64_t lda,
                                                            const TB* __restrict__ B, int64_t ldb, int M,
                                                            int N, int K, int kchunk, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float As[kRK][kRG + 4];
  __shared__ __attribute__((aligned(16))) float Bs[kRK][kRG + 4];
  const int nN = (N + kRG - 1) / kRG;
  const int mb = blockIdx.x / nN, nb = blockIdx.x % nN;
  const int ks = blockIdx.y * kchunk, ke = min(K, ks + kchunk);
  const int tid = threadIdx.x, tm = tid / 16, tn = tid % 16;
  float acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = ks; k0 < ke; k0 += kRK) {
    __syncthreads();
    for (int u = tid; u < kRK * kRG; u += 256) {
      const int kk = u / kRG, c = u % kRG;
      const int k = k0 + kk;
      const int m = mb * kRG + c, n = nb * kRG + c;
      As[kk][c] = (k < ke && m < M) ? A[(int64_t)k * lda + m] : 0.0f;
      Bs[kk][c] = (k < ke && n < N) ? Elem<TB>::load(B, (int64_t)k * ldb + n) : 0.0f;
    }
    __syncthreads();
    for (int kk = 0; kk < kRK; ++kk) {
      float av[4], bv[4];
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tm * 4 + i];
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tn * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
  }
  float* out = part + (int64_t)blockIdx.y * M * N;
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int m = mb * kRG + tm * 4 + i, n = nb * kRG + tn * 4 + j;
      if (m < M && n < N) out[(int64_t)m * N + n] = acc[i][j];
    }
}

__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, int nsplit,
                                                         int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int p = 0; p < nsplit; ++p) s += part[(int64_t)p * n + i];
  out[i] = s;
}

// C[M,N] = A[M,K] * B[K,N], all fp32 row-major (dx_router = dlogits * W_r).
__global__ __launch_bounds__(256) void gemm_nn_f32_kernel(const float* __restrict__ A, const float* __restrict__ B,
                                                          float* __restrict__ C, int M, int N, int K) {
  __shared__ __attribute__((aligned(16))) float As[kRK][kRG + 4];
  __shared__ __attribute__((aligned(16))) float Bs[kRK][kRG + 4];
  const int nN = (N + kRG - 1) / kRG;
  const int mb = blockIdx.x / nN, nb = blockIdx.x % nN;
  const int tid = threadIdx.x, tm = tid / 16, tn = tid % 16;
  float acc[4][4];
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  for (int k0 = 0; k0 < K; k0 += kRK) {
    __syncthreads();
    for (int u = tid; u < kRK * kRG; u += 256) {
      const int kk = u % kRK, r = u / kRK;
      const int m = mb * kRG + r, k = k0 + kk;
      As[kk][r] = (m < M && k < K) ? A[(int64_t)m * K + k] : 0.0f;
      const int kk2 = u / kRG, c = u % kRG;
      const int n = nb * kRG + c, k2 = k0 + kk2;
      Bs[kk2][c] = (n < N && k2 < K) ? B[(int64_t)k2 * N + n] : 0.0f;
    }
    __syncthreads();
    for (int kk = 0; kk < kRK; ++kk) {
      float av[4], bv[4];
      for (int i = 0; i < 4; ++i) av[i] = As[kk][tm * 4 + i];
      for (int j = 0; j < 4; ++j) bv[j] = Bs[kk][tn * 4 + j];
      for (int i = 0; i < 4; ++i)
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    }
  }
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) {
      const int m = mb * kRG + tm * 4 + i, n = nb * kRG + tn * 4 + j;
      if (m < M && n < N) C[(int64_t)m * N + n] = acc[i][j];
    }
}

// dx[t] = dy[t] + sum_kept dX_perm[slot] + dx_router[t] (+ dx_shared[t])
template <typename TX>
__global__ __launch_bounds__(256) void unpermute_bwd_wide_kernel(const TX* __restrict__ dy,
                                                            const TX* __restrict__ dX_perm,
                                                            const int32_t* __restrict__ slot,
                                                            const float* __restrict__ dx_router,
                                                            const TX* __restrict__ dx_shared, TX* __restrict__ dx,
                                                            int T, int d, int k) {
  constexpr int V = Elem<TX>::kVec;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int nvec = d / V;
  __shared__ int32_t lsb[4][kListMax], lrb[4][kListMax];
  const int n = kept_columns(slot + (int64_t)t * k, k, lane, lsb[wave], lrb[wave]);
  const int32_t* ls = lsb[wave];
  for (int v = lane; v < nvec; v += 64) {
    float acc[V], tmp[V];
    Elem<TX>::unpack(ld128(dy + (int64_t)t * d + v * V), acc);
    for (int i = 0; i < n; ++i) {
      const int s = ls[i];
      Elem<TX>::unpack(ld128(dX_perm + (int64_t)s * d + v * V), tmp);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += tmp[e];
    }
    if (dx_router) {
      const float* pr = dx_router + (int64_t)t * d + v * V;
#pragma unroll
      for (int e = 0; e < V; e += 4) {
        const float4 q = *reinterpret_cast<const float4*>(pr + e);
        acc[e] += q.x; acc[e + 1] += q.y; acc[e + 2] += q.z; acc[e + 3] += q.w;
      }
    }
    if (dx_shared) {
      Elem<TX>::unpack(ld128(dx_shared + (int64_t)t * d + v * V), tmp);
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] += tmp[e];
    }
    st128(dx + (int64_t)t * d + v * V, Elem<TX>::pack(acc));
  }
}

}  // namespace

// k <= 8: the narrow kernels with KM = k rounded up to 1, 2, 4 or 8; wider
// tables: the compacted kernels
template <typename TX>
void launch_combine_t(const CombineArgs& a, hipStream_t st) {
  const dim3 g((a.T + 3) / 4), b(256);
#define MOE_LAUNCH(KM)                                                                                        \
  hipLaunchKernelGGL((combine_narrow_kernel<TX, KM>), g, b, 0, st, (const TX*)a.x, (const TX*)a.y_perm, a.slot, \
                     a.topk_w, (const TX*)a.y_shared, (TX*)a.y, a.T, a.d, a.k)
  if (a.k <= 1) MOE_LAUNCH(1);
  else if (a.k <= 2) MOE_LAUNCH(2);
  else if (a.k <= 4) MOE_LAUNCH(4);
  else if (a.k <= kWideK) MOE_LAUNCH(8);
  else
    hipLaunchKernelGGL((combine_wide_kernel<TX>), g, b, 0, st, (const TX*)a.x, (const TX*)a.y_perm, a.slot,
                       a.topk_w, (const TX*)a.y_shared, (TX*)a.y, a.T, a.d, a.k);
#undef MOE_LAUNCH
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  if (a.dtype == MOE_DT_BF16) launch_combine_t<uint16_t>(a, st);
  else launch_combine_t<float>(a, st);
  return hipGetLastError();
}

int aux_num_blocks(int T) { return (T + kAuxTok - 1) / kAuxTok; }

hipError_t launch_aux(const AuxArgs& a, hipStream_t st) {
  const int nblk = (a.alpha == 0.0f) ? 0 : aux_num_blocks(a.T);
  if (nblk > 0)
    hipLaunchKernelGGL(aux_partial_kernel, dim3(nblk), dim3(256), 0, st, a.probs, a.T, a.E, a.ws_partial);
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(kAuxFin), 0, st, a.ws_partial, nblk, a.counts, a.T, a.E, a.k,
                     a.alpha, a.aux_out);
  return hipGetLastError();
}

template <typename TX>
void launch_combine_bwd_t(const CombineBwdArgs& a, hipStream_t st) {
  const int tok_blocks = (a.T + 3) / 4;
  const GroupRank job{a.offsets, a.E, a.shared_rows, a.has_shared, a.order};
  const dim3 g(tok_blocks + (a.order ? 1 : 0)), b(256);
#define MOE_LAUNCH(KM)                                                                                   \
  hipLaunchKernelGGL((combine_bwd_narrow_kernel<TX, KM>), g, b, 0, st, (const TX*)a.dy, (const TX*)a.y_perm, \
                     a.slot, a.topk_w, (TX*)a.dO, a.dg, a.T, a.d, a.k, job)
  if (a.k <= 1) MOE_LAUNCH(1);
  else if (a.k <= 2) MOE_LAUNCH(2);
  else if (a.k <= 4) MOE_LAUNCH(4);
  else if (a.k <= kWideK) MOE_LAUNCH(8);
  else
    hipLaunchKernelGGL((combine_bwd_wide_kernel<TX>), g, b, 0, st, (const TX*)a.dy, (const TX*)a.y_perm, a.slot,
                       a.topk_w, (TX*)a.dO, a.dg, a.T, a.d, a.k, job);
#undef MOE_LAUNCH
}

hipError_t launch_combine_bwd(const CombineBwdArgs& a, hipStream_t st) {
  if (a.dtype == MOE_DT_BF16) launch_combine_bwd_t<uint16_t>(a, st);
  else launch_combine_bwd_t<float>(a, st);
  return hipGetLastError();
}

hipError_t launch_dlogits(const DlogitsArgs& a, hipStream_t st) {
  int64_t blocks = (a.T + 3) / 4;
  int nsw = 0, chunk = 0;
  if (a.gx) {  // extra workgroups: the weight split and the row ranges
    nsw = router_dw_splits(a.T, a.E, a.d);
    chunk = (a.T + nsw - 1) / nsw;
    const int64_t nw = (int64_t)a.kp * (a.d / 8) > nsw + 1 ? (int64_t)a.kp * (a.d / 8) : nsw + 1;
    blocks += (nw + 255) / 256;
  }
  hipLaunchKernelGGL(dlogits_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a.probs, a.topk_idx, a.topk_w, a.dg,
                     a.counts, a.dlogits, a.T, a.E, a.k, a.gate, a.renorm, a.alpha, a.gx, a.gw, a.kp, a.w_router,
                     a.wsplit, a.offs, a.d, nsw, chunk);
  return hipGetLastError();
}

// dW_r is split over the token axis: chunks of at most 1024 tokens (each chunk
// is summed sequentially in fp32, the chunk sums in a fixed order), and enough
// chunks that the split kernel has about 1024 workgroups.
static int router_grad_chunk(int T, int E, int d) {
  const int tiles = ((E + kRG - 1) / kRG) * ((d + kRG - 1) / kRG);
  const int want = (1024 + tiles - 1) / tiles;
  int chunk = (T + want - 1) / want;
  chunk = (chunk + 15) / 16 * 16;
  if (chunk > 1024) chunk = 1024;
  if (chunk < 64) chunk = 64;
  return chunk;
}

int router_grad_splits(int T, int E, int d) {
  const int c = router_grad_chunk(T, E, d);
  return (T + c - 1) / c;
}

hipError_t launch_router_grads(const RouterGradArgs& a, hipStream_t st) {
  const int chunk = router_grad_chunk(a.T, a.E, a.d);
  const int ns = router_grad_splits(a.T, a.E, a.d);
  const int tiles = ((a.E + kRG - 1) / kRG) * ((a.d + kRG - 1) / kRG);
  const int64_t n = (int64_t)a.E * a.d;
  if (a.dtype == MOE_DT_BF16) {
    // the grouped matmul on exactly split fp32 operands
    const hipError_t e = launch_router_dw_gemm(a, st);
    if (e != hipSuccess) return e;
    return launch_router_dx_gemm(a, st);
  }
  if (ns > 0)
    hipLaunchKernelGGL(gemm_tn_split_kernel<float>, dim3(tiles, ns), dim3(256), 0, st, a.dlogits, (int64_t)a.E,
                       (const float*)a.x, (int64_t)a.d, a.E, a.d, a.T, chunk, a.ws_partial);
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.ws_partial, ns, n,
                     a.dw_router);
  const int tiles2 = ((a.T + kRG - 1) / kRG) * ((a.d + kRG - 1) / kRG);
  if (tiles2 > 0)
    hipLaunchKernelGGL(gemm_nn_f32_kernel, dim3(tiles2), dim3(256), 0, st, a.dlogits, a.w_router, a.dx_router, a.T,
                     a.d, a.E);
  return hipGetLastError();
}

template <typename TX>
void launch_unpermute_bwd_t(const UnpermuteArgs& a, hipStream_t st) {
  const dim3 g((a.T + 3) / 4), b(256);
#define MOE_LAUNCH(KM)                                                                                     \
  hipLaunchKernelGGL((unpermute_bwd_narrow_kernel<TX, KM>), g, b, 0, st, (const TX*)a.dy, (const TX*)a.dX_perm, \
                     a.slot, a.dx_router, (const TX*)a.dx_shared, (TX*)a.dx, a.T, a.d, a.k)
  if (a.k <= 1) MOE_LAUNCH(1);
  else if (a.k <= 2) MOE_LAUNCH(2);
  else if (a.k <= 4) MOE_LAUNCH(4);
  else if (a.k <= kWideK) MOE_LAUNCH(8);
  else
    hipLaunchKernelGGL((unpermute_bwd_wide_kernel<TX>), g, b, 0, st, (const TX*)a.dy, (const TX*)a.dX_perm, a.slot,
                       a.dx_router, (const TX*)a.dx_shared, (TX*)a.dx, a.T, a.d, a.k);
#undef MOE_LAUNCH
}

hipError_t launch_unpermute_bwd(const UnpermuteArgs& a, hipStream_t st) {
  if (a.dtype == MOE_DT_BF16) launch_unpermute_bwd_t<uint16_t>(a, st);
  else launch_unpermute_bwd_t<float>(a, st);
  return hipGetLastError();
}

}  // namespace moe
