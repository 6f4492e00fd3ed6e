// Quantile Balancing of the selection bias.
//
// [WIKI] = "Mixture-of-Experts" (notes.yuuk.io), finding on Quantile
// Balancing (Kimi K3): each expert's bias comes from a quantile of routing
// margins at the target load q = T k / E, the margins taken against the
// top-(k+1) cutoff, and is applied from the next step on. Reading:
//   key[t, j] = s[t, j] + b[j] (fp32, the routing keys of the sigmoid-type gates);
//   c_k, c_k1 = the k-th and (k+1)-th keys of token t (descending, lower index
//   first on ties); margin m[t, j] = key - c_k1 if j is among the first k, else
//   key - c_k, so that moving b[j] alone by delta keeps or wins token t for j
//   exactly when m + delta > 0;
//   q = ceil(T k / E) clamped to [1, T - 1]; mu_q, mu_(q+1) = the q-th and
//   (q+1)-th largest margins of expert j; b[j] -= (mu_q + mu_(q+1)) * 0.5.
// The page approximates the quantile by margin histograms reduced across
// devices; on one device it is computed exactly.
//
// Kernels:
//   1. qb_cut_kernel     one wave per token: k+1 rounds of a wave argmax on
//                        (key desc, index asc) give c_k, c_k1 and the index of
//                        the k-th selected expert
//   2. qb_margin_kernel  64 x 64 tiles: margins from probs, bias and the cuts,
//                        written transposed (mT [E, T]) through LDS
//   3. qb_select_kernel  one workgroup per expert: two exact radix selects
//                        (ranks q and q+1) over the order-preserving integer
//                        image of the margins, then the bias step
#include "common.h"
#include "internal.h"

// keys, margins and the bias step are single fp32 operations, as in the routing
#pragma clang fp contract(off)

namespace moe {

namespace {

struct Cut {
  float ck, ck1;
  int ik;  // index of the k-th selected expert
  int pad;
};

// selected(j) == key > c_k, or key == c_k and j <= i_k
__global__ __launch_bounds__(256) void qb_cut_kernel(const float* __restrict__ probs,
                                                     const float* __restrict__ bias, int T, int E, int k,
                                                     Cut* __restrict__ cut) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int QE = (E + 63) / 64;  // at most 8 (E <= 512)
  float key[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int e = lane + 64 * q;
    key[q] = (q < QE && e < E) ? probs[(int64_t)t * E + e] + bias[e] : -__builtin_inff();
  }
  uint32_t taken = 0;
  float ck = 0.0f, ck1 = 0.0f;
  int ik = 0;
  for (int r = 0; r <= k; ++r) {
    float bk = -__builtin_inff();
    int be = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = lane + 64 * q;
      if (q < QE && e < E && !(taken & (1u << q)) && (key[q] > bk || be == 0x7fffffff)) {
        bk = key[q];
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
    if (r == k) ck1 = bk;
  }
  if (lane == 0) cut[t] = Cut{ck, ck1, ik, 0};
}

// mT[j, t] = margin of expert j at token t, 64 tokens x 64 experts per block.
__global__ __launch_bounds__(256) void qb_margin_kernel(const float* __restrict__ probs,
                                                        const float* __restrict__ bias,
                                                        const Cut* __restrict__ cut, int T, int E,
                                                        float* __restrict__ mT) {
  __shared__ float tile[64][65];
  const int tb = blockIdx.x * 64, eb = blockIdx.y * 64;
  const int c = threadIdx.x & 63;
  for (int r = threadIdx.x >> 6; r < 64; r += 4) {
    const int t = tb + r, j = eb + c;
    float m = 0.0f;
    if (t < T && j < E) {
      const float key = probs[(int64_t)t * E + j] + bias[j];
      const Cut ct = cut[t];
      const bool sel = key > ct.ck || (key == ct.ck && j <= ct.ik);
      m = key - (sel ? ct.ck1 : ct.ck);
    }
    tile[r][c] = m;
  }
  __syncthreads();
  for (int r = threadIdx.x >> 6; r < 64; r += 4) {
    const int j = eb + r, t = tb + c;
    if (t < T && j < E) mT[(int64_t)j * T + t] = tile[c][r];
  }
}

constexpr int kSel = 1024;

// fp32 bit pattern -> unsigned key with the same order (larger float, larger key)
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Key of rank `rank` (1-based, descending) among the T keys of one column: a
// radix select over four 8-bit digits with an LDS histogram per digit.
__device__ uint32_t radix_rank_desc(const float* __restrict__ col, int T, uint32_t rank, uint32_t* hist,
                                    uint32_t* sh) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t prefix = 0, mask = 0, need = rank;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int t = tid; t < T; t += kSel) {
      const uint32_t k = order_key(col[t]);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t c[4], s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        c[i] = hist[255 - 4 * lane - i];
        s += c[i];
      }
      uint32_t incl = s;
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      uint32_t above = incl - s;
      if (above < need && need <= incl) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (above < need && need <= above + c[i]) {
            sh[0] = 255u - 4u * lane - i;
            sh[1] = need - above;
          }
          above += c[i];
        }
      }
    }
    __syncthreads();
    prefix |= sh[0] << shift;
    mask |= 255u << shift;
    need = sh[1];
    __syncthreads();  // sh and hist are reused by the next digit
  }
  return prefix;
}

__global__ __launch_bounds__(kSel) void qb_select_kernel(const float* __restrict__ mT, int T, int q,
                                                         float* __restrict__ bias) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sh[2];
  const int j = blockIdx.x;
  const float* col = mT + (int64_t)j * T;
  const float mq = order_value(radix_rank_desc(col, T, (uint32_t)q, hist, sh));
  const float mq1 = order_value(radix_rank_desc(col, T, (uint32_t)q + 1, hist, sh));
  if (threadIdx.x == 0) {
    const float half = (mq + mq1) * 0.5f;
    bias[j] = bias[j] - half;
  }
}

}  // namespace

size_t qb_workspace_bytes(int T, int E) { return (size_t)T * sizeof(Cut) + (size_t)T * E * 4 + 256; }

hipError_t launch_bias_quantile(const float* probs, float* bias, int T, int E, int k, void* ws, hipStream_t st) {
  if (T < 2 || k >= E) return hipSuccess;
  int64_t q = ((int64_t)T * k + E - 1) / E;
  if (q > T - 1) q = T - 1;
  if (q < 1) q = 1;
  Cut* cut = reinterpret_cast<Cut*>(ws);
  float* mT = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(ws) + ((size_t)T * sizeof(Cut) + 255) / 256 * 256);
  hipLaunchKernelGGL(qb_cut_kernel, dim3((T + 3) / 4), dim3(256), 0, st, probs, bias, T, E, k, cut);
  hipLaunchKernelGGL(qb_margin_kernel, dim3((T + 63) / 64, (E + 63) / 64), dim3(256), 0, st, probs, bias, cut, T, E,
                     mT);
  hipLaunchKernelGGL(qb_select_kernel, dim3(E), dim3(kSel), 0, st, mT, T, (int)q, bias);
  return hipGetLastError();
}

}  // namespace moe
