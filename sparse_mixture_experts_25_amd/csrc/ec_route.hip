// Expert-choice routing: the experts pick their tokens.
//
// [WIKI] = "Mixture-of-Experts" (notes.yuuk.io), survey finding on MoE-based
// LLMs: in Expert Choice routing each expert, rather than each token, takes
// its top-k. Here expert e takes the C' = min(C, T) tokens of largest
// probability p[t, e] (C from the capacity formula of [SW] eq. (3)), equal
// probabilities broken by the lower token index, and seats them in token
// order at rows e*C' ... e*C' + C' - 1.
//
// Experts compare probabilities of different tokens, so p itself must be
// reproducible bit for bit: the softmax uses exp_c, an fp32 sum in ascending
// expert order and one correctly rounded division.
//
// Kernels (all on the caller's stream, scratch in the workspace):
//   1. router logits (the token-choice logits kernels, logits-only mode)
//   2. ec_softmax_kernel   lane = token: p in place in probs [T,E] and a
//                          transposed copy pT [E,T] for the column selection
//   3. ec_select_kernel    one workgroup per expert: exact C'-th largest key by
//                          a 4 x 8-bit radix select over pT[e], then a
//                          token-order compaction (ballots + per-wave counts)
//                          writing row_token and selpos [E,T] (row or -1)
//   4. ec_table_kernel     LDS transpose selpos -> slot [T,E]; topk_w [T,E]
//   5. gather_rows_kernel  x_perm[row] = x[row_token[row]]
// No atomics touch memory outside LDS; the LDS histogram counts are exact
// integers, so the result does not depend on the order of the atomic adds.
#include "common.h"
#include "gate_math.h"
#include "internal.h"

namespace moe {

namespace {

// p[t, :] = softmax of h[t, :] (+ offset) with the fixed-operation contract.
// One token per lane, one wave per workgroup (spreads small batches over the
// CUs); three passes over the row (max, sum, write).
__global__ __launch_bounds__(64) void ec_softmax_kernel(float* __restrict__ probs, const float* __restrict__ offset,
                                                        int T, int E, float* __restrict__ pT) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  if (t >= T) return;
  float* row = probs + (int64_t)t * E;
  float m = -__builtin_inff();
  for (int e = 0; e < E; ++e) {
    const float h = offset ? row[e] + offset[e] : row[e];
    m = fmaxf(m, h);
  }
  float z = 0.0f;
  for (int e = 0; e < E; ++e) {
    const float h = offset ? row[e] + offset[e] : row[e];
    z = z + exp_c(h - m);
  }
  for (int e = 0; e < E; ++e) {
    const float h = offset ? row[e] + offset[e] : row[e];
    const float p = exp_c(h - m) / z;
    row[e] = p;
    pT[(int64_t)e * T + t] = p;
  }
}

constexpr int kSel = 1024;  // threads of a selection workgroup

// Column selection for expert e = blockIdx.x. Probabilities are >= +0, so their
// fp32 bit patterns order like the values; the radix select walks the bytes of
// the key from the top, narrowing to the exact key K* of rank C' (1-based,
// descending). The tokens with key > K* and the first `need` tokens with key
// == K* (in token order) are taken.
__global__ __launch_bounds__(kSel) void ec_select_kernel(const float* __restrict__ pT, int T, int E, int Cp,
                                                         int32_t* __restrict__ selpos,
                                                         int32_t* __restrict__ row_token,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t weq[kSel / 64], wsel[kSel / 64];
  __shared__ uint32_t sh_digit, sh_need;
  const int e = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t* keys = reinterpret_cast<const uint32_t*>(pT + (int64_t)e * T);
  uint32_t prefix = 0, mask = 0, need = (uint32_t)Cp;
  if (Cp > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int t = tid; t < T; t += kSel) {
        const uint32_t k = keys[t];
        if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns bins 255-4l .. 252-4l; counts above a lane's bins by a scan
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
              sh_digit = 255u - 4u * lane - i;
              sh_need = need - above;
            }
            above += c[i];
          }
        }
      }
      __syncthreads();
      prefix |= sh_digit << shift;
      mask |= 255u << shift;
      need = sh_need;
    }
  }
  const uint32_t kstar = prefix;
  const int64_t rowbase = (int64_t)e * Cp;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint32_t base_eq = 0, base_sel = 0;
  for (int t0 = 0; t0 < T; t0 += kSel) {
    const int t = t0 + tid;
    const bool valid = t < T && Cp > 0;
    const uint32_t k = valid ? keys[t] : 0u;
    const bool eq = valid && k == kstar;
    const uint64_t beq = __ballot(eq);
    if (lane == 0) weq[wave] = (uint32_t)__popcll(beq);
    __syncthreads();
    uint32_t eq_before = base_eq + (uint32_t)__popcll(beq & lt), eq_round = 0;
    for (int w = 0; w < kSel / 64; ++w) {
      if (w < wave) eq_before += weq[w];
      eq_round += weq[w];
    }
    const bool sel = valid && (k > kstar || (eq && eq_before < need));
    const uint64_t bsel = __ballot(sel);
    if (lane == 0) wsel[wave] = (uint32_t)__popcll(bsel);
    __syncthreads();
    uint32_t pos = base_sel + (uint32_t)__popcll(bsel & lt), sel_round = 0;
    for (int w = 0; w < kSel / 64; ++w) {
      if (w < wave) pos += wsel[w];
      sel_round += wsel[w];
    }
    if (t < T) selpos[(int64_t)e * T + t] = sel ? (int32_t)(rowbase + pos) : -1;
    if (sel && pos < (uint32_t)Cp) row_token[rowbase + pos] = t;
    base_eq += eq_round;
    base_sel += sel_round;
    __syncthreads();
  }
  if (tid == 0) {
    counts[e] = Cp;
    offsets[e] = (int32_t)rowbase;
    if (e == E - 1) offsets[E] = (int32_t)((int64_t)E * Cp);
  }
}

// slot[t, e] = selpos[e, t]; topk_w[t, e] = probs[t, e] where taken, else 0.
// 64 x 64 tiles through LDS so both sides are read and written along rows.
__global__ __launch_bounds__(256) void ec_table_kernel(const int32_t* __restrict__ selpos,
                                                       const float* __restrict__ probs, int T, int E,
                                                       int32_t* __restrict__ slot, float* __restrict__ w) {
  __shared__ int32_t tile[64][65];
  const int tb = blockIdx.x * 64, eb = blockIdx.y * 64;
  const int c = threadIdx.x & 63;
  for (int r = threadIdx.x >> 6; r < 64; r += 4) {
    const int e = eb + r, t = tb + c;
    tile[r][c] = (e < E && t < T) ? selpos[(int64_t)e * T + t] : -1;
  }
  __syncthreads();
  for (int r = threadIdx.x >> 6; r < 64; r += 4) {
    const int t = tb + r, e = eb + c;
    if (t < T && e < E) {
      const int32_t s = tile[c][r];
      slot[(int64_t)t * E + e] = s;
      w[(int64_t)t * E + e] = s >= 0 ? probs[(int64_t)t * E + e] : 0.0f;
    }
  }
}

// x_perm[row] = x[row_token[row]], one wave per row, 16-byte vectors.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ x,
                                                          const int32_t* __restrict__ row_token, int64_t rows,
                                                          int T, int64_t row_bytes, uint8_t* __restrict__ x_perm) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave;
  if (r >= rows) return;
  const int64_t t = row_token[r];
  if (t < 0 || t >= T) return;
  const int nvec = (int)(row_bytes / 16);
  for (int v = lane; v < nvec; v += 64)
    st128(x_perm + r * row_bytes + (int64_t)v * 16, ld128(x + t * row_bytes + (int64_t)v * 16));
}

}  // namespace

size_t ec_workspace_bytes(int T, int E) { return (size_t)T * E * 8; }

hipError_t launch_route_ec(const RouteEcArgs& a, hipStream_t st) {
  if (a.T == 0) {
    hipLaunchKernelGGL(ec_select_kernel, dim3(a.E), dim3(kSel), 0, st, (const float*)nullptr, 0, a.E, 0,
                       (int32_t*)nullptr, (int32_t*)nullptr, a.counts, a.offsets);
    return hipGetLastError();
  }
  RouterArgs r{a.x, a.w_router, a.logit_offset, nullptr, a.probs, nullptr, nullptr, a.T, a.d, a.E, 0,
               kGateLogitsOnly, 0, a.dtype};
  bool offset_applied = false;
  hipError_t e = launch_router_logits(r, st, &offset_applied);
  if (e != hipSuccess) return e;
  float* pT = reinterpret_cast<float*>(a.ws);
  int32_t* selpos = reinterpret_cast<int32_t*>(pT + (int64_t)a.T * a.E);
  hipLaunchKernelGGL(ec_softmax_kernel, dim3((a.T + 63) / 64), dim3(64), 0, st, a.probs,
                     offset_applied ? nullptr : a.logit_offset, a.T, a.E, pT);
  hipLaunchKernelGGL(ec_select_kernel, dim3(a.E), dim3(kSel), 0, st, pT, a.T, a.E, a.Cp, selpos, a.row_token,
                     a.counts, a.offsets);
  hipLaunchKernelGGL(ec_table_kernel, dim3((a.T + 63) / 64, (a.E + 63) / 64), dim3(256), 0, st, selpos, a.probs,
                     a.T, a.E, a.slot, a.topk_w);
  const int64_t rows = (int64_t)a.E * a.Cp;
  if (rows > 0 && a.x_perm)  // without x_perm the matmuls read the rows through row_token
    hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                       (const uint8_t*)a.x, a.row_token, rows, a.T, (int64_t)a.d * a.elem_bytes,
                       (uint8_t*)a.x_perm);
  return hipGetLastError();
}

}  // namespace moe
