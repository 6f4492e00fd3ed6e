// Reference oracle for the token-routed MoE layer (forward and backward).
//
// TEST INFRASTRUCTURE ONLY. This file is the slow, plain CPU statement of what
// the layer computes. Only the test suite, the smoke check and the CPU-baseline
// leg of the benchmark may load it. The GPU library never links, calls or
// includes it, and it includes nothing from the GPU library.
//
// Pages cited (by title):
//   [SW]   "Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散"
//          (ta-paperlens.web.app explainer of the Switch Transformer paper)
//   [WIKI] "Mixture-of-Experts" (notes.yuuk.io concept page)
//
// Precision modes (argument `mode` everywhere):
//   0  exact: every value stays in double and nothing is rounded. The router
//      logits are double sums too. This mode exists for finite differences.
//   1  fp32 layer: the router contract below, and every stored tensor is
//      rounded to fp32 at the rounding points.
//   2  bf16 layer: the router contract below, and every stored activation,
//      expert output and gradient is rounded to bf16 (round to nearest even)
//      at the rounding points. The router stays fp32.
// All floating arrays cross this interface as double. In modes 1 and 2 the
// inputs hold values that are exactly representable in the layer's storage type.
//
// Rounding points: the pre-activation(s) and the activation saved by the first
// expert matmul, each expert output row, the layer output, the scaled upstream
// gradient fed to each expert, the activation gradient, the expert input
// gradient, each weight gradient and the final input gradient. Between rounding
// points all arithmetic is double.
//
// Router contract (modes 1 and 2). The pages fix the router to float32
// ([SW] section on the three stabilisation measures) but not the order of the
// sum, and a bit-exact routing decision needs one. Logit h[t,e] is the fp32
// sum over j = 0..d-1 in ascending order of single-rounded fused multiply-adds,
// starting from +0.0f; an optional per-expert offset is then added with one
// fp32 add. The sigmoid gate is 1/(1 + exp_c(-h)) with fp32 add and division,
// where exp_c is the fixed-operation exponential below (Cody-Waite range
// reduction, Cody & Waite 1980, then a degree-7 Taylor polynomial in Horner form).
// The square-root-softplus gate is sqrt(max(h, 0) + log1p_c(exp_c(-|h|))) with
// one fp32 add and a correctly rounded fp32 square root, where log1p_c is the
// fixed-operation log(1 + u) below (the inverse-hyperbolic-tangent series).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

#include <omp.h>

#pragma STDC FP_CONTRACT OFF

namespace {

enum { MODE_EXACT = 0, MODE_F32 = 1, MODE_BF16 = 2 };
enum { GATE_SOFTMAX = 0, GATE_SIGMOID_BIAS = 1, GATE_SQRT_SOFTPLUS_BIAS = 2 };
enum { ACT_RELU = 0, ACT_SWIGLU = 1 };

// Round a double to the nearest bf16 value (ties to even), by scaling the
// significand to 8 bits. bf16 has fp32's exponent range: normals down to
// 2^-126, subnormals in steps of 2^-133, largest finite (2 - 2^-7) * 2^127.
double round_bf16(double v) {
  if (v == 0.0 || !std::isfinite(v)) return v;
  int e;
  std::frexp(v, &e);           // v = m * 2^e, 0.5 <= |m| < 1
  int q = e - 8;               // quantum exponent for 8 significant bits
  if (q < -133) q = -133;      // subnormal range has a fixed quantum
  double r = std::nearbyint(std::ldexp(v, -q));  // default mode: ties to even
  double out = std::ldexp(r, q);
  const double maxb = std::ldexp(255.0, 127 - 7);  // (2 - 2^-7) * 2^127
  if (std::fabs(out) > maxb) return v > 0 ? INFINITY : -INFINITY;
  return out;
}

double rnd(int mode, double v) {
  if (mode == MODE_F32) return (double)(float)v;
  if (mode == MODE_BF16) return round_bf16(v);
  return v;
}

// exp_c: the fixed-operation fp32 exponential used by the sigmoid gate.
// ln2 is split into a 16-bit-significand head and an fp32 tail; the Taylor
// coefficients are 1/k! rounded to fp32. The range is clamped so that the
// result is never an fp32 subnormal.
float exp_c(float x) {
  if (x > 86.0f) return INFINITY;
  if (x < -86.0f) return 0.0f;
  const float log2e = 1.44269504088896341f;
  const float ln2_hi = 0.693145751953125f;        // 0x3F317200
  const float ln2_lo = 1.42860682030941723e-6f;   // ln2 - ln2_hi
  float n = std::nearbyint(x * log2e);
  float r = std::fma(-n, ln2_hi, x);
  r = std::fma(-n, ln2_lo, r);
  const float c7 = 1.98412698412698413e-4f;  // 1/5040
  const float c6 = 1.38888888888888889e-3f;  // 1/720
  const float c5 = 8.33333333333333333e-3f;  // 1/120
  const float c4 = 4.16666666666666667e-2f;  // 1/24
  const float c3 = 1.66666666666666667e-1f;  // 1/6
  const float c2 = 0.5f;
  float p = c7;
  p = std::fma(p, r, c6);
  p = std::fma(p, r, c5);
  p = std::fma(p, r, c4);
  p = std::fma(p, r, c3);
  p = std::fma(p, r, c2);
  p = std::fma(p, r, 1.0f);
  p = std::fma(p, r, 1.0f);
  int ni = (int)n;  // within [-125, 125] after the clamp
  uint32_t bits = (uint32_t)(ni + 127) << 23;
  float scale;
  std::memcpy(&scale, &bits, 4);
  return p * scale;
}

float sigmoid_c(float h) {
  float e = exp_c(-h);
  float den = 1.0f + e;
  return 1.0f / den;
}

// log1p_c(u) for u in [0, 1]: log(1 + u) = 2 artanh(z) with z = u / (2 + u), so
// z lies in [0, 1/3], and artanh(z) = z + z^3/3 + z^5/5 + ... The series is cut
// after the z^15 term (the first dropped term is below 2e-9 of the sum at
// z = 1/3) and evaluated as z * P(z^2), P in Horner form with fp32 coefficients
// 2/(2i + 1). Every operation is one correctly rounded fp32 operation.
float log1p_c(float u) {
  const float z = u / (2.0f + u);
  const float z2 = z * z;
  float p = 0.133333333333333333f;       // 2/15
  p = std::fma(p, z2, 0.153846153846153846f);  // 2/13
  p = std::fma(p, z2, 0.181818181818181818f);  // 2/11
  p = std::fma(p, z2, 0.222222222222222222f);  // 2/9
  p = std::fma(p, z2, 0.285714285714285714f);  // 2/7
  p = std::fma(p, z2, 0.4f);                   // 2/5
  p = std::fma(p, z2, 0.666666666666666667f);  // 2/3
  p = std::fma(p, z2, 2.0f);
  return z * p;
}

// [WIKI] (cross-cutting finding on the three generations of gating functions):
// DeepSeek-V4 replaces the sigmoid by the square root of softplus. softplus(h) =
// log(1 + e^h) is evaluated as max(h, 0) + log(1 + e^-|h|), which never
// overflows; the square root is the correctly rounded fp32 one.
float sqrt_softplus_c(float h) {
  const float u = exp_c(-std::fabs(h));
  const float sp = (h > 0.0f ? h : 0.0f) + log1p_c(u);
  return std::sqrt(sp);
}

// softplus(v) = log(1 + e^v) in the same fixed fp32 operations as the
// square-root-softplus gate (without the square root).
float softplus_c(float v) {
  const float u = exp_c(-std::fabs(v));
  return (v > 0.0f ? v : 0.0f) + log1p_c(u);
}

double softplus_d(double v) { return std::max(v, 0.0) + std::log1p(std::exp(-std::fabs(v))); }
double sigmoid_d(double v) { return 1.0 / (1.0 + std::exp(-v)); }

// The gate's derivative written with the gate value s = g(h) (the backward
// only has the saved gate values):
//   sigmoid:            s (1 - s)
//   sqrt(softplus):     sigmoid(h) / (2 s) = (1 - exp(-s^2)) / (2 s), since
//                       exp(-softplus(h)) = 1 - sigmoid(h); 0 at s = 0 (its limit).
double gate_deriv(int gate, double s) {
  if (gate == GATE_SIGMOID_BIAS) return s * (1.0 - s);
  if (s <= 0.0) return 0.0;
  return -std::expm1(-s * s) / (2.0 * s);
}

}  // namespace

extern "C" {

// OpenMP threads of the parallel loops below (timing only; no arithmetic).
void orc_set_threads(int n) { omp_set_num_threads(n); }
int orc_get_threads() { return omp_get_max_threads(); }

double orc_round_bf16(double v) { return round_bf16(v); }

// Elementwise rounding of n values at a storage precision (mode as above).
void orc_round_array(int mode, int64_t n, const double* in, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = rnd(mode, in[i]);
}
float orc_exp_contract(float x) { return exp_c(x); }
float orc_sigmoid_contract(float x) { return sigmoid_c(x); }
float orc_log1p_contract(float x) { return log1p_c(x); }
float orc_softplus_contract(float x) { return softplus_c(x); }
float orc_sqrt_softplus_contract(float x) { return sqrt_softplus_c(x); }
double orc_gate_deriv(int gate, double s) { return gate_deriv(gate, s); }

// [SW] eq. (3): capacity = tokens per batch / number of experts * capacity
// factor, rounded up, evaluated in double in exactly this order.
// Returns -1 (no limit) when the capacity factor is not positive.
int orc_capacity(int T, int E, double cf) {
  if (cf <= 0.0) return -1;
  return (int)std::ceil((double)T / (double)E * cf);
}

// [SW] eq. (1), first half: router logits h = W_r . x, plus an optional fixed
// per-expert offset (the skew used by two workloads; it has no gradient).
void orc_logits(int mode, int T, int d, int E, const double* x, const double* Wr,
                const double* offset, double* h) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    for (int e = 0; e < E; ++e) {
      if (mode == MODE_EXACT) {
        double acc = 0.0;
        for (int j = 0; j < d; ++j) acc += x[(size_t)t * d + j] * Wr[(size_t)e * d + j];
        if (offset) acc += offset[e];
        h[(size_t)t * E + e] = acc;
      } else {
        float acc = 0.0f;
        for (int j = 0; j < d; ++j)
          acc = std::fma((float)x[(size_t)t * d + j], (float)Wr[(size_t)e * d + j], acc);
        if (offset) acc = acc + (float)offset[e];
        h[(size_t)t * E + e] = acc;
      }
    }
  }
}

// Gate and top-k selection.
//  softmax ([SW] eq. (1)): probs = softmax(h) over all experts; the selection
//    key is h itself (softmax is monotone, so the chosen set and its order are
//    those of p in exact arithmetic).
//  sigmoid + bias ([WIKI], bullets on sigmoid gating with a learnable expert
//    bias and on DeepSeek-V3's bias used only for the routing decision):
//    probs = s = sigmoid_c(h); key = s + b (one fp32 add); the bias takes no
//    part in the weights.
//  square root of softplus + bias ([WIKI], DeepSeek-V4's gate in place of the
//    sigmoid, the selection bias kept as for the sigmoid):
//    probs = s = sqrt_softplus_c(h); key = s + b as above.
// Selection: experts ordered by key descending, equal keys by index ascending;
// the first k are chosen and idx[t, 0..k-1] lists them in that order.
// Weights: without renormalisation w_r = p[e_r] ([SW] numpy sketch: gate is
// the largest probability); with renormalisation w_r = p[e_r] / sum_s p[e_s].
void orc_gate(int mode, int T, int E, int k, int gate, int renorm, const double* h,
              const double* sel_bias, double* probs, int* idx, double* w) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const double* ht = h + (size_t)t * E;
    double* pt = probs + (size_t)t * E;
    std::vector<double> key(E);
    if (gate == GATE_SOFTMAX) {
      double m = ht[0];
      for (int e = 1; e < E; ++e) m = std::max(m, ht[e]);
      double z = 0.0;
      for (int e = 0; e < E; ++e) z += std::exp(ht[e] - m);
      for (int e = 0; e < E; ++e) pt[e] = rnd(mode == MODE_EXACT ? 0 : 1, std::exp(ht[e] - m) / z);
      for (int e = 0; e < E; ++e) key[e] = ht[e];
    } else {
      for (int e = 0; e < E; ++e) {
        if (mode == MODE_EXACT) {
          const double hv = ht[e];
          pt[e] = gate == GATE_SIGMOID_BIAS
                      ? 1.0 / (1.0 + std::exp(-hv))
                      : std::sqrt(std::max(hv, 0.0) + std::log1p(std::exp(-std::fabs(hv))));
          key[e] = pt[e] + (sel_bias ? sel_bias[e] : 0.0);
        } else {
          float s = gate == GATE_SIGMOID_BIAS ? sigmoid_c((float)ht[e]) : sqrt_softplus_c((float)ht[e]);
          pt[e] = s;
          key[e] = sel_bias ? (double)(s + (float)sel_bias[e]) : (double)s;
        }
      }
    }
    std::vector<int> order(E);
    std::iota(order.begin(), order.end(), 0);
    std::sort(order.begin(), order.end(), [&](int a, int b) {
      if (key[a] != key[b]) return key[a] > key[b];
      return a < b;
    });
    double sum = 0.0;
    for (int r = 0; r < k; ++r) sum += pt[order[r]];
    for (int r = 0; r < k; ++r) {
      int e = order[r];
      idx[(size_t)t * k + r] = e;
      double v = renorm ? pt[e] / sum : pt[e];
      w[(size_t)t * k + r] = rnd(mode == MODE_EXACT ? 0 : 1, v);
    }
  }
}

// Softmax for expert-choice routing. Experts compare probabilities of different
// tokens, so the probabilities themselves decide the routing and need a fixed
// fp32 contract: m = max_j h_j; e_j = exp_c(h_j - m) (one fp32 subtraction);
// z = sum of e_j in ascending j with fp32 adds from +0; p_j = e_j / z (one
// correctly rounded fp32 division). Mode 0 uses the plain double softmax.
void orc_softmax_ec(int mode, int T, int E, const double* h, double* probs) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const double* ht = h + (size_t)t * E;
    double* pt = probs + (size_t)t * E;
    if (mode == MODE_EXACT) {
      double m = ht[0];
      for (int e = 1; e < E; ++e) m = std::max(m, ht[e]);
      double z = 0.0;
      for (int e = 0; e < E; ++e) z += std::exp(ht[e] - m);
      for (int e = 0; e < E; ++e) pt[e] = std::exp(ht[e] - m) / z;
      continue;
    }
    float m = (float)ht[0];
    for (int e = 1; e < E; ++e) m = std::max(m, (float)ht[e]);
    std::vector<float> ev(E);
    float z = 0.0f;
    for (int e = 0; e < E; ++e) {
      ev[e] = exp_c((float)ht[e] - m);
      z = z + ev[e];
    }
    for (int e = 0; e < E; ++e) pt[e] = ev[e] / z;
  }
}

// Expert-choice routing ([WIKI], survey finding on MoE-based LLMs: the experts,
// not the tokens, take the top-k). Each expert e takes the C tokens of largest
// probs[t, e], equal values broken by the lower token index (C >= T: every
// token). Its seats are listed in ascending token order: row = e * C' + rank,
// C' = min(C, T). Token tables have one column per expert:
//   slot[t, e] = row, or -1 if e did not take t;  w[t, e] = probs[t, e] or 0.
// counts[e] = C' (rows of expert e), offsets[e] = e * C', row_token[row] = t.
void orc_expert_choice(int T, int E, int C, const double* probs, int* slot, double* w, int* row_token,
                       int* counts, int* offsets) {
  const int Cp = std::min(C, T);
  for (int e = 0; e < E; ++e) {
    std::vector<int> order(T);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
      const double pa = probs[(size_t)a * E + e], pb = probs[(size_t)b * E + e];
      if (pa != pb) return pa > pb;
      return a < b;
    });
    std::vector<int> chosen(order.begin(), order.begin() + Cp);
    std::sort(chosen.begin(), chosen.end());
    for (int t = 0; t < T; ++t) {
      slot[(size_t)t * E + e] = -1;
      w[(size_t)t * E + e] = 0.0;
    }
    for (int r = 0; r < Cp; ++r) {
      const int t = chosen[r], row = e * Cp + r;
      slot[(size_t)t * E + e] = row;
      w[(size_t)t * E + e] = probs[(size_t)t * E + e];
      row_token[row] = t;
    }
    counts[e] = Cp;
    offsets[e] = e * Cp;
  }
  offsets[E] = E * Cp;
}

// [SW] section on expert capacity: a fixed number of seats per expert, filled
// in token order; tokens beyond it skip the expert and ride the residual.
// pos(t, r) = number of assignments (t', r') with t' < t (a token's k experts
// are distinct) routed to the same expert; kept iff pos < C (C < 0: no limit).
// counts = assignments per expert before drops; offsets = exclusive prefix sum
// of kept rows per expert; slot = offsets[e] + pos for kept pairs, -1 else;
// row_token[slot] = t.
void orc_positions(int T, int k, int E, int C, const int* idx, int* counts,
                   int* offsets, int* slot, int* row_token) {
  std::vector<int> pos((size_t)T * k);
  std::vector<int> cnt(E, 0);
  for (int t = 0; t < T; ++t)
    for (int r = 0; r < k; ++r) {
      int e = idx[(size_t)t * k + r];
      pos[(size_t)t * k + r] = cnt[e]++;
    }
  for (int e = 0; e < E; ++e) counts[e] = cnt[e];
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) {
    int kept = (C < 0) ? cnt[e] : std::min(cnt[e], C);
    offsets[e + 1] = offsets[e] + kept;
  }
  for (int t = 0; t < T; ++t)
    for (int r = 0; r < k; ++r) {
      int e = idx[(size_t)t * k + r];
      int p = pos[(size_t)t * k + r];
      bool keep = (C < 0) || (p < C);
      int s = keep ? offsets[e] + p : -1;
      slot[(size_t)t * k + r] = s;
      if (keep) row_token[s] = t;
    }
}

// [SW] eq. (4) and the numpy sketch after it: loss = alpha * E * sum_i f_i P_i,
// f_i = share of the T*k assignments sent to expert i (counted before the
// capacity step), P_i = mean router probability of expert i over the batch.
double orc_aux(int mode, int T, int E, int k, double alpha, const double* probs,
               const int* counts) {
  double L = 0.0;
  for (int i = 0; i < E; ++i) {
    double P = 0.0;
    for (int t = 0; t < T; ++t) P += probs[(size_t)t * E + i];
    P /= (double)T;
    double f = (double)counts[i] / ((double)T * (double)k);
    L += f * P;
  }
  L *= alpha * (double)E;
  return mode == MODE_EXACT ? L : (double)(float)L;
}

// One expert FFN over n rows ([SW] section on the FFN being replaced by N
// copies; the activation variants follow the workloads).
//  ReLU:   A = x W1^T (f wide),  H = max(A, 0),      Y = H W2^T
//  SwiGLU: A = x W1^T (2f wide: gate half then up half),
//          H = silu(A_gate) * A_up with silu(z) = z * sigmoid(z),  Y = H W2^T
// W1 is [f or 2f, d] row-major, W2 is [d, f]. A (saved) and H are rounded at
// the storage precision; H is formed from the unrounded pre-activations.
void orc_ffn_fwd(int mode, int n, int d, int f, int act, const double* X,
                 const double* W1, const double* W2, double* A, double* H, double* Y) {
  const int f1 = act == ACT_SWIGLU ? 2 * f : f;
#pragma omp parallel for schedule(dynamic, 1)
  for (int row = 0; row < n; ++row) {
    const double* x = X + (size_t)row * d;
    std::vector<double> a(f1);
    for (int i = 0; i < f1; ++i) {
      double acc = 0.0;
      const double* wi = W1 + (size_t)i * d;
      for (int j = 0; j < d; ++j) acc += wi[j] * x[j];
      a[i] = acc;
      A[(size_t)row * f1 + i] = rnd(mode, acc);
    }
    std::vector<double> hv(f);
    for (int i = 0; i < f; ++i) {
      double v;
      if (act == ACT_RELU) {
        v = a[i] > 0.0 ? a[i] : 0.0;
      } else {
        double g = a[i], u = a[f + i];
        v = g / (1.0 + std::exp(-g)) * u;
      }
      hv[i] = rnd(mode, v);
      H[(size_t)row * f + i] = hv[i];
    }
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      const double* wc = W2 + (size_t)c * f;
      for (int i = 0; i < f; ++i) acc += wc[i] * hv[i];
      Y[(size_t)row * d + c] = rnd(mode, acc);
    }
  }
}

// [SW] eq. (2) plus the residual pass-through of dropped tokens:
// y[t] = x[t] + sum over kept r of w[t,r] * y_perm[slot[t,r]] (+ y_shared[t]).
// The weights are not renormalised after a drop. The shared expert (when
// present) is added with weight 1 ([WIKI] bullet on shared experts).
void orc_combine(int mode, int T, int d, int k, const double* x, const double* y_perm,
                 const int* slot, const double* w, const double* y_shared, double* y) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < d; ++c) {
      double acc = x[(size_t)t * d + c];
      for (int r = 0; r < k; ++r) {
        int s = slot[(size_t)t * k + r];
        if (s >= 0) acc += w[(size_t)t * k + r] * y_perm[(size_t)s * d + c];
      }
      if (y_shared) acc += y_shared[(size_t)t * d + c];
      y[(size_t)t * d + c] = rnd(mode, acc);
    }
}

// Backward of the combine for loss L = sum_t <dy_t, y_t> (+ aux):
// dO[slot] = w * dy[t] (rounded; the gradient fed to the expert), and
// dg[t,r] = <dy[t], y_perm[slot]> for kept pairs, 0 for dropped ones
// ([SW] eq. (2): the router learns through the multiplication by p_i).
void orc_combine_bwd(int mode, int T, int d, int k, const double* dy, const double* y_perm,
                     const int* slot, const double* w, double* dO, double* dg) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int r = 0; r < k; ++r) {
      int s = slot[(size_t)t * k + r];
      if (s < 0) {
        dg[(size_t)t * k + r] = 0.0;
        continue;
      }
      double acc = 0.0;
      for (int c = 0; c < d; ++c) {
        acc += dy[(size_t)t * d + c] * y_perm[(size_t)s * d + c];
        dO[(size_t)s * d + c] = rnd(mode, w[(size_t)t * k + r] * dy[(size_t)t * d + c]);
      }
      dg[(size_t)t * k + r] = mode == MODE_EXACT ? acc : (double)(float)acc;
    }
}

// Backward through one expert for n rows, given the upstream dO rows and the
// saved pre-activation(s) A:
//  dH = dO W2;  ReLU: dA = dH * [A > 0]
//  SwiGLU: with g = A_gate, u = A_up, s = sigmoid(g):
//          dA_up = dH * g * s,   dA_gate = dH * u * s * (1 + g * (1 - s))
//  dX = dA W1 (over the f or 2f rows of W1).
void orc_ffn_bwd(int mode, int n, int d, int f, int act, const double* dO, const double* A,
                 const double* W1, const double* W2, double* dA, double* dX) {
  const int f1 = act == ACT_SWIGLU ? 2 * f : f;
#pragma omp parallel for schedule(dynamic, 1)
  for (int row = 0; row < n; ++row) {
    const double* go = dO + (size_t)row * d;
    const double* ar = A + (size_t)row * f1;
    std::vector<double> da(f1);
    for (int i = 0; i < f; ++i) {
      double dh = 0.0;
      for (int c = 0; c < d; ++c) dh += W2[(size_t)c * f + i] * go[c];
      if (act == ACT_RELU) {
        da[i] = rnd(mode, ar[i] > 0.0 ? dh : 0.0);
      } else {
        double g = ar[i], u = ar[f + i];
        double s = 1.0 / (1.0 + std::exp(-g));
        da[f + i] = rnd(mode, dh * g * s);
        da[i] = rnd(mode, dh * u * s * (1.0 + g * (1.0 - s)));
      }
    }
    for (int i = 0; i < f1; ++i) dA[(size_t)row * f1 + i] = da[i];
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int i = 0; i < f1; ++i) acc += da[i] * W1[(size_t)i * d + j];
      dX[(size_t)row * d + j] = rnd(mode, acc);
    }
  }
}

// Weight gradient of one expert: dW[i, j] = sum over the expert's n rows of
// G[row, i] * V[row, j]; all zeros when n == 0.
void orc_wgrad(int mode, int n, int M, int N, const double* G, const double* V, double* dW) {
#pragma omp parallel for schedule(static)
  for (int i = 0; i < M; ++i)
    for (int j = 0; j < N; ++j) {
      double acc = 0.0;
      for (int row = 0; row < n; ++row) acc += G[(size_t)row * M + i] * V[(size_t)row * N + j];
      dW[(size_t)i * N + j] = rnd(mode, acc);
    }
}

// Gradient of the loss with respect to the router logits h[t, :].
// Gate path ([SW] eq. (2): the output is scaled by the gate, so the router gets
// gradient through it), with dg[t,r] = dL/dw[t,r]:
//  softmax, no renorm:  dh_j = sum_r dg_r * p_{e_r} * (delta(j, e_r) - p_j)
//  softmax, renorm:     dh_{e_r} = w_r * (dg_r - sum_s w_s dg_s), 0 elsewhere
//  sigmoid-type gates s = g(h) (sigmoid, sqrt-softplus), with g' = gate_deriv(s):
//   no renorm:          dh_{e_r} = dg_r * g'(s_{e_r})
//   renorm:             dh_{e_r} = (dg_r - sum_s w_s dg_s) / sum_s s_{e_s} * g'(s_{e_r})
// Aux path ([SW] eq. (4): f is a constant, only P carries gradient):
//  dh_j += (alpha * E / T) * sum_i f_i * dp_i/dh_j, i.e.
//  softmax: (alpha E / T) * p_j * (f_j - sum_i f_i p_i);  sigmoid-type: (alpha E / T) f_j g'(s_j).
// The selection bias and the fixed logit offsets receive no gradient.
// T: tokens to process (rows of probs/idx/w/dg/dlogits); T_batch: the batch size
// that normalises f and P in the aux loss (equal to T for a whole batch).
void orc_router_dlogits(int T, int T_batch, int E, int k, int gate, int renorm, double alpha,
                        const double* probs, const int* idx, const double* w,
                        const double* dg, const int* counts, double* dlogits) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t) {
    const double* p = probs + (size_t)t * E;
    double* o = dlogits + (size_t)t * E;
    for (int j = 0; j < E; ++j) o[j] = 0.0;
    const int* it = idx + (size_t)t * k;
    const double* wt = w + (size_t)t * k;
    const double* gt = dg + (size_t)t * k;
    if (gate == GATE_SOFTMAX) {
      if (!renorm) {
        for (int r = 0; r < k; ++r) {
          int e = it[r];
          for (int j = 0; j < E; ++j) o[j] += gt[r] * p[e] * ((j == e ? 1.0 : 0.0) - p[j]);
        }
      } else {
        double sdot = 0.0;
        for (int r = 0; r < k; ++r) sdot += wt[r] * gt[r];
        for (int r = 0; r < k; ++r) o[it[r]] += wt[r] * (gt[r] - sdot);
      }
    } else {
      if (!renorm) {
        for (int r = 0; r < k; ++r) o[it[r]] += gt[r] * gate_deriv(gate, p[it[r]]);
      } else {
        double sdot = 0.0, ssum = 0.0;
        for (int r = 0; r < k; ++r) {
          sdot += wt[r] * gt[r];
          ssum += p[it[r]];
        }
        for (int r = 0; r < k; ++r) o[it[r]] += (gt[r] - sdot) / ssum * gate_deriv(gate, p[it[r]]);
      }
    }
    if (alpha != 0.0) {
      double c = alpha * (double)E / (double)T_batch;
      double fp = 0.0;
      for (int i = 0; i < E; ++i) fp += (double)counts[i] / ((double)T_batch * k) * p[i];
      for (int j = 0; j < E; ++j) {
        double fj = (double)counts[j] / ((double)T_batch * k);
        if (gate == GATE_SOFTMAX) o[j] += c * p[j] * (fj - fp);
        else o[j] += c * fj * gate_deriv(gate, p[j]);
      }
    }
  }
}

// dW_r[e, j] = sum_t dlogits[t, e] * x[t, j] (stored fp32 outside mode 0);
// dx_router[t, j] = sum_e dlogits[t, e] * W_r[e, j] (kept in double; it is a
// term of dx, which is rounded once).
void orc_router_grads(int mode, int T, int d, int E, const double* dlogits, const double* x,
                      const double* Wr, double* dWr, double* dx_router) {
#pragma omp parallel for schedule(static)
  for (int e = 0; e < E; ++e)
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int t = 0; t < T; ++t) acc += dlogits[(size_t)t * E + e] * x[(size_t)t * d + j];
      dWr[(size_t)e * d + j] = mode == MODE_EXACT ? acc : (double)(float)acc;
    }
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < d; ++j) {
      double acc = 0.0;
      for (int e = 0; e < E; ++e) acc += dlogits[(size_t)t * E + e] * Wr[(size_t)e * d + j];
      dx_router[(size_t)t * d + j] = acc;
    }
}

// [WIKI] (finding on Quantile Balancing, which restates DeepSeek-V3's rule):
// the selection bias moves by a fixed step against the load imbalance,
// b_j <- b_j + gamma * sign(mean load - l_j), where l_j = counts[j] is the
// number of assignments expert j received in the batch (before capacity drops)
// and the mean load is sum_i l_i / E. Since E > 0 the sign equals
// sign(sum_i l_i - E l_j), which is decided here exactly in integers. The step
// is one fp32 add: b + gamma, b - gamma, or b unchanged. Bias values cross the
// interface as double holding fp32 values.
void orc_bias_update(int E, const int* counts, double gamma, const double* bias_in, double* bias_out) {
  int64_t total = 0;
  for (int i = 0; i < E; ++i) total += counts[i];
  for (int j = 0; j < E; ++j) {
    const int64_t diff = total - (int64_t)E * counts[j];
    const float b = (float)bias_in[j], g = (float)gamma;
    bias_out[j] = diff > 0 ? (double)(b + g) : diff < 0 ? (double)(b - g) : (double)b;
  }
}

// [WIKI] (finding on Quantile Balancing, Kimi K3): each expert's selection
// bias is set from a quantile of routing margins at the target load
// q = T k / E (tokens times experts per token over experts), the margins taken
// against the top-(k+1) cutoff, and the result used from the next step on.
// Reading written out here (fp32 like the routing itself):
//   key[t, j] = s[t, j] + b[j] (s = the gate values in probs);
//   per token, with keys ordered descending (ties: lower index first), c_k and
//   c_k1 are the k-th and (k+1)-th keys; margin m[t, j] = key[t, j] - c_k1 if
//   j is among the first k, else key[t, j] - c_k. Moving b[j] alone by delta
//   keeps or wins token t for j exactly when m[t, j] + delta > 0 (up to ties).
//   Per expert, mu_1 >= mu_2 >= ... are its margins over the batch; with
//   q = ceil(T k / E) clamped to [1, T - 1], delta[j] = -(mu_q + mu_(q+1)) / 2,
//   so that exactly q margins clear it, and b[j] <- b[j] + delta[j]: one fp32
//   add of the two margins, a multiply by 0.5 (exact) and one fp32 subtraction.
// The page's histogram of margins is the distributed approximation of this
// quantile; one device computes it exactly. T < 2, or k >= E (every expert
// takes every token, nothing to balance), leaves the bias unchanged.
int qb_target(int T, int E, int k) {
  int64_t q = ((int64_t)T * k + E - 1) / E;
  if (q > T - 1) q = T - 1;
  if (q < 1) q = 1;
  return (int)q;
}

void orc_bias_quantile(int T, int E, int k, const double* probs, const double* bias_in, double* bias_out) {
  for (int j = 0; j < E; ++j) bias_out[j] = bias_in[j];
  if (T < 2 || k >= E) return;
  std::vector<float> m((size_t)T * E);
  for (int t = 0; t < T; ++t) {
    std::vector<float> key(E);
    for (int j = 0; j < E; ++j) key[j] = (float)probs[(size_t)t * E + j] + (float)bias_in[j];
    std::vector<int> order(E);
    std::iota(order.begin(), order.end(), 0);
    std::sort(order.begin(), order.end(), [&](int a, int b) {
      if (key[a] != key[b]) return key[a] > key[b];
      return a < b;
    });
    std::vector<char> sel(E, 0);
    for (int r = 0; r < k; ++r) sel[order[r]] = 1;
    const float ck = key[order[k - 1]];
    const float ck1 = key[order[k]];
    for (int j = 0; j < E; ++j) m[(size_t)t * E + j] = key[j] - (sel[j] ? ck1 : ck);
  }
  const int q = qb_target(T, E, k);
  for (int j = 0; j < E; ++j) {
    std::vector<float> col(T);
    for (int t = 0; t < T; ++t) col[t] = m[(size_t)t * E + j];
    std::sort(col.begin(), col.end(), [](float a, float b) { return a > b; });
    const float sum = col[q - 1] + col[q];
    const float half = sum * 0.5f;
    bias_out[j] = (double)((float)bias_in[j] - half);
  }
}

// ---------------------------------------------------------------- noisy top-k gating
// [WIKI] (cross-cutting findings on Shazeer et al. 2017): top-k sparse gating
// with noisy softmax, trained with an importance loss (dispersion of each
// expert's summed softmax weight) and a load loss (dispersion of a smoothed
// load estimate); total loss = main loss + alpha (importance + load). The page
// names these but does not print them; they are written out here as that
// paper defines them:
//   clean logits h = W_g x and noise logits n = W_noise x (one router matrix of
//   2E rows: h = rows 0..E-1, n = rows E..2E-1); eps ~ N(0, 1) is an input;
//   H = h + eps * softplus(n);
//   gate: softmax over the top-k of H (the softmax gate on H, renormalised);
//   Importance_e = sum_t G[t, e];  L_imp = CV(Importance)^2;
//   Load_e = sum_t Phi((h[t, e] - r[t, e]) / softplus(n[t, e])), where r[t, e]
//   is the k-th largest H[t, :] with e left out (the (k+1)-th key if e is
//   selected, the k-th otherwise); L_load = CV(Load)^2;
//   aux = alpha (L_imp + L_load); CV(v)^2 = population variance / mean^2
//   (0 for a zero mean).
// H is formed in fp32 as one multiply and one add with softplus_c (the routing
// decision depends on it); the losses and gradients are plain double math on
// those stored values, with the selection and the rivals taken from the fp32 H.
// Mode 0 keeps H in double.
void orc_noisy_logits(int mode, int T, int E, const double* logits2, const double* eps, double* H) {
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      const double h = logits2[(size_t)t * 2 * E + e], n = logits2[(size_t)t * 2 * E + E + e];
      const double ep = eps[(size_t)t * E + e];
      if (mode == MODE_EXACT) {
        H[(size_t)t * E + e] = h + ep * softplus_d(n);
      } else {
        const float sp = softplus_c((float)n);
        const float prod = (float)ep * sp;
        H[(size_t)t * E + e] = (double)((float)h + prod);
      }
    }
}

// per token: selected set (first k of H desc, index asc), the k-th and (k+1)-th
// expert; rival[e] = index whose H is the k-th largest with e left out
static void noisy_rivals(int E, int k, const double* Ht, std::vector<int>& rival, std::vector<char>& sel) {
  std::vector<int> order(E);
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int a, int b) {
    if (Ht[a] != Ht[b]) return Ht[a] > Ht[b];
    return a < b;
  });
  sel.assign(E, 0);
  for (int r = 0; r < k; ++r) sel[order[r]] = 1;
  rival.assign(E, -1);
  for (int e = 0; e < E; ++e) rival[e] = sel[e] ? (k < E ? order[k] : -1) : order[k - 1];
}

static double cv2(const std::vector<double>& v) {
  const int n = (int)v.size();
  double mean = 0.0;
  for (double x : v) mean += x;
  mean /= n;
  if (mean == 0.0) return 0.0;
  double var = 0.0;
  for (double x : v) var += (x - mean) * (x - mean);
  var /= n;
  return var / (mean * mean);
}
// d CV^2 / d v_e = 2 / (n mean^2) * (v_e - mean - var / mean)
static void cv2_grad(const std::vector<double>& v, std::vector<double>& g) {
  const int n = (int)v.size();
  double mean = 0.0;
  for (double x : v) mean += x;
  mean /= n;
  g.assign(n, 0.0);
  if (mean == 0.0) return;
  double var = 0.0;
  for (double x : v) var += (x - mean) * (x - mean);
  var /= n;
  for (int e = 0; e < n; ++e) g[e] = 2.0 / (n * mean * mean) * (v[e] - mean - var / mean);
}

static double phi_cdf(double z) { return 0.5 * std::erfc(-z / std::sqrt(2.0)); }
static double phi_pdf(double z) { return std::exp(-0.5 * z * z) / std::sqrt(2.0 * M_PI); }

// Importance and load (per expert) of a batch; returns aux = alpha (CV^2 + CV^2).
double orc_noisy_aux(int mode, int T, int E, int k, const double* logits2, const double* eps, const int* idx,
                     const double* w, double alpha, double* imp_out, double* load_out) {
  std::vector<double> H((size_t)T * E);
  orc_noisy_logits(mode, T, E, logits2, eps, H.data());
  std::vector<double> imp(E, 0.0), load(E, 0.0);
  std::vector<int> rival;
  std::vector<char> sel;
  for (int t = 0; t < T; ++t) {
    for (int r = 0; r < k; ++r) imp[idx[(size_t)t * k + r]] += w[(size_t)t * k + r];
    if (k >= E) continue;  // every expert always taken: no rival, load term constant
    noisy_rivals(E, k, &H[(size_t)t * E], rival, sel);
    for (int e = 0; e < E; ++e) {
      const double h = logits2[(size_t)t * 2 * E + e], n = logits2[(size_t)t * 2 * E + E + e];
      const double z = (h - H[(size_t)t * E + rival[e]]) / softplus_d(n);
      load[e] += phi_cdf(z);
    }
  }
  for (int e = 0; e < E; ++e) {
    if (imp_out) imp_out[e] = imp[e];
    if (load_out) load_out[e] = load[e];
  }
  if (alpha == 0.0 || T == 0) return 0.0;
  return alpha * (cv2(imp) + (k >= E ? 0.0 : cv2(load)));
}

// Gradient of L = sum <dy, y> + aux with respect to the clean and noise logits,
// dlogits2 [T, 2E] = [dL/dh | dL/dn], from the gate gradient dg[t, r] = dL/dw[t, r]:
//   gate path: the softmax-over-top-k Jacobian on H with dg plus the importance
//   term alpha dCV^2/dImportance_e, then dH/dh = 1, dH/dn = eps sigmoid(n);
//   load path: for every (t, e), c = alpha dCV^2/dLoad_e phi(z) / softplus(n_e)
//   goes to h_e (+c), n_e (-c z sigmoid(n_e)) and to the rival j
//   (h_j: -c, n_j: -c eps_j sigmoid(n_j)).
void orc_noisy_dlogits(int mode, int T, int E, int k, const double* logits2, const double* eps, const int* idx,
                       const double* w, const double* dg, double alpha, double* dlogits2) {
  std::vector<double> imp(E), load(E), gimp, gload;
  orc_noisy_aux(mode, T, E, k, logits2, eps, idx, w, alpha, imp.data(), load.data());
  cv2_grad(imp, gimp);
  cv2_grad(load, gload);
  std::vector<double> H((size_t)T * E);
  orc_noisy_logits(mode, T, E, logits2, eps, H.data());
  std::vector<int> rival;
  std::vector<char> sel;
  for (int t = 0; t < T; ++t) {
    double* oh = dlogits2 + (size_t)t * 2 * E;
    double* on = oh + E;
    for (int j = 0; j < 2 * E; ++j) oh[j] = 0.0;
    const double* lh = logits2 + (size_t)t * 2 * E;
    const double* ln = lh + E;
    const double* ep = eps + (size_t)t * E;
    std::vector<double> dH(E, 0.0), gr(k);
    double sdot = 0.0;
    for (int r = 0; r < k; ++r) {
      gr[r] = dg[(size_t)t * k + r] + alpha * gimp[idx[(size_t)t * k + r]];
      sdot += w[(size_t)t * k + r] * gr[r];
    }
    for (int r = 0; r < k; ++r) dH[idx[(size_t)t * k + r]] += w[(size_t)t * k + r] * (gr[r] - sdot);
    for (int e = 0; e < E; ++e) {
      oh[e] += dH[e];
      on[e] += dH[e] * ep[e] * sigmoid_d(ln[e]);
    }
    if (alpha == 0.0 || k >= E) continue;
    noisy_rivals(E, k, &H[(size_t)t * E], rival, sel);
    for (int e = 0; e < E; ++e) {
      const double sp = softplus_d(ln[e]);
      const int j = rival[e];
      const double z = (lh[e] - H[(size_t)t * E + j]) / sp;
      const double c = alpha * gload[e] * phi_pdf(z) / sp;
      oh[e] += c;
      on[e] += -c * z * sigmoid_d(ln[e]);
      oh[j] -= c;
      on[j] -= c * ep[j] * sigmoid_d(ln[j]);
    }
  }
}

// dx[t] = dy[t] (residual) + sum over kept r of dX_perm[slot[t,r]]
//         + dx_router[t] (+ dx_shared[t]).
void orc_unpermute_bwd(int mode, int T, int d, int k, const double* dy, const double* dX_perm,
                       const int* slot, const double* dx_router, const double* dx_shared,
                       double* dx) {
#pragma omp parallel for schedule(static)
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < d; ++c) {
      double acc = dy[(size_t)t * d + c];
      for (int r = 0; r < k; ++r) {
        int s = slot[(size_t)t * k + r];
        if (s >= 0) acc += dX_perm[(size_t)s * d + c];
      }
      if (dx_router) acc += dx_router[(size_t)t * d + c];
      if (dx_shared) acc += dx_shared[(size_t)t * d + c];
      dx[(size_t)t * d + c] = rnd(mode, acc);
    }
}

}  // extern "C"
