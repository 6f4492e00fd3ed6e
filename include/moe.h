/*
 * moe.h - C ABI of the MI355X (gfx950) token-routed Mixture-of-Experts layer.
 *
 * One layer, forward and backward, on one GPU. Every call enqueues HIP kernels
 * on the caller's stream and returns at once: no host synchronisation and no
 * device allocation. The calls keep no state between them (the opt-in timing
 * hook of moe_profile.h is per host thread), so they are re-entrant; the one
 * exception is moe_dispatch_noalloc, whose fixed scratch array is shared by
 * its calls on one GPU (see there). The caller
 * owns every buffer, including the tensors the forward produces and the
 * backward consumes.
 *
 * Pages cited by title:
 *   [SW]   "Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散"
 *          (ta-paperlens.web.app, explainer of the Switch Transformer paper)
 *   [WIKI] "Mixture-of-Experts" (notes.yuuk.io concept page)
 *   [LRMOE] LRMoE news item (ai-cafe.club), section "この記事のポイント"
 *
 * Conventions for every entry point
 *   - Pointers are device pointers unless stated otherwise; tensors are dense
 *     and row-major with the shapes given. `act` below means the activation
 *     storage type: bf16 (MOE_DT_BF16) or fp32 (MOE_DT_F32). Router tensors
 *     (w_router, probs, topk_w, logit_offset, sel_bias, dw_router) are fp32.
 *   - Device pointers must be 16-byte aligned. d_model and d_ff must be
 *     multiples of 8. One expert's weight matrix (f1 x d_model elements, f1 =
 *     d_ff, or 2 d_ff for SwiGLU) must be under 4 GiB: larger configs are
 *     MOE_ERR_UNSUPPORTED (the matmuls address it with 32-bit offsets).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   - Arguments are validated on the host before any HIP call; a bad argument
 *     returns an error and enqueues nothing. MOE_ERR_HIP reports a launch error
 *     taken from hipGetLastError after the launches. Kernels that run
 *     asynchronously report nothing back.
 *   - Where a call takes a workspace, `ws` must hold at least the
 *     `workspace_bytes` that moe_plan returns for the same config. Its contents
 *     need not be initialised and are clobbered.
 *   - Capacity mode (capacity_factor > 0) keeps at most C rows per expert;
 *     dropless mode (capacity_factor <= 0) keeps every assignment. max_rows
 *     (from moe_plan) bounds the number of kept rows; rows of the permuted
 *     buffers at or beyond the kept count are never read or written.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define MOE_OK 0
#define MOE_ERR_INVALID_ARG (-1)  /* null pointer, bad size, misalignment */
#define MOE_ERR_UNSUPPORTED (-2)  /* unknown gate / activation / dtype combination */
#define MOE_ERR_WORKSPACE (-3)    /* workspace missing or smaller than moe_plan says */
#define MOE_ERR_HIP (-4)          /* a kernel launch failed */

/* gates */
#define MOE_GATE_SOFTMAX 0        /* [SW] eq. (1); selection on the logits */
#define MOE_GATE_SIGMOID_BIAS 1   /* [WIKI] sigmoid gate + per-expert bias used only to select */
#define MOE_GATE_SQRT_SOFTPLUS_BIAS 2 /* [WIKI] sqrt(softplus) gate (DeepSeek-V4) + the same selection bias */
#define MOE_GATE_NOISY_TOPK 3     /* [WIKI] noisy top-k softmax gating (Shazeer et al. 2017); router has 2E rows,
                                     routed with moe_route_noisy; renormalize must be 1; E <= 256 */
/* routing ([WIKI] survey finding on MoE-based LLMs names expert-choice routing) */
#define MOE_ROUTING_TOKEN_CHOICE 0  /* each token takes its top_k experts (moe_route + moe_dispatch) */
#define MOE_ROUTING_EXPERT_CHOICE 1 /* each expert takes its C tokens (moe_route_ec); top_k must equal
                                       num_experts and every [T,k] table has one column per expert */
/* expert activations */
#define MOE_ACT_RELU 0
#define MOE_ACT_SWIGLU 1          /* silu(x Wg^T) * (x Wu^T); W1 stacks [Wg; Wu] */
/* activation / expert-weight storage types */
#define MOE_DT_F32 0
#define MOE_DT_BF16 1

/* Layer description. Field names follow the vocabulary of [SW] (section on
 * using the method in practice: num_experts, capacity_factor, expert capacity,
 * aux-loss coefficient). Host memory. */
typedef struct moe_config {
  int32_t num_tokens;       /* T: tokens in the batch */
  int32_t d_model;          /* d */
  int32_t d_ff;             /* f: expert hidden width (each half, for SwiGLU) */
  int32_t num_experts;      /* E: routed experts */
  int32_t top_k;            /* k: experts per token, 1 <= k <= E */
  float capacity_factor;    /* > 0: capacity mode ([SW] eq. (3)); <= 0: dropless; must be finite */
  int32_t renormalize;      /* 1: the k selected weights are divided by their sum */
  int32_t gate;             /* MOE_GATE_* */
  int32_t act;              /* MOE_ACT_* */
  int32_t dtype;            /* MOE_DT_*: activations and expert weights */
  float aux_alpha;          /* alpha of [SW] eq. (4); 0 disables the aux loss; must be finite */
  int32_t num_shared_experts; /* 0 or 1: an always-on expert added with weight 1 ([WIKI]) */
  int32_t routing;          /* MOE_ROUTING_*; expert choice needs the softmax gate, renormalize = 0,
                               aux_alpha = 0, capacity_factor > 0 and top_k = num_experts */
} moe_config;

/* Sizes derived from a config (host memory), filled by moe_plan. */
typedef struct moe_plan_info {
  int32_t expert_capacity;  /* C = ceil(T / E * capacity_factor) in double; -1 when dropless */
  int32_t f1;               /* width of the first expert matmul: f (ReLU) or 2f (SwiGLU) */
  int64_t max_rows;         /* rows the permuted buffers must hold: T*k, or min(T*k, E*C) */
  size_t workspace_bytes;   /* workspace any call of this config needs */
} moe_plan_info;

/* Tensors the forward produced, handed to the backward (device memory).
 * Shapes use R = max_rows and f1 from moe_plan. */
typedef struct moe_saved {
  const void* x;                 /* [T, d] act: layer input */
  const float* probs;            /* [T, E] router probabilities (softmax) or sigmoid scores */
  const int32_t* topk_idx;       /* [T, k] */
  const float* topk_w;           /* [T, k] */
  const int32_t* slot;           /* [T, k] row in the permuted buffers, -1 = dropped */
  const int32_t* expert_counts;  /* [E] assignments per expert before drops */
  const int32_t* expert_offsets; /* [E+1] first permuted row of each expert */
  const void* x_perm;            /* [R, d]  act, or NULL: routed rows read as x[row_token[r]] */
  const void* act_saved;         /* [R, f1] act: pre-activation(s); SwiGLU only (ReLU: may be NULL) */
  const void* h_saved;           /* [R, f]  act: activation fed to the second matmul */
  const void* y_perm;            /* [R, d]  act: expert outputs */
  const void* act_shared;        /* [T, f1] shared expert (NULL without one; ReLU: may be NULL) */
  const void* h_shared;          /* [T, f]  shared expert (NULL without one) */
  const float* noisy_logits;     /* [T, 2E] clean | noise logits (noisy gating only, else NULL) */
  const float* noise;            /* [T, E]  eps (noisy gating only, else NULL) */
  const int32_t* row_token;      /* [R] token of each routed row; needed when x_perm is NULL */
} moe_saved;

/* Layer parameters (device memory). */
typedef struct moe_weights {
  const float* w_router;  /* [E, d] fp32 */
  const void* w1;         /* [E, f1, d] act (SwiGLU: rows [0,f) gate, [f,2f) up) */
  const void* w2;         /* [E, d, f]  act */
  const void* ws1;        /* [f1, d] shared expert, NULL without one */
  const void* ws2;        /* [d, f]  shared expert, NULL without one */
} moe_weights;

/* Gradients written by moe_backward (device memory; every one is overwritten,
 * experts with no kept rows get zeros). */
typedef struct moe_grads {
  void* dx;          /* [T, d] act */
  float* dw_router;  /* [E, d] fp32 */
  void* dw1;         /* [E, f1, d] act */
  void* dw2;         /* [E, d, f] act */
  void* dws1;        /* [f1, d] act, shared expert only */
  void* dws2;        /* [d, f] act, shared expert only */
} moe_grads;

/* Validate a config and derive its sizes. Host only; enqueues nothing.
 * cfg, out: host pointers. */
int moe_plan(const moe_config* cfg, moe_plan_info* out);

/* Router: [SW] eq. (1) and the top-k choice of the section on routing.
 *   h[t,e] = sum_j x[t,j] * w_router[e,j] in fp32, ascending j, one fused
 *            multiply-add per term from +0 (this fixed order makes the routing
 *            reproducible bit for bit); plus logit_offset[e] (one fp32 add) when given.
 *   softmax gate: probs = softmax(h) over the E experts; selection key = h.
 *   sigmoid gate: probs = s = 1/(1 + exp_c(-h)) with exp_c the library's fixed
 *            fp32 exponential (Cody-Waite reduction + degree-7 Taylor); key = s + sel_bias[e].
 *   sqrt-softplus gate ([WIKI], finding on the gating functions: DeepSeek-V4
 *            replaces the sigmoid by sqrt(softplus)): probs = s =
 *            sqrt(max(h,0) + log1p_c(exp_c(-|h|))), one fp32 add and the correctly
 *            rounded fp32 square root; log1p_c is the library's fixed fp32 log(1+u)
 *            (artanh series of z = u/(2+u) through z^15); key = s + sel_bias[e].
 *   topk_idx[t,:] = the k experts of largest key, equal keys broken by the lower
 *            index, listed in that order. topk_w[t,r] = probs[t,e_r], divided by the
 *            sum over the k selected when cfg->renormalize.
 * x: [T,d] act. w_router: [E,d]. logit_offset, sel_bias: [E] or NULL (sel_bias
 * is used only by the sigmoid gate). Outputs probs [T,E], topk_idx [T,k], topk_w [T,k]. */
int moe_route(const moe_config* cfg, const void* x, const float* w_router,
              const float* logit_offset, const float* sel_bias, float* probs,
              int32_t* topk_idx, float* topk_w, void* stream);

/* Noisy top-k routing ([WIKI], findings on Shazeer et al. 2017: top-k sparse
 * gating with noisy softmax). The page names the method only; it follows that
 * paper:
 *   logits2[t, :] = [h | n]: the router logits of the 2E-row router
 *     (rows 0..E-1 = W_g, rows E..2E-1 = W_noise), each by the moe_route contract;
 *   H[t, e] = h + noise[t, e] * softplus_c(n), softplus_c(n) = max(n, 0) +
 *     log1p_c(exp_c(-|n|)) (the library's fixed fp32 functions), one fp32
 *     multiply and one fp32 add;
 *   then the softmax gate of moe_route on H with renormalisation: the k largest
 *     H (lower index on ties), weights = softmax over those k; probs = softmax(H).
 * w_router [2E, d]; noise [T, E] fp32, the N(0, 1) draws (an input). Outputs
 * logits2 [T, 2E] (kept for the loss and the backward), probs [T, E],
 * topk_idx [T, k], topk_w [T, k]. Requires cfg->gate == MOE_GATE_NOISY_TOPK. */
int moe_route_noisy(const moe_config* cfg, const void* x, const float* w_router, const float* noise,
                    float* logits2, float* probs, int32_t* topk_idx, float* topk_w, void* stream);

/* Importance and load losses of noisy top-k gating ([WIKI], findings on Shazeer
 * et al. 2017: total loss = main + alpha (importance loss + load loss), the
 * first the dispersion of each expert's summed gate, the second that of a
 * smoothed load estimate), as that paper defines them:
 *   Importance_e = sum_t topk_w over the tokens that selected e;
 *   Load_e = sum_t Phi((h[t,e] - r[t,e]) / softplus(n[t,e])), r[t,e] = the k-th
 *     largest H of token t with e left out (the (k+1)-th H if e is selected,
 *     else the k-th); no load term when k = E;
 *   aux = aux_alpha (CV^2(Importance) + CV^2(Load)), CV^2 = population variance /
 *     mean^2 (0 for a zero mean). Computed in fp32 in a fixed order.
 * Inputs as written by moe_route_noisy; aux_out: one fp32 on the device. Needs
 * the workspace. moe_aux_loss returns MOE_ERR_UNSUPPORTED for this gate. */
int moe_aux_noisy(const moe_config* cfg, const float* logits2, const float* noise, const int32_t* topk_idx,
                  const float* topk_w, float* aux_out, void* ws, size_t ws_bytes, void* stream);

/* Expert-choice routing and permutation in one call ([WIKI], survey finding on
 * MoE-based LLMs: the experts, not the tokens, take the top-k).
 *   h as in moe_route (+ logit_offset[e]); probs[t,:] = softmax(h[t,:]) with a
 *     fixed fp32 contract, since experts compare probabilities across tokens:
 *     m = max_e h; z = sum over ascending e of exp_c(h_e - m) (fp32 adds from +0);
 *     p_e = exp_c(h_e - m) / z (one correctly rounded division).
 *   Each expert e takes the C' = min(C, T) tokens of largest probs[t,e]
 *     (C = ceil(T / E * capacity_factor) in double, as in moe_plan), equal
 *     values broken by the lower token index; its rows are e*C' .. e*C'+C'-1,
 *     filled in ascending token order.
 *   slot[t,e] = row, or -1 if expert e did not take token t; topk_w[t,e] =
 *     probs[t,e] where taken, else 0; expert_counts[e] = C'; expert_offsets[e]
 *     = e*C'; row_token[row] = t; x_perm[row] = x[t] (bitwise copy).
 * The outputs feed moe_expert_ffn, moe_combine and moe_backward unchanged
 * (k = E; moe_backward needs no topk_idx in this mode). A token no expert took
 * gets y = x. Requires cfg->routing == MOE_ROUTING_EXPERT_CHOICE.
 * x [T,d] act, w_router [E,d]; outputs probs [T,E], topk_w [T,E], slot [T,E],
 * expert_counts [E], expert_offsets [E+1], row_token [E*C'], x_perm [E*C',d]
 * or NULL (no permuted copy: see moe_expert_ffn_rows). Needs the workspace. */
int moe_route_ec(const moe_config* cfg, const void* x, const float* w_router,
                 const float* logit_offset, float* probs, float* topk_w, int32_t* slot,
                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_token,
                 void* x_perm, void* ws, size_t ws_bytes, void* stream);

/* Capacity, positions and permutation: [SW] eq. (3) and the section on expert
 * capacity (seats fixed before the data is seen, overflow rides the residual),
 * with the compacted expert-contiguous layout of [LRMOE].
 *   pos(t,r) = number of earlier tokens t' < t routed to the same expert;
 *   kept iff pos < C (always in dropless mode).
 *   expert_counts[e] = assignments before drops; expert_offsets = exclusive
 *   prefix sum of kept rows (offsets[E] = kept total); slot[t,r] =
 *   offsets[e] + pos if kept else -1; row_token[slot] = t;
 *   x_perm[slot] = x[t] (bitwise copy).
 * topk_idx may come from moe_route or from the caller (values must lie in [0,E)).
 * Token-choice routing only (MOE_ERR_UNSUPPORTED otherwise), as is moe_route.
 * Outputs: expert_counts [E], expert_offsets [E+1], slot [T,k], row_token [R],
 * x_perm [R,d] act. x_perm may be NULL: only the positions are written (x may
 * then be NULL too), and the expert matmuls read each routed row from x
 * through row_token instead ([WIKI], cross-cutting findings on fusing dispatch
 * into the expert matmuls: moe_expert_ffn_rows, and moe_backward with
 * moe_saved.x_perm NULL). Needs the workspace. */
int moe_dispatch(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                 int32_t* expert_counts, int32_t* expert_offsets, int32_t* slot,
                 int32_t* row_token, void* x_perm, void* ws, size_t ws_bytes, void* stream);

/* moe_dispatch without a workspace, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). Same arguments (less ws, ws_bytes),
 * outputs and semantics as moe_dispatch, with the same kernels; its scratch
 * (the per-chunk expert histograms, ceil(T*k / 1024) * E int32) lives in a
 * fixed 4 MiB device array of the library, one per GPU, kept until the process
 * ends. Returns MOE_ERR_WORKSPACE, enqueuing nothing, when ceil(T*k / 1024) * E
 * exceeds 2^20 (e.g. T*k above 4M assignments at E = 256). It calls no
 * allocator: the first call on a device looks up the array's device address
 * (hipGetSymbolAddress, with that device current) and keeps it. Every call on
 * one GPU uses that GPU's one array: calls that may overlap on one GPU (other
 * streams, other threads) race and must be ordered by the caller. Nothing in
 * the array needs clearing between calls (each call writes what it reads). */
int moe_dispatch_noalloc(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                         int32_t* expert_counts, int32_t* expert_offsets, int32_t* slot,
                         int32_t* row_token, void* x_perm, void* stream);

/* Expert FFNs over the compacted rows (grouped matmul over ragged groups),
 * [SW] section on replacing the FFN by N expert copies; [LRMOE] variable-size
 * grouped GEMM. For each expert e and its rows r in [offsets[e], offsets[e+1]):
 *   ReLU:   act = x_perm W1_e^T, h = max(act, 0)
 *   SwiGLU: act = x_perm W1_e^T ([gate | up], 2f wide), h = silu(gate) * up
 *   y_perm = h W2_e^T
 * act and h are stored in the activation type (bf16: round to nearest even
 * from the fp32 accumulator; h is formed from the unrounded accumulators).
 * With ReLU, act_saved / act_shared are optional (NULL: not written): the
 * backward takes the derivative from the sign of h, and h > 0 exactly when
 * act > 0 (a value that rounds to zero gives zero in both).
 * With a shared expert, the same is computed for every token row of x with
 * ws1/ws2 into act_shared [T,f1], h_shared [T,f], y_shared [T,d]; those pointers
 * must be NULL without one. Inputs: x_perm [R,d], expert_offsets [E+1] (device,
 * as written by moe_dispatch), w1 [E,f1,d], w2 [E,d,f]. Outputs: act_saved
 * [R,f1], h_saved [R,f], y_perm [R,d]. Needs the workspace. */
int moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                   const void* w1, const void* w2, const void* x, const void* ws1,
                   const void* ws2, void* act_saved, void* h_saved, void* y_perm,
                   void* act_shared, void* h_shared, void* y_shared, void* ws,
                   size_t ws_bytes, void* stream);

/* moe_expert_ffn without the permuted copy: the dispatch step fused into the
 * first matmul's operand loads ([WIKI], cross-cutting findings: the fused
 * dispatch / first linear / activation / second linear / combine pipeline of
 * the MegaMoE and Mixture-of-Kittens kernels). Routed row r is read as
 * x[row_token[r]] (row_token [R] as written by moe_dispatch or moe_route_ec,
 * device memory); everything else, outputs included, is as in moe_expert_ffn,
 * and the results are bitwise the same. x [T,d] serves both the routed rows
 * and the shared expert. x must be under 4 GiB (T*d*sizeof(act) < 2^32,
 * MOE_ERR_UNSUPPORTED otherwise, as for moe_backward without x_perm): its rows
 * are addressed with 32-bit offsets. Needs the workspace. */
int moe_expert_ffn_rows(const moe_config* cfg, const void* x, const int32_t* row_token,
                        const int32_t* expert_offsets, const void* w1, const void* w2,
                        const void* ws1, const void* ws2, void* act_saved, void* h_saved,
                        void* y_perm, void* act_shared, void* h_shared, void* y_shared,
                        void* ws, size_t ws_bytes, void* stream);

/* Combine: [SW] eq. (2) plus the residual.
 *   y[t] = x[t] + sum over kept r of topk_w[t,r] * y_perm[slot[t,r]] (+ y_shared[t])
 * accumulated in fp32 and stored once in the activation type. A token whose
 * every choice was dropped gets y = x bit for bit. Weights are not
 * renormalised after drops. x [T,d], y_perm [R,d], slot [T,k], topk_w [T,k],
 * y_shared [T,d] or NULL; output y [T,d]. */
int moe_combine(const moe_config* cfg, const void* x, const void* y_perm, const int32_t* slot,
                const float* topk_w, const void* y_shared, void* y, void* stream);

/* moe_expert_ffn_rows with the combine of [SW] eq. (2) (plus the residual,
 * as in moe_combine) fused into the down projection's epilogue, for top-1
 * token-choice layers without a shared expert in bf16 ([WIKI], cross-cutting
 * findings: the fused dispatch / linear / activation / linear / combine
 * pipelines). With one choice per token, the routed row r = slot[t] is the only
 * expert row of token t, so the tile that computes y_perm[r] also writes
 *   y[t] = x[t] + topk_w[t] * y_perm[r]   (fp32, one rounding to bf16)
 * with no atomics; extra workgroups of the same launch write y[t] = x[t] for
 * the tokens whose choice was dropped (slot[t] == -1). y_perm, act_saved and
 * h_saved are as in moe_expert_ffn_rows, and y is bitwise moe_combine's result
 * for the same inputs. Inputs: x [T,d], row_token [R], expert_offsets [E+1],
 * slot [T,1] and topk_w [T,1] as written by moe_dispatch and moe_route, w1, w2
 * (device). Outputs: act_saved [R,f1] (ReLU: optional), h_saved [R,f],
 * y_perm [R,d], y [T,d] (16-byte aligned; must not overlap the inputs). Returns
 * MOE_ERR_UNSUPPORTED unless dtype is bf16, top_k is 1, there is no shared
 * expert and the routing is token choice; x must be under 4 GiB as for
 * moe_expert_ffn_rows. Needs the workspace. */
int moe_expert_ffn_combine(const moe_config* cfg, const void* x, const int32_t* row_token,
                           const int32_t* expert_offsets, const int32_t* slot, const float* topk_w,
                           const void* w1, const void* w2, void* act_saved, void* h_saved, void* y_perm,
                           void* y, void* ws, size_t ws_bytes, void* stream);

/* Switch load-balancing loss, [SW] eq. (4) and the numpy sketch after it:
 *   aux = alpha * E * sum_i f_i * P_i,  f_i = expert_counts[i] / (T*k) (counted
 *   before drops), P_i = mean over t of probs[t,i].
 * probs [T,E], expert_counts [E]; aux_out: one fp32 on the device. Writes 0
 * when aux_alpha == 0. Needs the workspace. */
int moe_aux_loss(const moe_config* cfg, const float* probs, const int32_t* expert_counts,
                 float* aux_out, void* ws, size_t ws_bytes, void* stream);

/* Aux-loss-free balancing step on the selection bias ([WIKI], finding on
 * Quantile Balancing, which restates DeepSeek-V3's fixed-step rule):
 *   sel_bias[j] <- sel_bias[j] + gamma * sign(mean load - expert_counts[j]),
 *   mean load = sum_i expert_counts[i] / E.
 * The sign is decided exactly (in 64-bit integers, as sign(sum - E * count));
 * the step is one fp32 add (b + gamma, b - gamma, or b unchanged). Call it after
 * moe_dispatch on the counts of the same batch; the updated bias steers the
 * next moe_route. Only cfg->num_experts is used (the config must still be
 * valid). expert_counts: [E] int32, non-negative (device). sel_bias: [E] fp32
 * (device), updated in place. gamma: finite and >= 0 (else MOE_ERR_INVALID_ARG). */
int moe_bias_update(const moe_config* cfg, const int32_t* expert_counts, float gamma,
                    float* sel_bias, void* stream);

/* Quantile Balancing of the selection bias ([WIKI], finding on Quantile
 * Balancing: the bias of each expert is set from the quantile of routing
 * margins at the target load, margins taken against the top-(k+1) cutoff, and
 * used from the next step on). With key[t,j] = probs[t,j] + sel_bias[j] (fp32)
 * and, per token, c_k and c_k1 its k-th and (k+1)-th keys (descending, lower
 * index first on ties):
 *   margin[t,j] = key - c_k1 if j is among the token's k selected experts,
 *                 key - c_k otherwise
 *   (moving sel_bias[j] alone by delta keeps or wins token t for j exactly when
 *   margin + delta > 0);
 *   q = ceil(T*k/E) clamped to [1, T-1]; mu_q >= mu_(q+1) the q-th and (q+1)-th
 *   largest margins of expert j;
 *   sel_bias[j] <- sel_bias[j] - (mu_q + mu_(q+1)) * 0.5   (fp32 add, exact halving,
 *   fp32 subtraction).
 * The page estimates the quantile from margin histograms reduced across
 * devices; here it is exact. T < 2 or top_k >= E leaves the bias unchanged.
 * probs: [T,E] the gate values moe_route wrote for this batch (sigmoid-type
 * gates only; softmax -> MOE_ERR_UNSUPPORTED). sel_bias: [E] fp32, updated in
 * place, to be used by the next moe_route. Needs the workspace. */
int moe_bias_quantile(const moe_config* cfg, const float* probs, float* sel_bias, void* ws,
                      size_t ws_bytes, void* stream);

/* Backward of the layer for the loss L = sum_t <dy[t], y[t]> + aux (aux term
 * only when aux_alpha != 0): [SW] eq. (2) (the gate multiplies the expert
 * output, so the router is trained through it) and eq. (4) (only P carries
 * gradient). Writes every field of *g:
 *   dx = dy + sum over kept r of dX_perm[slot] + dx_router (+ dx_shared)
 *   dw1, dw2 per expert from its rows (zeros for experts with no rows),
 *   dws1, dws2 for the shared expert, dw_router = dlogits^T x in fp32.
 * Noisy gating: dlogits is [T, 2E] (clean and noise logits: the gate path through
 * H = h + eps softplus(n), the importance loss through the gates and the load
 * loss through Phi, also to each token's rival expert); w_router and dw_router
 * are [2E, d]; s->noisy_logits and s->noise must be set.
 * The routed rows of x for dw1 come from s->x_perm, or, when it is NULL, from
 * s->x through s->row_token (gathered as they are loaded; bitwise the same).
 * dy: [T,d] act. s, w, g: host structs holding device pointers. Needs the workspace. */
int moe_backward(const moe_config* cfg, const void* dy, const moe_saved* s,
                 const moe_weights* w, const moe_grads* g, void* ws, size_t ws_bytes,
                 void* stream);

/* Static string naming a status code. */
const char* moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
