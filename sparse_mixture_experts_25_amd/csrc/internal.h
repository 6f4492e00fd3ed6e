// Host-side launch interfaces between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct RouterArgs {
  const void* x;
  const float* w_router;
  const float* logit_offset;
  const float* sel_bias;
  float* probs;
  int32_t* topk_idx;
  float* topk_w;
  int T, d, E, k, gate, renorm, dtype;
};
hipError_t launch_router(const RouterArgs& a, hipStream_t st);
// gate value of RouterArgs asking for the logits only (probs <- h)
constexpr int kGateLogitsOnly = -1;
// Logits only into a.probs; *offset_applied says whether a.logit_offset was
// already added (the wide-d kernel adds it, the narrow one does not).
hipError_t launch_router_logits(const RouterArgs& a, hipStream_t st, bool* offset_applied);

struct RouteEcArgs {
  const void* x;
  const float* w_router;
  const float* logit_offset;
  float* probs;
  float* topk_w;
  int32_t* slot;
  int32_t* counts;
  int32_t* offsets;
  int32_t* row_token;
  void* x_perm;
  void* ws;  // ec_workspace_bytes(T, E)
  int T, d, E, Cp, dtype, elem_bytes;
};
size_t ec_workspace_bytes(int T, int E);
hipError_t launch_route_ec(const RouteEcArgs& a, hipStream_t st);
hipError_t launch_bias_update(const int32_t* counts, int E, float gamma, float* bias, hipStream_t st);
size_t qb_workspace_bytes(int T, int E);
// noisy top-k gating: routing over the stacked [W_g; W_noise] router
hipError_t launch_route_noisy(const RouterArgs& a, const float* noise, float* logits2, hipStream_t st);
struct NoisyArgs {
  const float* logits2;   // [T, 2E] clean | noise logits
  const float* noise;     // [T, E] eps
  const int32_t* topk_idx;
  const float* topk_w;
  float* ws;              // noisy_workspace_bytes(T, E)
  int T, E, k;
  float alpha;
};
int noisy_num_blocks(int T);
size_t noisy_workspace_bytes(int T, int E);
hipError_t launch_noisy_stats(const NoisyArgs& a, float* aux_out, hipStream_t st);
hipError_t launch_noisy_dlogits(const NoisyArgs& a, const float* dg, float* dl2, hipStream_t st);
hipError_t launch_bias_quantile(const float* probs, float* bias, int T, int E, int k, void* ws, hipStream_t st);

struct DispatchArgs {
  const void* x;
  const int32_t* topk_idx;
  int32_t* counts;
  int32_t* offsets;
  int32_t* slot;
  int32_t* row_token;
  void* x_perm;
  int32_t* ws_chunk;   // [nchunks, E] per-chunk expert counts
  int T, d, E, k, capacity, elem_bytes;
};
int dispatch_num_chunks(int T, int k);
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t st);
// The same launches with the per-chunk histograms in a file-scope device array
// of kDispatchScratchInts int32 (4 MiB) instead of a workspace; a.ws_chunk is
// ignored. Needs dispatch_fits_scratch(T, k, E).
constexpr int64_t kDispatchScratchInts = int64_t(1) << 20;
bool dispatch_fits_scratch(int T, int k, int E);
hipError_t launch_dispatch_noalloc(const DispatchArgs& a, hipStream_t st);

// One grouped matmul launch.
//  ragged-M kind (forward and input-gradient matmuls): for each group g,
//    C[rows_g, N] = A[rows_g, K] * op(B_g), rows_g = [off[g], off[g+1]) of A and C.
//    B_g is [N, K] (b_kcontig) or [K, N]. An optional extra dense group (the
//    shared expert) has rows [0, shared_rows) of A_sh / C_sh and weight B_sh.
//  ragged-K kind (weight gradients): for each group g,
//    C_g[M, N] = sum over rows in [off[g], off[g+1]) of A[row, :M]^T (x) B[row, :N];
//    the extra group sums over rows [0, shared_rows) of A_sh / B_sh into C_sh.
enum GemmEpi {
  EPI_STORE = 0,       // C = acc
  EPI_RELU_FWD = 1,    // C = acc (pre-activation), C2 = max(acc, 0)
  EPI_SWIGLU_FWD = 2,  // C = [gate | up] pre-activations, C2 = silu(gate) * up
  EPI_RELU_BWD = 3,    // C = acc * (X > 0)
  EPI_SWIGLU_BWD = 4,  // acc = dh; X = saved [gate | up]; C = [d gate | d up]
  EPI_STORE_F32 = 5,   // C (fp32) = acc (ragged-M, B MN-contiguous)
  // C = X + sum over r < slot_k with slot[row, r] >= 0 of Y[slot] + acc (+ Y_sh):
  // the input gradient of the layer (dy + expert input gradients + router
  // term + shared expert), rows = tokens (ragged-M, one group, B MN-contiguous)
  EPI_UNPERMUTE = 6,
  // top-1 combine in the down projection's epilogue (bf16, no shared expert,
  // B K-contiguous): C = acc (y_perm) and, for routed row r of token
  // t = row_tok[r], Yc[t] = X[t] + tok_w[t] * C[r] rounded once; extra
  // workgroups past copy_base copy X[t] to Yc[t] for the tokens t < copy_tokens
  // whose slot is -1
  EPI_COMBINE1 = 7,
};

struct GemmArgs {
  int kind;       // 0 ragged-M, 1 ragged-K
  int epi;
  int b_kcontig;  // ragged-M only
  int M, N, K;    // ragged-M: N, K fixed. ragged-K: M, N fixed.
  const int32_t* offsets;
  int E;
  int shared_rows;
  int has_shared;         // 1: an extra dense group exists (it may have 0 rows)
  int64_t max_rows;       // upper bound on the routed rows (sum over groups)
  const int32_t* order;   // ragged-K: processing order of the groups (nullable: 0..G-1)
  const void* A; int64_t lda;
  const void* B; int64_t ldb; int64_t strideB;
  const void* A_sh; const void* B_sh;
  void* C; int64_t ldc; int64_t strideC; void* C_sh;
  void* C2; int64_t ldc2; void* C2_sh;
  const void* X; int64_t ldx; const void* X_sh;
  int f;  // SwiGLU half width
  const int32_t* slot; int slot_k; const void* Y; const void* Y_sh;  // EPI_UNPERMUTE
  int row_cap;  // most rows any routed group can have (expert capacity), 0: no bound but max_rows
  // set by launch_gemm_bf16 when one grouped matmul runs as two launches:
  // 0 all groups; 1 only groups with at least split_rows rows (the extra dense
  // group counts shared_rows); 2 only groups with fewer
  int split_part; int split_rows;
  // Row maps of the routed groups (nullable; the shared group reads its rows
  // in place). ragged-M: row r of A is row a_rows[r] of A (the rows are
  // gathered as they are loaded, so no permuted copy is needed); ragged-K:
  // k-row r of B is row b_rows[r] of B. src_rows: rows of the mapped operand.
  const int32_t* a_rows; const int32_t* b_rows; int64_t src_rows;
  // EPI_COMBINE1 (X, ldx: x; slot: [T] slots of the top-1 choice)
  const int32_t* row_tok; const float* tok_w; void* Yc; int copy_tokens; int64_t copy_base;
};
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t st);
// order[0..E(+1)): the groups with rows sorted by row count, largest first
// (ties: lower index; the shared group, index E, counts shared_rows rows), with
// the groups without rows spread evenly between them (rank_groups_by_rows).
hipError_t launch_group_order(const int32_t* offsets, int E, int shared_rows, int has_shared, int32_t* order,
                              hipStream_t st);
hipError_t launch_gemm_f32(const GemmArgs& a, hipStream_t st);

struct CombineArgs {
  const void* x;
  const void* y_perm;
  const int32_t* slot;
  const float* topk_w;
  const void* y_shared;
  void* y;
  int T, d, k, dtype;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);

struct AuxArgs {
  const float* probs;
  const int32_t* counts;
  float* aux_out;
  float* ws_partial;  // [nblk, E]
  int T, E, k;
  float alpha;
};
int aux_num_blocks(int T);
hipError_t launch_aux(const AuxArgs& a, hipStream_t st);

// Backward pieces.
struct CombineBwdArgs {
  const void* dy;
  const void* y_perm;
  const int32_t* slot;
  const float* topk_w;
  void* dO;      // [R, d]
  float* dg;     // [T, k]
  int T, d, k, dtype;
  // when order is set, one extra workgroup also ranks the expert groups by row
  // count into order (as launch_group_order)
  const int32_t* offsets; int E, shared_rows, has_shared; int32_t* order;
};
hipError_t launch_combine_bwd(const CombineBwdArgs& a, hipStream_t st);

struct DlogitsArgs {
  const float* probs;
  const int32_t* topk_idx;
  const float* topk_w;
  const float* dg;
  const int32_t* counts;
  float* dlogits;  // [T, E] (nullable when gx is set)
  int T, E, k, gate, renorm;
  float alpha;
  // bf16 layers: also write every split operand of the router products
  // (RouterGradArgs::gx, gw, wsplit, router_dx_k(E) wide) and their row ranges
  // (offs), in extra workgroups for the weights, so no split kernel runs
  uint16_t* gx; uint16_t* gw; int kp;
  const float* w_router; uint16_t* wsplit; int32_t* offs; int d;
};
hipError_t launch_dlogits(const DlogitsArgs& a, hipStream_t st);

struct RouterGradArgs {
  const float* dlogits;  // [T, E]
  const void* x;         // [T, d] act
  const float* w_router; // [E, d]
  float* dw_router;      // [E, d]
  float* dx_router;      // [T, d]
  float* ws_partial;     // [nsplit, E, d]
  uint16_t* gx;          // bf16 [T, router_dx_k(E)] split dlogits for dx_router (bf16 layers)
  uint16_t* gw;          // bf16 [T, router_dx_k(E)] split dlogits for dW_router (bf16 layers)
  uint16_t* wsplit;      // bf16 [router_dx_k(E), d] split router weights (bf16 layers)
  int32_t* offs;         // [2 + router_dw_splits + 1] row ranges of the dx group and the dW chunks
  int T, d, E, dtype;
  // bf16 layers with k <= 2: the dx_router product also finishes the input
  // gradient, dx = dy + sum_kept dX_perm[slot] + dx_router (+ dx_shared), and
  // dx_router is not stored (dx non-null selects this)
  const void* dy; const int32_t* slot; int k; const void* dX_perm; const void* dX_sh; void* dx;
  int split_done;  // gx, gw, wsplit and offs already written (by the dlogits kernel)
};
// width of the split operands: 3E rounded up to 8
inline int router_dx_k(int E) { return (3 * E + 7) / 8 * 8; }
// token chunks of the matrix-core dW_router (each an fp32 partial of router_dx_k(E) x d)
int router_dw_splits(int T, int E, int d);
int router_grad_splits(int T, int E, int d);
hipError_t launch_router_grads(const RouterGradArgs& a, hipStream_t st);
// matrix-core router gradients for bf16 activations (split-fp32 operands);
// dw first (it also writes the split operands dx uses)
hipError_t launch_router_dw_gemm(const RouterGradArgs& a, hipStream_t st);
hipError_t launch_router_dx_gemm(const RouterGradArgs& a, hipStream_t st);

struct UnpermuteArgs {
  const void* dy;
  const void* dX_perm;
  const int32_t* slot;
  const float* dx_router;
  const void* dx_shared;
  void* dx;
  int T, d, k, dtype;
};
hipError_t launch_unpermute_bwd(const UnpermuteArgs& a, hipStream_t st);

}  // namespace moe
