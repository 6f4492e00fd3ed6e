// C ABI of the MoE layer: argument validation, sizes, workspace carving and
// the launch sequence of each call. No allocation and no host synchronisation.
// State kept between calls: the opt-in stage-timing hook of moe_profile.h,
// which is per host thread (a call reads the hook of the thread that makes it),
// and, for moe_dispatch_noalloc only, its fixed device scratch array (one per
// GPU) with the cached per-device address of it (dispatch.hip).
#include <math.h>
#include <string.h>

#include "internal.h"
#include "../../include/moe.h"
#include "../../include/moe_profile.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int elem_bytes(const moe_config* c) { return c->dtype == MOE_DT_BF16 ? 2 : 4; }

int check_config(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->num_tokens < 0 || c->d_model < 8 || c->d_ff < 8) return MOE_ERR_INVALID_ARG;
  if (c->d_model % 8 || c->d_ff % 8) return MOE_ERR_INVALID_ARG;
  if (c->num_experts < 1 || c->top_k < 1 || c->top_k > c->num_experts) return MOE_ERR_INVALID_ARG;
  if (c->routing != MOE_ROUTING_TOKEN_CHOICE && c->routing != MOE_ROUTING_EXPERT_CHOICE) return MOE_ERR_UNSUPPORTED;
  const bool ec = c->routing == MOE_ROUTING_EXPERT_CHOICE;
  if (c->num_experts > 512 || (!ec && c->top_k > 64)) return MOE_ERR_UNSUPPORTED;
  if (ec) {
    // token tables carry one column per expert; capacity sets the seats
    if (c->top_k != c->num_experts || !(c->capacity_factor > 0.0f)) return MOE_ERR_INVALID_ARG;
    if (c->gate != MOE_GATE_SOFTMAX || c->renormalize || c->aux_alpha != 0.0f) return MOE_ERR_UNSUPPORTED;
  }
  if ((int64_t)c->num_tokens * c->top_k > (int64_t)0x7fffffff) return MOE_ERR_UNSUPPORTED;
  if (c->gate != MOE_GATE_SOFTMAX && c->gate != MOE_GATE_SIGMOID_BIAS && c->gate != MOE_GATE_SQRT_SOFTPLUS_BIAS &&
      c->gate != MOE_GATE_NOISY_TOPK)
    return MOE_ERR_UNSUPPORTED;
  // noisy gating: softmax over the top-k (renormalised), 2E router rows (<= 512)
  if (c->gate == MOE_GATE_NOISY_TOPK && (ec || !c->renormalize || c->num_experts > 256)) return MOE_ERR_UNSUPPORTED;
  if (c->act != MOE_ACT_RELU && c->act != MOE_ACT_SWIGLU) return MOE_ERR_UNSUPPORTED;
  if (c->dtype != MOE_DT_F32 && c->dtype != MOE_DT_BF16) return MOE_ERR_UNSUPPORTED;
  if (c->num_shared_experts != 0 && c->num_shared_experts != 1) return MOE_ERR_UNSUPPORTED;
  if (!isfinite(c->capacity_factor) || !isfinite(c->aux_alpha)) return MOE_ERR_INVALID_ARG;
  // The matmuls address one expert's weight matrix (and a 256-row activation
  // tile) as a base plus a 32-bit per-lane byte offset: each expert matrix must
  // stay under 4 GiB.
  const uint64_t f1 = c->act == MOE_ACT_SWIGLU ? 2 * (uint64_t)c->d_ff : (uint64_t)c->d_ff;  // < 2^32
  const uint64_t eb = c->dtype == MOE_DT_BF16 ? 2 : 4;
  const uint64_t wide = f1 > (uint64_t)c->d_model ? f1 : (uint64_t)c->d_model;
  const uint64_t lim = uint64_t(1) << 32;
  if (f1 * (uint64_t)c->d_model >= lim / eb || 256 * wide >= lim / eb) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int capacity_of(const moe_config* c) {
  if (c->capacity_factor <= 0.0f) return -1;
  // evaluated in double in the order of the capacity formula
  const double v = ceil((double)c->num_tokens / (double)c->num_experts * (double)c->capacity_factor);
  return v < 2147483647.0 ? (int)v : 2147483647;  // v >= 0: T >= 0, E >= 1, cf > 0 and finite
}

int64_t max_rows_of(const moe_config* c, int C) {
  const int64_t tk = (int64_t)c->num_tokens * c->top_k;
  if (C < 0) return tk;
  const int64_t ec = (int64_t)c->num_experts * C;
  return tk < ec ? tk : ec;
}

// Backward workspace layout.
struct BwdWs {
  size_t dO, dA, dXp, dg, dl, dxr, part, dA_sh, dX_sh, order, gx, gw, wsp, offs, nz, total;
};
// router rows: E, or 2E (clean and noise) for noisy gating
int64_t router_rows(const moe_config* c) {
  return c->gate == MOE_GATE_NOISY_TOPK ? 2 * (int64_t)c->num_experts : c->num_experts;
}
BwdWs bwd_layout(const moe_config* c, int64_t R) {
  const int64_t T = c->num_tokens, d = c->d_model, E = router_rows(c), k = c->top_k;
  const int64_t f1 = c->act == MOE_ACT_SWIGLU ? 2 * (int64_t)c->d_ff : c->d_ff;
  const int64_t eb = elem_bytes(c);
  const int64_t ns = moe::router_grad_splits((int)T, (int)E, (int)d);
  BwdWs w;
  size_t o = 0;
  w.dO = o; o += align_up(R * d * eb);
  w.dA = o; o += align_up(R * f1 * eb);
  w.dXp = o; o += align_up(R * d * eb);
  w.dg = o; o += align_up(T * k * 4);
  w.dl = o; o += align_up(T * E * 4);
  w.dxr = o; o += align_up(T * d * 4);
  const int64_t kp = moe::router_dx_k((int)E);
  const int64_t nsw = moe::router_dw_splits((int)T, (int)E, (int)d);
  const int64_t part_f = ns * E * d, part_w = c->dtype == MOE_DT_BF16 ? nsw * kp * d : 0;
  w.part = o; o += align_up((part_f > part_w ? part_f : part_w) * 4);
  w.dA_sh = o; o += c->num_shared_experts ? align_up(T * f1 * eb) : 0;
  w.dX_sh = o; o += c->num_shared_experts ? align_up(T * d * eb) : 0;
  w.order = o; o += align_up((E + 1) * 4);
  w.gx = o; o += c->dtype == MOE_DT_BF16 ? align_up(T * kp * 2) : 0;
  w.gw = o; o += c->dtype == MOE_DT_BF16 ? align_up(T * kp * 2) : 0;
  w.wsp = o; o += c->dtype == MOE_DT_BF16 ? align_up(kp * d * 2) : 0;
  w.offs = o; o += align_up((3 + nsw) * 4);
  w.nz = o;
  o += c->gate == MOE_GATE_NOISY_TOPK ? align_up(moe::noisy_workspace_bytes((int)T, c->num_experts)) : 0;
  w.total = o;
  return w;
}

size_t workspace_of(const moe_config* c, int64_t R) {
  size_t ws = align_up((size_t)moe::dispatch_num_chunks(c->num_tokens, c->top_k) * c->num_experts * 4);
  const size_t aux = align_up((size_t)moe::aux_num_blocks(c->num_tokens) * c->num_experts * 4);
  if (aux > ws) ws = aux;
  const size_t bw = bwd_layout(c, R).total;
  if (bw > ws) ws = bw;
  if (c->routing == MOE_ROUTING_EXPERT_CHOICE) {
    const size_t ec = align_up(moe::ec_workspace_bytes(c->num_tokens, c->num_experts));
    if (ec > ws) ws = ec;
  }
  if (c->gate == MOE_GATE_SIGMOID_BIAS || c->gate == MOE_GATE_SQRT_SOFTPLUS_BIAS) {
    const size_t qb = align_up(moe::qb_workspace_bytes(c->num_tokens, c->num_experts));
    if (qb > ws) ws = qb;
  }
  if (c->gate == MOE_GATE_NOISY_TOPK) {
    const size_t nz = align_up(moe::noisy_workspace_bytes(c->num_tokens, c->num_experts));
    if (nz > ws) ws = nz;
  }
  return ws;
}

int launch_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Opt-in timing hook (moe_profile.h): an event pair around each launch of the
// armed stage. One per host thread: arming it on one thread changes nothing for
// calls made on another.
constexpr int kMaxProfPairs = 4096;
struct Prof {
  bool armed = false;
  bool all = false;
  char only[64] = {0};
  hipEvent_t* ev = nullptr;
  int max = 0, n = 0;
  const char* names[kMaxProfPairs];
};
thread_local Prof g_prof;

struct StageTimer {
  int idx = -1;
  hipStream_t s;
  StageTimer(const char* name, hipStream_t st) : s(st) {
    if (!g_prof.armed || g_prof.n >= g_prof.max) return;
    if (!g_prof.all && strcmp(g_prof.only, name) != 0) return;
    idx = g_prof.n++;
    g_prof.names[idx] = name;
    (void)hipEventRecord(g_prof.ev[2 * idx], s);
  }
  ~StageTimer() {
    if (idx >= 0) (void)hipEventRecord(g_prof.ev[2 * idx + 1], s);
  }
};

// Routed rows read in place through row_token are addressed anywhere in x with
// 32-bit per-lane byte offsets: x must stay under 4 GiB.
bool rows_in_place_fit(const moe_config* c) {
  return (uint64_t)c->num_tokens * (uint64_t)c->d_model * (uint64_t)elem_bytes(c) < (uint64_t(1) << 32);
}

int gemm(const moe_config* c, moe::GemmArgs a, hipStream_t st, const char* stage) {
  StageTimer pt(stage, st);
  hipError_t e = c->dtype == MOE_DT_BF16 ? moe::launch_gemm_bf16(a, st) : moe::launch_gemm_f32(a, st);
  return launch_status(e);
}

}  // namespace

extern "C" {

const char* moe_status_string(int s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int moe_plan(const moe_config* c, moe_plan_info* out) {
  if (!out) return MOE_ERR_INVALID_ARG;
  const int st = check_config(c);
  if (st) return st;
  const int C = capacity_of(c);
  const int64_t R = max_rows_of(c, C);
  out->expert_capacity = C;
  out->f1 = c->act == MOE_ACT_SWIGLU ? 2 * c->d_ff : c->d_ff;
  out->max_rows = R;
  out->workspace_bytes = workspace_of(c, R);
  return MOE_OK;
}

int moe_route(const moe_config* c, const void* x, const float* w_router, const float* logit_offset,
              const float* sel_bias, float* probs, int32_t* topk_idx, float* topk_w, void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (c->routing != MOE_ROUTING_TOKEN_CHOICE || c->gate == MOE_GATE_NOISY_TOPK) return MOE_ERR_UNSUPPORTED;
  const bool empty = c->num_tokens == 0;  // token-indexed pointers may then be NULL
  if (!w_router || (!empty && (!x || !probs || !topk_idx || !topk_w))) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
  if (empty) return MOE_OK;
  moe::RouterArgs a{x, w_router, logit_offset, sel_bias, probs, topk_idx, topk_w, c->num_tokens, c->d_model,
                    c->num_experts, c->top_k, c->gate, c->renormalize ? 1 : 0, c->dtype};
  StageTimer pt("route", (hipStream_t)stream);
  return launch_status(moe::launch_router(a, (hipStream_t)stream));
}

int moe_route_noisy(const moe_config* c, const void* x, const float* w_router, const float* noise,
                    float* logits2, float* probs, int32_t* topk_idx, float* topk_w, void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (c->gate != MOE_GATE_NOISY_TOPK) return MOE_ERR_UNSUPPORTED;
  const bool empty = c->num_tokens == 0;
  if (!w_router || (!empty && (!x || !noise || !logits2 || !probs || !topk_idx || !topk_w)))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
  if (empty) return MOE_OK;
  moe::RouterArgs a{x, w_router, nullptr, nullptr, probs, topk_idx, topk_w, c->num_tokens, c->d_model,
                    c->num_experts, c->top_k, MOE_GATE_SOFTMAX, 1, c->dtype};
  StageTimer pt("route", (hipStream_t)stream);
  return launch_status(moe::launch_route_noisy(a, noise, logits2, (hipStream_t)stream));
}

int moe_aux_noisy(const moe_config* c, const float* logits2, const float* noise, const int32_t* topk_idx,
                  const float* topk_w, float* aux_out, void* ws, size_t ws_bytes, void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (c->gate != MOE_GATE_NOISY_TOPK) return MOE_ERR_UNSUPPORTED;
  if (!aux_out || (c->num_tokens > 0 && (!logits2 || !noise || !topk_idx || !topk_w))) return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < workspace_of(c, max_rows_of(c, capacity_of(c)))) return MOE_ERR_WORKSPACE;
  moe::NoisyArgs a{logits2, noise, topk_idx, topk_w, (float*)ws, c->num_tokens, c->num_experts, c->top_k,
                   c->aux_alpha};
  StageTimer pt("aux", (hipStream_t)stream);
  return launch_status(moe::launch_noisy_stats(a, aux_out, (hipStream_t)stream));
}

int moe_route_ec(const moe_config* c, const void* x, const float* w_router, const float* logit_offset, float* probs,
                 float* topk_w, int32_t* slot, int32_t* expert_counts, int32_t* expert_offsets, int32_t* row_token,
                 void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (c->routing != MOE_ROUTING_EXPERT_CHOICE) return MOE_ERR_UNSUPPORTED;
  const bool empty = c->num_tokens == 0;
  if (!w_router || !expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARG;
  if (!empty && (!x || !probs || !topk_w || !slot || !row_token)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  const int C = capacity_of(c);
  if (!ws || ws_bytes < workspace_of(c, max_rows_of(c, C))) return MOE_ERR_WORKSPACE;
  const int Cp = C < c->num_tokens ? C : c->num_tokens;
  moe::RouteEcArgs a{x, w_router, logit_offset, probs, topk_w, slot, expert_counts, expert_offsets, row_token,
                     x_perm, ws, c->num_tokens, c->d_model, c->num_experts, Cp, c->dtype, elem_bytes(c)};
  StageTimer pt("route_ec", (hipStream_t)stream);
  return launch_status(moe::launch_route_ec(a, (hipStream_t)stream));
}

int moe_dispatch(const moe_config* c, const void* x, const int32_t* topk_idx, int32_t* expert_counts,
                 int32_t* expert_offsets, int32_t* slot, int32_t* row_token, void* x_perm, void* ws,
                 size_t ws_bytes, void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (c->routing != MOE_ROUTING_TOKEN_CHOICE) return MOE_ERR_UNSUPPORTED;
  const bool empty = c->num_tokens == 0;
  // x_perm is optional (NULL: positions only); x is read only to fill it
  if (!expert_counts || !expert_offsets || (!empty && (!topk_idx || !slot || !row_token || (x_perm && !x))))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  const int C = capacity_of(c);
  const size_t need = workspace_of(c, max_rows_of(c, C));
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  moe::DispatchArgs a{x, topk_idx, expert_counts, expert_offsets, slot, row_token, x_perm, (int32_t*)ws,
                      c->num_tokens, c->d_model, c->num_experts, c->top_k, C, elem_bytes(c)};
  StageTimer pt("dispatch", (hipStream_t)stream);
  return launch_status(moe::launch_dispatch(a, (hipStream_t)stream));
}

int moe_dispatch_noalloc(const moe_config* c, const void* x, const int32_t* topk_idx, int32_t* expert_counts,
                         int32_t* expert_offsets, int32_t* slot, int32_t* row_token, void* x_perm, void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (c->routing != MOE_ROUTING_TOKEN_CHOICE) return MOE_ERR_UNSUPPORTED;
  const bool empty = c->num_tokens == 0;
  // x_perm is optional (NULL: positions only); x is read only to fill it
  if (!expert_counts || !expert_offsets || (!empty && (!topk_idx || !slot || !row_token || (x_perm && !x))))
    return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_INVALID_ARG;
  // the per-chunk histograms must fit the library's fixed scratch array
  if (!moe::dispatch_fits_scratch(c->num_tokens, c->top_k, c->num_experts)) return MOE_ERR_WORKSPACE;
  moe::DispatchArgs a{x, topk_idx, expert_counts, expert_offsets, slot, row_token, x_perm, nullptr,
                      c->num_tokens, c->d_model, c->num_experts, c->top_k, capacity_of(c), elem_bytes(c)};
  StageTimer pt("dispatch", (hipStream_t)stream);
  return launch_status(moe::launch_dispatch_noalloc(a, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// The top-1 combine fused into the down projection (moe_expert_ffn_combine).
struct Combine1 {
  const int32_t* slot;
  const float* topk_w;
  void* y;
};

// The expert FFNs; routed rows from x_perm, or (x_perm NULL) from x through
// row_token, gathered as the first matmul loads them; with cb, the down
// projection's epilogue also writes the top-1 combine.
int expert_ffn(const moe_config* c, const void* x_perm, const int32_t* row_token, const int32_t* expert_offsets,
               const void* w1, const void* w2, const void* x, const void* ws1, const void* ws2, void* act_saved,
               void* h_saved, void* y_perm, void* act_shared, void* h_shared, void* y_shared, void* ws,
               size_t ws_bytes, void* stream, const Combine1* cb = nullptr) {
  int st = check_config(c);
  if (st) return st;
  const bool empty = c->num_tokens == 0;
  // ReLU: the pre-activations are optional (the backward takes the sign of h)
  const bool need_act = c->act == MOE_ACT_SWIGLU;
  const bool rows_in_place = x_perm == nullptr;
  if (rows_in_place && !rows_in_place_fit(c)) return MOE_ERR_UNSUPPORTED;
  if (!expert_offsets || !w1 || !w2 ||
      (!empty && ((rows_in_place ? (!x || !row_token) : false) || (need_act && !act_saved) || !h_saved || !y_perm)))
    return MOE_ERR_INVALID_ARG;
  const bool sh = c->num_shared_experts > 0;
  if (sh && (!ws1 || !ws2 || (!empty && (!x || (need_act && !act_shared) || !h_shared || !y_shared))))
    return MOE_ERR_INVALID_ARG;
  if (!sh && (ws1 || ws2 || act_shared || h_shared || y_shared)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x_perm, x, w1, w2, act_saved, h_saved, y_perm};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARG;
  const int C = capacity_of(c);
  const int64_t R = max_rows_of(c, C);
  if (!ws || ws_bytes < workspace_of(c, R)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int T = c->num_tokens, d = c->d_model, f = c->d_ff, E = c->num_experts;
  const int f1 = c->act == MOE_ACT_SWIGLU ? 2 * f : f;
  const int shr = sh ? T : 0;

  moe::GemmArgs g1{};
  g1.kind = 0;
  g1.epi = c->act == MOE_ACT_SWIGLU ? moe::EPI_SWIGLU_FWD : moe::EPI_RELU_FWD;
  g1.b_kcontig = 1;
  g1.N = f1; g1.K = d; g1.f = f;
  g1.has_shared = sh ? 1 : 0;
  g1.offsets = expert_offsets; g1.E = E; g1.shared_rows = shr;
  g1.max_rows = R;
  g1.row_cap = C > 0 ? C : 0;
  g1.A = rows_in_place ? x : x_perm; g1.lda = d;
  if (rows_in_place) {
    g1.a_rows = row_token;
    g1.src_rows = T;
  }
  g1.B = w1; g1.ldb = d; g1.strideB = (int64_t)f1 * d;
  g1.A_sh = x; g1.B_sh = ws1;
  g1.C = act_saved; g1.ldc = f1; g1.C_sh = act_shared;
  g1.C2 = h_saved; g1.ldc2 = f; g1.C2_sh = h_shared;
  if ((st = gemm(c, g1, s, "ffn_gemm1"))) return st;

  moe::GemmArgs g2{};
  g2.kind = 0;
  g2.epi = moe::EPI_STORE;
  g2.b_kcontig = 1;
  g2.N = d; g2.K = f; g2.f = f;
  g2.has_shared = sh ? 1 : 0;
  g2.offsets = expert_offsets; g2.E = E; g2.shared_rows = shr;
  g2.max_rows = R;
  g2.row_cap = C > 0 ? C : 0;
  g2.A = h_saved; g2.lda = f;
  g2.B = w2; g2.ldb = f; g2.strideB = (int64_t)d * f;
  g2.A_sh = h_shared; g2.B_sh = ws2;
  g2.C = y_perm; g2.ldc = d; g2.C_sh = y_shared;
  if (cb) {
    g2.epi = moe::EPI_COMBINE1;
    g2.X = x; g2.ldx = d;
    g2.slot = cb->slot; g2.slot_k = 1;
    g2.row_tok = row_token; g2.tok_w = cb->topk_w;
    g2.Yc = cb->y; g2.copy_tokens = T;
    return gemm(c, g2, s, "ffn_gemm2_combine");
  }
  return gemm(c, g2, s, "ffn_gemm2");
}

}  // namespace

extern "C" {

int moe_expert_ffn(const moe_config* c, const void* x_perm, const int32_t* expert_offsets, const void* w1,
                   const void* w2, const void* x, const void* ws1, const void* ws2, void* act_saved,
                   void* h_saved, void* y_perm, void* act_shared, void* h_shared, void* y_shared, void* ws,
                   size_t ws_bytes, void* stream) {
  if (c && c->num_tokens > 0 && !x_perm) return MOE_ERR_INVALID_ARG;
  return expert_ffn(c, x_perm, nullptr, expert_offsets, w1, w2, x, ws1, ws2, act_saved, h_saved, y_perm, act_shared,
                    h_shared, y_shared, ws, ws_bytes, stream);
}

int moe_expert_ffn_rows(const moe_config* c, const void* x, const int32_t* row_token, const int32_t* expert_offsets,
                        const void* w1, const void* w2, const void* ws1, const void* ws2, void* act_saved,
                        void* h_saved, void* y_perm, void* act_shared, void* h_shared, void* y_shared, void* ws,
                        size_t ws_bytes, void* stream) {
  return expert_ffn(c, nullptr, row_token, expert_offsets, w1, w2, x, ws1, ws2, act_saved, h_saved, y_perm,
                    act_shared, h_shared, y_shared, ws, ws_bytes, stream);
}

int moe_expert_ffn_combine(const moe_config* c, const void* x, const int32_t* row_token,
                           const int32_t* expert_offsets, const int32_t* slot, const float* topk_w, const void* w1,
                           const void* w2, void* act_saved, void* h_saved, void* y_perm, void* y, void* ws,
                           size_t ws_bytes, void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (c->dtype != MOE_DT_BF16 || c->top_k != 1 || c->num_shared_experts != 0 ||
      c->routing != MOE_ROUTING_TOKEN_CHOICE)
    return MOE_ERR_UNSUPPORTED;
  if (c->num_tokens > 0 && (!x || !row_token || !slot || !topk_w || !y)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(y)) return MOE_ERR_INVALID_ARG;
  const Combine1 cb{slot, topk_w, y};
  return expert_ffn(c, nullptr, row_token, expert_offsets, w1, w2, x, nullptr, nullptr, act_saved, h_saved, y_perm,
                    nullptr, nullptr, nullptr, ws, ws_bytes, stream, c->num_tokens > 0 ? &cb : nullptr);
}

int moe_combine(const moe_config* c, const void* x, const void* y_perm, const int32_t* slot, const float* topk_w,
                const void* y_shared, void* y, void* stream) {
  int st = check_config(c);
  if (st) return st;
  const bool empty = c->num_tokens == 0;
  if (!empty && (!x || !y_perm || !slot || !topk_w || !y)) return MOE_ERR_INVALID_ARG;
  if (!empty && (c->num_shared_experts > 0) != (y_shared != nullptr)) return MOE_ERR_INVALID_ARG;
  if (c->num_shared_experts == 0 && y_shared) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y_perm) || !aligned16(y) || !aligned16(y_shared)) return MOE_ERR_INVALID_ARG;
  if (c->num_tokens == 0) return MOE_OK;
  moe::CombineArgs a{x, y_perm, slot, topk_w, y_shared, y, c->num_tokens, c->d_model, c->top_k, c->dtype};
  StageTimer pt("combine", (hipStream_t)stream);
  return launch_status(moe::launch_combine(a, (hipStream_t)stream));
}

int moe_aux_loss(const moe_config* c, const float* probs, const int32_t* expert_counts, float* aux_out, void* ws,
                 size_t ws_bytes, void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (c->gate == MOE_GATE_NOISY_TOPK) return MOE_ERR_UNSUPPORTED;  // moe_aux_noisy
  if (!expert_counts || !aux_out || (c->num_tokens > 0 && !probs)) return MOE_ERR_INVALID_ARG;
  const int C = capacity_of(c);
  if (!ws || ws_bytes < workspace_of(c, max_rows_of(c, C))) return MOE_ERR_WORKSPACE;
  moe::AuxArgs a{probs, expert_counts, aux_out, (float*)ws, c->num_tokens, c->num_experts, c->top_k,
                 c->aux_alpha};
  StageTimer pt("aux", (hipStream_t)stream);
  return launch_status(moe::launch_aux(a, (hipStream_t)stream));
}

int moe_bias_update(const moe_config* c, const int32_t* expert_counts, float gamma, float* sel_bias,
                    void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (!expert_counts || !sel_bias || !aligned16(expert_counts) || !aligned16(sel_bias)) return MOE_ERR_INVALID_ARG;
  if (!isfinite(gamma) || gamma < 0.0f) return MOE_ERR_INVALID_ARG;
  StageTimer pt("bias_update", (hipStream_t)stream);
  return launch_status(moe::launch_bias_update(expert_counts, c->num_experts, gamma, sel_bias, (hipStream_t)stream));
}

int moe_bias_quantile(const moe_config* c, const float* probs, float* sel_bias, void* ws, size_t ws_bytes,
                      void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (c->gate == MOE_GATE_SOFTMAX || c->routing != MOE_ROUTING_TOKEN_CHOICE) return MOE_ERR_UNSUPPORTED;
  if (!sel_bias || (c->num_tokens > 0 && !probs) || !aligned16(probs) || !aligned16(sel_bias))
    return MOE_ERR_INVALID_ARG;
  if (!ws || ws_bytes < workspace_of(c, max_rows_of(c, capacity_of(c)))) return MOE_ERR_WORKSPACE;
  StageTimer pt("bias_quantile", (hipStream_t)stream);
  return launch_status(moe::launch_bias_quantile(probs, sel_bias, c->num_tokens, c->num_experts, c->top_k, ws,
                                                 (hipStream_t)stream));
}

int moe_backward(const moe_config* c, const void* dy, const moe_saved* sv, const moe_weights* w,
                 const moe_grads* g, void* ws, size_t ws_bytes, void* stream) {
  int st = check_config(c);
  if (st) return st;
  if (!sv || !w || !g) return MOE_ERR_INVALID_ARG;
  const bool sh = c->num_shared_experts > 0;
  const bool empty = c->num_tokens == 0;  // token- and row-indexed pointers may then be NULL
  if (!sv->expert_counts || !sv->expert_offsets) return MOE_ERR_INVALID_ARG;
  const bool ec = c->routing == MOE_ROUTING_EXPERT_CHOICE;  // topk_idx is implied (column = expert)
  const bool noisy = c->gate == MOE_GATE_NOISY_TOPK;
  if (noisy && !empty && (!sv->noisy_logits || !sv->noise)) return MOE_ERR_INVALID_ARG;
  const bool relu = c->act == MOE_ACT_RELU;  // the ReLU mask comes from h > 0, which equals act > 0
  // routed rows of x: x_perm, or (x_perm NULL) x through row_token
  if (!empty && (!dy || !sv->x || !sv->probs || (!ec && !sv->topk_idx) || !sv->topk_w || !sv->slot ||
                 (!sv->x_perm && !sv->row_token) || (!relu && !sv->act_saved) || !sv->h_saved || !sv->y_perm ||
                 !g->dx))
    return MOE_ERR_INVALID_ARG;
  if (!w->w_router || !w->w1 || !w->w2 || !g->dw_router || !g->dw1 || !g->dw2) return MOE_ERR_INVALID_ARG;
  if (!empty && !sv->x_perm && !rows_in_place_fit(c)) return MOE_ERR_UNSUPPORTED;
  if (sh && (!w->ws1 || !w->ws2 || !g->dws1 || !g->dws2 ||
             (!empty && ((!relu && !sv->act_shared) || !sv->h_shared))))
    return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {dy, sv->x, sv->x_perm, sv->act_saved, sv->h_saved, sv->y_perm, w->w_router,
                        w->w1, w->w2, g->dx, g->dw_router, g->dw1, g->dw2};
  for (const void* p : ptrs)
    if (!aligned16(p)) return MOE_ERR_INVALID_ARG;
  const int C = capacity_of(c);
  const int64_t R = max_rows_of(c, C);
  if (!ws || ws_bytes < workspace_of(c, R)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int T = c->num_tokens, d = c->d_model, f = c->d_ff, E = c->num_experts, k = c->top_k;
  const int f1 = c->act == MOE_ACT_SWIGLU ? 2 * f : f;
  const int shr = sh ? T : 0;
  const BwdWs L = bwd_layout(c, R);
  uint8_t* base = (uint8_t*)ws;
  void* dO = base + L.dO;
  void* dA = base + L.dA;
  void* dXp = base + L.dXp;
  float* dg = (float*)(base + L.dg);
  float* dl = (float*)(base + L.dl);
  float* dxr = (float*)(base + L.dxr);
  float* part = (float*)(base + L.part);
  void* dA_sh = sh ? base + L.dA_sh : nullptr;
  void* dX_sh = sh ? base + L.dX_sh : nullptr;
  int32_t* order = (int32_t*)(base + L.order);

  // the weight-gradient launches run the experts with the most rows first; the
  // ranking rides along as the first workgroup of the combine backward launch
  if (T > 0) {
    moe::CombineBwdArgs cb{dy, sv->y_perm, sv->slot, sv->topk_w, dO, dg, T, d, k, c->dtype,
                           sv->expert_offsets, E, shr, sh ? 1 : 0, order};
    StageTimer pt("bwd_combine", s);
    if ((st = launch_status(moe::launch_combine_bwd(cb, s)))) return st;
  }
  // dA = act'(dO W2_e), rows of each expert (and dy ws2 for the shared expert)
  moe::GemmArgs a2{};
  a2.kind = 0;
  a2.epi = c->act == MOE_ACT_SWIGLU ? moe::EPI_SWIGLU_BWD : moe::EPI_RELU_BWD;
  a2.b_kcontig = 0;
  a2.N = f; a2.K = d; a2.f = f;
  a2.has_shared = sh ? 1 : 0;
  a2.offsets = sv->expert_offsets; a2.E = E; a2.shared_rows = shr;
  a2.max_rows = R;
  a2.row_cap = C > 0 ? C : 0;
  a2.A = dO; a2.lda = d;
  a2.B = w->w2; a2.ldb = f; a2.strideB = (int64_t)d * f;
  a2.A_sh = dy; a2.B_sh = w->ws2;
  a2.C = dA; a2.ldc = f1; a2.C_sh = dA_sh;
  // ReLU derivative from the sign of the saved activation h (h > 0 exactly when the
  // pre-activation is > 0); SwiGLU from the saved [gate | up] pre-activations
  if (relu) {
    a2.X = sv->h_saved; a2.ldx = f; a2.X_sh = sv->h_shared;
  } else {
    a2.X = sv->act_saved; a2.ldx = f1; a2.X_sh = sv->act_shared;
  }
  if ((st = gemm(c, a2, s, "bwd_dgrad2"))) return st;
  if (T == 0 && (st = launch_status(moe::launch_group_order(sv->expert_offsets, E, shr, sh ? 1 : 0, order, s))))
    return st;
  // dW2_e = dO^T h over the expert's rows
  moe::GemmArgs w2g{};
  w2g.kind = 1;
  w2g.epi = moe::EPI_STORE;
  w2g.M = d; w2g.N = f;
  w2g.has_shared = sh ? 1 : 0;
  w2g.max_rows = R;
  w2g.row_cap = C > 0 ? C : 0;
  w2g.order = order;
  w2g.offsets = sv->expert_offsets; w2g.E = E; w2g.shared_rows = shr;
  w2g.A = dO; w2g.lda = d;
  w2g.B = sv->h_saved; w2g.ldb = f;
  w2g.A_sh = dy; w2g.B_sh = sv->h_shared;
  w2g.C = g->dw2; w2g.ldc = f; w2g.strideC = (int64_t)d * f; w2g.C_sh = g->dws2;
  if ((st = gemm(c, w2g, s, "bwd_wgrad2"))) return st;
  // dX_perm = dA W1_e
  moe::GemmArgs a1{};
  a1.kind = 0;
  a1.epi = moe::EPI_STORE;
  a1.b_kcontig = 0;
  a1.N = d; a1.K = f1; a1.f = f;
  a1.has_shared = sh ? 1 : 0;
  a1.offsets = sv->expert_offsets; a1.E = E; a1.shared_rows = shr;
  a1.max_rows = R;
  a1.row_cap = C > 0 ? C : 0;
  a1.A = dA; a1.lda = f1;
  a1.B = w->w1; a1.ldb = d; a1.strideB = (int64_t)f1 * d;
  a1.A_sh = dA_sh; a1.B_sh = w->ws1;
  a1.C = dXp; a1.ldc = d; a1.C_sh = dX_sh;
  if ((st = gemm(c, a1, s, "bwd_dgrad1"))) return st;
  // dW1_e = dA^T x_perm over the expert's rows (x_perm's rows gathered from x
  // through row_token when no permuted copy was made)
  moe::GemmArgs w1g{};
  w1g.kind = 1;
  w1g.epi = moe::EPI_STORE;
  w1g.M = f1; w1g.N = d;
  w1g.has_shared = sh ? 1 : 0;
  w1g.max_rows = R;
  w1g.row_cap = C > 0 ? C : 0;
  w1g.order = order;
  w1g.offsets = sv->expert_offsets; w1g.E = E; w1g.shared_rows = shr;
  w1g.A = dA; w1g.lda = f1;
  w1g.B = sv->x_perm ? sv->x_perm : sv->x; w1g.ldb = d;
  if (!sv->x_perm) {
    w1g.b_rows = sv->row_token;
    w1g.src_rows = T;
  }
  w1g.A_sh = dA_sh; w1g.B_sh = sv->x;
  w1g.C = g->dw1; w1g.ldc = d; w1g.strideC = (int64_t)f1 * d; w1g.C_sh = g->dws1;
  if ((st = gemm(c, w1g, s, "bwd_wgrad1"))) return st;
  // router: dlogits, dW_r, dx_router
  if (noisy) {
    moe::NoisyArgs na{sv->noisy_logits, sv->noise, sv->topk_idx, sv->topk_w, (float*)(base + L.nz), T, E, k,
                      c->aux_alpha};
    StageTimer pt("bwd_dlogits", s);
    if ((st = launch_status(moe::launch_noisy_dlogits(na, dg, dl, s)))) return st;
  } else if (T > 0) {
    moe::DlogitsArgs dla{sv->probs, ec ? nullptr : sv->topk_idx, sv->topk_w, dg, sv->expert_counts, dl, T, E, k, c->gate,
                         c->renormalize ? 1 : 0, c->aux_alpha};
    if (c->dtype == MOE_DT_BF16) {  // the split operands straight from the dlogits kernel
      dla.dlogits = nullptr;
      dla.gx = (uint16_t*)(base + L.gx);
      dla.gw = (uint16_t*)(base + L.gw);
      dla.kp = moe::router_dx_k(E);
      dla.w_router = w->w_router;
      dla.wsplit = (uint16_t*)(base + L.wsp);
      dla.offs = (int32_t*)(base + L.offs);
      dla.d = d;
    }
    StageTimer pt("bwd_dlogits", s);
    if ((st = launch_status(moe::launch_dlogits(dla, s)))) return st;
  }
  // bf16 layers with one or two experts per token finish dx in the router
  // product's epilogue (with more, the epilogue's gather of k rows per token has
  // too few loads in flight and the separate pass is faster)
  const bool fuse_dx = c->dtype == MOE_DT_BF16 && k <= 2;
  moe::RouterGradArgs rg{dl, sv->x, w->w_router, g->dw_router, dxr, part, (uint16_t*)(base + L.gx),
                         (uint16_t*)(base + L.gw), (uint16_t*)(base + L.wsp), (int32_t*)(base + L.offs), T, d,
                         (int)router_rows(c), c->dtype, dy, sv->slot, k, dXp, dX_sh, fuse_dx ? g->dx : nullptr};
  rg.split_done = (!noisy && T > 0 && c->dtype == MOE_DT_BF16) ? 1 : 0;
  {
    StageTimer pt("bwd_router_grads", s);
    if ((st = launch_status(moe::launch_router_grads(rg, s)))) return st;
  }
  if (T > 0 && !fuse_dx) {
    moe::UnpermuteArgs ua{dy, dXp, sv->slot, dxr, dX_sh, g->dx, T, d, k, c->dtype};
    StageTimer pt("bwd_unpermute", s);
    if ((st = launch_status(moe::launch_unpermute_bwd(ua, s)))) return st;
  }
  return MOE_OK;
}

int moe_profile_arm(const char* stage, void* const* events, int max_pairs) {
  if (!events || max_pairs < 1) return MOE_ERR_INVALID_ARG;
  if (stage && strlen(stage) >= sizeof(g_prof.only)) return MOE_ERR_INVALID_ARG;
  g_prof.all = stage == nullptr;
  if (stage) strcpy(g_prof.only, stage);
  g_prof.ev = (hipEvent_t*)events;
  g_prof.max = max_pairs < kMaxProfPairs ? max_pairs : kMaxProfPairs;
  g_prof.n = 0;
  g_prof.armed = true;
  return MOE_OK;
}

int moe_profile_disarm(void) {
  g_prof.armed = false;
  return g_prof.n;
}

const char* moe_profile_stage(int i) { return (i >= 0 && i < g_prof.n) ? g_prof.names[i] : nullptr; }

}  // extern "C"
