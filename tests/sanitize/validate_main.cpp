// Host-side validation of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer (built by tests/test_sanitizers.py). Every call
// made here must return from the library's argument checks before any HIP
// call: null or misaligned pointers, missing or short workspaces, and
// boundary / random configs through moe_plan (whose size arithmetic is where
// an overflow would hide).
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/moe.h"
#include "../../include/moe_profile.h"

static uint64_t g_state = 0x243f6a8885a308d3ull;
static uint64_t next_u64() {
  // xorshift64 (Marsaglia 2003)
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return g_state;
}
template <typename T, int N>
static T pick(const T (&v)[N]) { return v[next_u64() % N]; }

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

int main() {
  const int32_t toks[] = {-1, 0, 1, 7, 64, 256, 8192, 16384, 1 << 20, 1 << 26, INT_MAX};
  const int32_t dims[] = {-8, 0, 7, 8, 60, 64, 768, 2048, 7168, 65528, 65536, 1 << 20, INT_MAX - 7};
  const int32_t experts[] = {-1, 0, 1, 4, 64, 128, 256, 512, 513, INT_MAX};
  const int32_t ks[] = {-1, 0, 1, 2, 8, 64, 65, 512};
  const float cfs[] = {-1.0f, 0.0f, 0.5f, 1.0f, 1.25f, 2.0f, 1e30f, INFINITY, NAN};
  const int32_t enums[] = {-1, 0, 1, 2, 3, 4, 1 << 30};
  const float alphas[] = {0.0f, 0.01f, -1.0f, NAN, INFINITY};
  alignas(16) static unsigned char fake[256];  // never dereferenced by the checks exercised here
  void* A = fake;
  void* MIS = fake + 4;
  int32_t* Ai = (int32_t*)fake;
  float* Af = (float*)fake;
  int n_ok = 0;
  for (int it = 0; it < 40000; ++it) {
    moe_config c;
    c.num_tokens = pick(toks);
    c.d_model = pick(dims);
    c.d_ff = pick(dims);
    c.num_experts = pick(experts);
    c.top_k = (it & 1) ? pick(ks) : (c.num_experts > 0 ? 1 + (int)(next_u64() % (uint64_t)c.num_experts) : 1);
    c.capacity_factor = pick(cfs);
    c.renormalize = (int)(next_u64() % 3) - 1;
    c.gate = (it % 5) ? (int)(next_u64() % 4) : pick(enums);
    c.act = (it % 7) ? (int)(next_u64() % 2) : pick(enums);
    c.dtype = (it % 11) ? (int)(next_u64() % 2) : pick(enums);
    c.aux_alpha = pick(alphas);
    c.num_shared_experts = (int)(next_u64() % 3);
    c.routing = (it % 3) ? 0 : (int)(next_u64() % 3);
    if (c.routing == 1 && (it & 2)) c.top_k = c.num_experts;
    moe_plan_info info;
    const int st = moe_plan(&c, &info);
    EXPECT(st == MOE_OK || st == MOE_ERR_INVALID_ARG || st == MOE_ERR_UNSUPPORTED);
    if (st == MOE_OK) {
      ++n_ok;
      EXPECT(info.max_rows >= 0);
      EXPECT(info.max_rows <= (int64_t)c.num_tokens * c.top_k);
      EXPECT(info.f1 == (c.act == MOE_ACT_SWIGLU ? 2 * c.d_ff : c.d_ff));
      EXPECT(info.workspace_bytes % 256 == 0);
      EXPECT(c.capacity_factor > 0.0f ? info.expert_capacity >= 0 : info.expert_capacity == -1);
    }
    // every entry point with null tensors: an error, no launch (an empty batch
    // with nothing to combine is the one call that may succeed without work)
    EXPECT(moe_route(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) != MOE_OK);
    EXPECT(moe_route_noisy(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) != MOE_OK);
    EXPECT(moe_route_ec(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                        nullptr, nullptr, 0, nullptr) != MOE_OK);
    EXPECT(moe_dispatch(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) !=
           MOE_OK);
    EXPECT(moe_expert_ffn(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                          nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) != MOE_OK);
    EXPECT(moe_expert_ffn_rows(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                               nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) != MOE_OK);
    EXPECT(moe_expert_ffn_combine(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                  nullptr, nullptr, nullptr, 0, nullptr) != MOE_OK);
    const int cb = moe_combine(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
    EXPECT(cb != MOE_OK || (st == MOE_OK && c.num_tokens == 0));
    EXPECT(moe_aux_loss(&c, nullptr, nullptr, nullptr, nullptr, 0, nullptr) != MOE_OK);
    EXPECT(moe_aux_noisy(&c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) != MOE_OK);
    EXPECT(moe_bias_update(&c, nullptr, 1e-3f, nullptr, nullptr) != MOE_OK);
    EXPECT(moe_bias_quantile(&c, nullptr, nullptr, nullptr, 0, nullptr) != MOE_OK);
    EXPECT(moe_backward(&c, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) != MOE_OK);
    if (st != MOE_OK) continue;
    // valid config: short workspace or misaligned tensors are refused
    const size_t ws = info.workspace_bytes;
    EXPECT(moe_dispatch(&c, A, Ai, Ai, Ai, Ai, Ai, A, A, ws ? ws - 1 : 0, nullptr) != MOE_OK || ws == 0);
    EXPECT(moe_dispatch(&c, MIS, Ai, Ai, Ai, Ai, Ai, MIS, A, ws, nullptr) != MOE_OK || c.routing != 0);
    EXPECT(moe_aux_loss(&c, Af, Ai, Af, nullptr, ws, nullptr) != MOE_OK);
    // the rows-in-place matmuls: a short workspace, or no row map with tokens, is refused
    EXPECT(moe_expert_ffn_rows(&c, A, Ai, Ai, A, A, nullptr, nullptr, A, A, A, nullptr, nullptr, nullptr, A,
                               ws ? ws - 1 : 0, nullptr) != MOE_OK || ws == 0);
    EXPECT(moe_expert_ffn_rows(&c, A, nullptr, Ai, A, A, nullptr, nullptr, A, A, A, nullptr, nullptr, nullptr, A, ws,
                               nullptr) != MOE_OK || c.num_tokens == 0);
    moe_saved sv = {};
    moe_weights w = {};
    moe_grads g = {};
    EXPECT(moe_backward(&c, A, &sv, &w, &g, A, ws, nullptr) != MOE_OK);
    w.w_router = (const float*)MIS;
    EXPECT(moe_backward(&c, A, &sv, &w, &g, A, ws, nullptr) != MOE_OK);
  }
  // null config, null plan output, status strings, the timing hook's checks
  moe_plan_info info;
  EXPECT(moe_plan(nullptr, &info) == MOE_ERR_INVALID_ARG);
  moe_config c0 = {64, 64, 64, 4, 1, 1.0f, 0, 0, 0, 1, 0.0f, 0, 0};
  EXPECT(moe_plan(&c0, nullptr) == MOE_ERR_INVALID_ARG);
  for (int s = -10; s <= 10; ++s) EXPECT(moe_status_string(s) != nullptr);
  EXPECT(moe_status_string(INT_MIN) != nullptr && moe_status_string(INT_MAX) != nullptr);
  EXPECT(moe_profile_arm("route", nullptr, 4) != 0);
  void* ev[2] = {nullptr, nullptr};
  EXPECT(moe_profile_arm("a stage name far longer than the sixty-three characters the hook keeps", ev, 1) != 0);
  EXPECT(moe_profile_disarm() == 0);
  EXPECT(moe_profile_stage(0) == nullptr && moe_profile_stage(-1) == nullptr);
  printf("validated configs %d, failures %d\n", n_ok, failures);
  return failures ? 1 : 0;
}
