/*
 * moe_profile.h - opt-in timing hook of the MoE layer library.
 *
 * For benchmarks: while armed, the library records a caller-owned HIP event
 * before and after every launch of the named stage, on the stream that stage
 * runs on, so the caller can read per-launch kernel durations with
 * hipEventElapsedTime. Disarmed (the default) it costs one branch per stage.
 *
 * The hook is per host thread: arm, run and disarm on one thread; only the
 * calls made on that thread are timed, and calls on other threads are not
 * affected (each thread has its own hook, disarmed until it arms it).
 *
 * Stage names (one stage = one kernel unless noted):
 *   "route" (moe_route, moe_route_noisy), "route_ec" (moe_route_ec, several
 *   kernels), "dispatch" (4 kernels), "ffn_gemm1", "ffn_gemm2",
 *   "ffn_gemm2_combine" (moe_expert_ffn_combine's down projection), "combine",
 *   "aux" (moe_aux_loss or moe_aux_noisy, 2 kernels), "bias_update",
 *   "bias_quantile" (several kernels), "bwd_combine", "bwd_dgrad2",
 *   "bwd_wgrad2", "bwd_dgrad1", "bwd_wgrad1", "bwd_dlogits",
 *   "bwd_router_grads" (3 kernels), "bwd_unpermute".
 */
#ifndef MOE_MI355X_PROFILE_H
#define MOE_MI355X_PROFILE_H

#ifdef __cplusplus
extern "C" {
#endif

/* Arm the hook. stage: a stage name above, or NULL for every stage.
 * events: host array of 2*max_pairs hipEvent_t (as void*), created by the
 * caller; pair i is events[2i] (start) and events[2i+1] (end). Recording stops
 * silently once max_pairs pairs are used. Returns 0, or -1 (MOE_ERR_INVALID_ARG)
 * for a NULL events array or max_pairs < 1. */
int moe_profile_arm(const char* stage, void* const* events, int max_pairs);

/* Disarm; returns the number of pairs recorded since moe_profile_arm. */
int moe_profile_disarm(void);

/* Stage name of recorded pair i (static string), or NULL when out of range. */
const char* moe_profile_stage(int i);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_PROFILE_H */
