/*
 * moe_peaks.h - attainable-peak probes of one MI355X (gfx950), exported by
 * libmoe_peaks.so, a measuring aid built beside (and kept out of) the layer
 * library libmoe.so.
 *
 * The layer's kernels are reported against published peaks (HBM 8 TB/s, bf16
 * matrix core 2.5 PFLOP/s, fp32 vector 78.6 TFLOP/s without packed FMA). These
 * calls measure what one kernel of the simplest possible form reaches on the
 * machine at hand, so each fraction can also be stated against that. Each
 * kernel does only the work it measures; the caller times one launch (HIP
 * events on `stream`) and divides the work stated below by the time.
 *
 * Conventions: device pointers, 16-byte aligned; `stream` is a hipStream_t as
 * void* (NULL = null stream). Arguments are checked on the host before any
 * launch; a bad one returns MOE_PEAK_ERR_INVALID_ARG and enqueues nothing.
 * MOE_PEAK_ERR_HIP reports a launch error (hipGetLastError). Workgroups have
 * 256 threads. The memory probes use the grid shapes that gave the highest
 * rates in a sweep on MI355X (few concurrent streams: 1-3 workgroups per CU);
 * the compute probes use MOE_PEAK_BLOCKS workgroups.
 */
#ifndef MOE_MI355X_PEAKS_H
#define MOE_MI355X_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_PEAK_OK 0
#define MOE_PEAK_ERR_INVALID_ARG (-1)
#define MOE_PEAK_ERR_HIP (-4)

/* workgroups of the compute probes: 8 per compute unit of the 256 */
#define MOE_PEAK_BLOCKS 2048

/* bytes of the `sink` buffer every probe writes (one 32-bit word per thread). */
size_t moe_peak_sink_bytes(void);

/* Streaming read: reads `bytes` (multiple of 16) from src once, 16 bytes per
 * load, two loads in flight per thread, 3 workgroups per CU; writes at most
 * moe_peak_sink_bytes() to sink.
 * Work: `bytes` read. Use a buffer far above the 256 MB last-level cache. */
int moe_peak_read(const void* src, size_t bytes, void* sink, void* stream);

/* Streaming write: fills `bytes` (multiple of 16) of dst, one 16-byte store in
 * flight per thread, 1 workgroup per CU. Work: `bytes` written. */
int moe_peak_write(void* dst, size_t bytes, void* stream);

/* Copy of `bytes` (multiple of 16) from src to dst; the ranges must not
 * overlap. Four 16-byte loads then stores per thread, 1 workgroup per CU.
 * Work: `bytes` read plus `bytes` written. */
int moe_peak_copy(void* dst, const void* src, size_t bytes, void* stream);

/* bf16 matrix core: every wave runs `iters` x 4 independent
 * v_mfma_f32_32x32x16_bf16 (32*32*16*2 flop each) on register operands.
 * Work: MOE_PEAK_BLOCKS * 4 * iters * 4 * 32768 flop. sink as above. */
int moe_peak_mfma_bf16(void* sink, int iters, void* stream);

/* fp32 vector ALU: every thread runs `iters` x 64 fused multiply-adds in 8
 * independent chains (unpacked v_fma_f32). Work: MOE_PEAK_BLOCKS * 256 *
 * iters * 64 * 2 flop. sink as above. */
int moe_peak_fma_f32(void* sink, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif
