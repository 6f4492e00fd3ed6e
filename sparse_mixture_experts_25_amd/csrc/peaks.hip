// Attainable-peak probes for the rooflines the layer's kernels are measured
// against: HBM streaming read, write and copy, the bf16 matrix core and the
// fp32 vector ALU. Each kernel does only the one kind of work it measures; the
// caller times a launch and divides the work the entry point documents.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_peaks.h"

namespace {

constexpr int kThreads = 256;
// Grid shapes of the memory probes: a sweep over workgroups per CU (1-16) and
// 16-byte accesses in flight per thread (1-8) on MI355X gave the highest rates
// with few concurrent streams: reads at 3 workgroups per CU with 2 loads in
// flight, writes at 1 per CU with 1 store, copies at 1 per CU with 4 of each.
// More concurrent streams lowered every rate (down to 4-5.5 TB/s).
constexpr int kReadBlocks = 3 * 256, kWriteBlocks = 256, kCopyBlocks = 256;

// Each thread keeps U independent 16-byte loads in flight per iteration and
// folds them into one register, written once at the end so no load is dead.
template <int U>
__global__ void __launch_bounds__(kThreads) peak_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                             uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * kThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kThreads;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = acc;
}

__global__ void __launch_bounds__(kThreads) peak_write_kernel(uint4* __restrict__ dst, size_t n16, uint32_t v) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  const uint4 w = make_uint4(v, v ^ 1u, v ^ 2u, v ^ 3u);
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = w;
}

template <int U>
__global__ void __launch_bounds__(kThreads) peak_copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                             size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (U - 1) * stride < n16; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < U; ++u) dst[i + u * stride] = v[u];
  }
  for (; i < n16; i += stride) dst[i] = src[i];
}

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

// Four independent 32x32x16 bf16 accumulation chains per wave; the operands
// stay in registers, so the loop is matrix-core issue and nothing else.
__global__ void __launch_bounds__(kThreads) peak_mfma_kernel(float* __restrict__ sink, int iters, int seed) {
  const int lane = threadIdx.x;
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    // small bf16 values (exponent field 0x3c..), different per lane and slot
    a[j] = (short)(0x3c00 + ((lane * 8 + j + seed) & 0x7f));
    b[j] = (short)(0x3c00 + ((lane * 3 + j * 5 + seed) & 0x7f));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

// Eight independent fp32 fused multiply-add chains per lane.
__global__ void __launch_bounds__(kThreads) peak_fma_kernel(float* __restrict__ sink, int iters, float seed) {
  const float m = 0.999f + 1e-7f * (float)threadIdx.x;
  const float c = seed;
  float r0 = 1.f, r1 = 2.f, r2 = 3.f, r3 = 4.f, r4 = 5.f, r5 = 6.f, r6 = 7.f, r7 = 8.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      r0 = __builtin_fmaf(r0, m, c);
      r1 = __builtin_fmaf(r1, m, c);
      r2 = __builtin_fmaf(r2, m, c);
      r3 = __builtin_fmaf(r3, m, c);
      r4 = __builtin_fmaf(r4, m, c);
      r5 = __builtin_fmaf(r5, m, c);
      r6 = __builtin_fmaf(r6, m, c);
      r7 = __builtin_fmaf(r7, m, c);
    }
  }
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = r0 + r1 + r2 + r3 + r4 + r5 + r6 + r7;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int finish() { return hipGetLastError() == hipSuccess ? MOE_PEAK_OK : MOE_PEAK_ERR_HIP; }

}  // namespace

extern "C" {

size_t moe_peak_sink_bytes(void) { return (size_t)MOE_PEAK_BLOCKS * kThreads * 4; }

int moe_peak_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || !aligned16(src) || !aligned16(sink)) return MOE_PEAK_ERR_INVALID_ARG;
  hipLaunchKernelGGL(peak_read_kernel<2>, dim3(kReadBlocks), dim3(kThreads), 0, (hipStream_t)stream,
                     (const uint4*)src, bytes / 16, (uint32_t*)sink);
  return finish();
}

int moe_peak_write(void* dst, size_t bytes, void* stream) {
  if (!dst || bytes == 0 || bytes % 16 || !aligned16(dst)) return MOE_PEAK_ERR_INVALID_ARG;
  hipLaunchKernelGGL(peak_write_kernel, dim3(kWriteBlocks), dim3(kThreads), 0, (hipStream_t)stream, (uint4*)dst,
                     bytes / 16, 0x3f800000u);
  return finish();
}

int moe_peak_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes == 0 || bytes % 16 || !aligned16(dst) || !aligned16(src)) return MOE_PEAK_ERR_INVALID_ARG;
  const char* s = (const char*)src;
  const char* d = (const char*)dst;
  if (s < d + bytes && d < s + bytes) return MOE_PEAK_ERR_INVALID_ARG;  // overlapping ranges
  hipLaunchKernelGGL(peak_copy_kernel<4>, dim3(kCopyBlocks), dim3(kThreads), 0, (hipStream_t)stream, (uint4*)dst,
                     (const uint4*)src, bytes / 16);
  return finish();
}

int moe_peak_mfma_bf16(void* sink, int iters, void* stream) {
  if (!sink || iters <= 0 || !aligned16(sink)) return MOE_PEAK_ERR_INVALID_ARG;
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(MOE_PEAK_BLOCKS), dim3(kThreads), 0, (hipStream_t)stream, (float*)sink,
                     iters, 1);
  return finish();
}

int moe_peak_fma_f32(void* sink, int iters, void* stream) {
  if (!sink || iters <= 0 || !aligned16(sink)) return MOE_PEAK_ERR_INVALID_ARG;
  hipLaunchKernelGGL(peak_fma_kernel, dim3(MOE_PEAK_BLOCKS), dim3(kThreads), 0, (hipStream_t)stream, (float*)sink,
                     iters, 1e-3f);
  return finish();
}

}  // extern "C"
