// Capacity, positions and the permutation into expert-contiguous rows.
//
// [SW] = "Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散"
// (ta-paperlens.web.app), eq. (3) and the section on expert capacity: seats per
// expert are fixed up front, assignments take them in token order, the rest
// skip the expert. [LRMOE] (ai-cafe.club LRMoE item, "この記事のポイント"): kept
// pairs are compacted so each expert's rows are contiguous for a variable-size
// grouped matmul.
//
// The assignments (t, r) are taken in token-major order a = t*k + r and cut
// into chunks of kChunk. Four launches:
//   1. per-chunk expert histogram (LDS integer atomics: exact counts)
//   2. one workgroup: per-expert totals over chunks, kept rows, the exclusive
//      scan over experts (offsets), and each chunk's base per expert (the
//      exclusive prefix over chunks, written over the histograms)
//   3. per chunk: the chunk's base per expert, the
//      stable rank of each assignment among equal experts inside the
//      chunk (wave ballots on the expert id bits give the set of lanes with the
//      same expert; the rank is the popcount of that set below the lane),
//      giving pos, slot and row_token
//   4. per token: copy the row of x into each of its kept slots (16-byte moves;
//      each row of x is read once); skipped when the caller passes no x_perm
//      (the expert matmuls then read the rows of x through row_token)
#include <atomic>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kChunk = 1024;      // assignments per chunk
constexpr int kSub = kChunk / 4;  // assignments per wave inside a chunk

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int total, int E,
                                                   int32_t* __restrict__ chunk_counts) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * kChunk;
  const int a1 = min(total, a0 + kChunk);
  for (int a = a0 + threadIdx.x; a < a1; a += 256) atomicAdd(&hist[idx[a]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup: per-expert totals over the chunk histograms, the kept rows and
// the exclusive scan over experts (offsets); the chunk histograms are replaced
// by their exclusive prefix over chunks (the assignments to each expert in
// earlier chunks: the base that assign_kernel reads). The chunks are split into
// G = 1024 / E contiguous ranges, one per group of E threads, so each expert's
// sum is G short chains of independent loads and a G-term combine rather than
// one chain over every chunk. Integer sums: the order does not change them.
constexpr int kScanThreads = 1024;  // >= E (moe_plan accepts at most 512 experts)
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t* __restrict__ chunk_counts, int nchunks,
                                                            int E, int C, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int part[kScanThreads];  // [G][E]: group sums, then their exclusive prefix over groups
  __shared__ int wsum[kScanThreads / 64];
  const int tid = threadIdx.x;
  const int G = kScanThreads / E;
  const int g = tid / E, e = tid % E;
  const bool act = g < G;
  const int cpg = (nchunks + G - 1) / G;
  const int c0 = g * cpg, c1 = min(nchunks, c0 + cpg);
  int s = 0;
  if (act)
    for (int c = c0; c < c1; ++c) s += chunk_counts[(int64_t)c * E + e];
  if (act) part[g * E + e] = s;
  __syncthreads();
  int total_e = 0;  // held by the threads of group 0 (tid = e)
  if (act && g == 0) {
    for (int h = 0; h < G; ++h) {
      const int v = part[h * E + e];
      part[h * E + e] = total_e;
      total_e += v;
    }
  }
  __syncthreads();
  if (act) {
    int run = part[g * E + e];
    for (int c = c0; c < c1; ++c) {
      const int64_t i = (int64_t)c * E + e;
      const int v = chunk_counts[i];
      chunk_counts[i] = run;
      run += v;
    }
  }
  // kept rows of expert tid and their exclusive scan over the experts
  int kept = 0;
  if (tid < E) {
    counts[tid] = total_e;
    kept = (C < 0) ? total_e : min(total_e, C);
  }
  const int lane = tid & 63, wave = tid >> 6;
  int incl = kept;
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
  for (int w = 0; w < kScanThreads / 64; ++w) {
    if (w < wave) wbase += wsum[w];
    tot += wsum[w];
  }
  if (tid < E) offsets[tid] = wbase + incl - kept;
  if (tid == 0) offsets[E] = tot;
}

__global__ __launch_bounds__(256) void assign_kernel(const int32_t* __restrict__ idx, int total, int k,
                                                     int E, int C, const int32_t* __restrict__ chunk_counts,
                                                     const int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ slot,
                                                     int32_t* __restrict__ row_token) {
  extern __shared__ int32_t sm[];
  int32_t* run = sm;  // [4][E]: running position per wave and expert
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int a0 = blockIdx.x * kChunk;
  // per-wave counts of each expert in the wave's sub-chunk
  for (int i = threadIdx.x; i < 4 * E; i += 256) run[i] = 0;
  __syncthreads();
  {
    const int s0 = a0 + wave * kSub;
    const int s1 = min(total, s0 + kSub);
    for (int a = s0 + lane; a < s1; a += 64) atomicAdd(&run[wave * E + idx[a]], 1);
  }
  __syncthreads();
  // bases: base(w, e) = (assignments to e in earlier chunks) + (in earlier waves of this chunk)
  for (int e = threadIdx.x; e < E; e += 256) {
    int b = chunk_counts[(int64_t)blockIdx.x * E + e];  // assignments to e in earlier chunks (scan_kernel)
    for (int w = 0; w < 4; ++w) {
      const int c = run[w * E + e];
      run[w * E + e] = b;
      b += c;
    }
  }
  __syncthreads();
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  int32_t* myrun = run + wave * E;
  const int s0 = a0 + wave * kSub;
  const int s1 = min(total, s0 + kSub);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = s0; base < s1; base += 64) {
    const int a = base + lane;
    const bool valid = a < s1;
    const int e = valid ? idx[a] : 0;
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int rank = __popcll(m & lt_mask);
    const int pos = valid ? myrun[e] + rank : 0;
    const bool leader = valid && (lane == 63 - __clzll(m));
    if (leader) myrun[e] = pos + 1;  // the leader holds the highest rank of its group
    if (valid) {
      const bool keep = (C < 0) || (pos < C);
      const int s = keep ? offsets[e] + pos : -1;
      slot[a] = s;
      if (keep) row_token[s] = a / k;
    }
  }
}

__global__ __launch_bounds__(256) void scatter_rows_kernel(const uint8_t* __restrict__ x,
                                                           const int32_t* __restrict__ slot, int T, int k,
                                                           int64_t row_bytes, uint8_t* __restrict__ x_perm) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int nvec = (int)(row_bytes / 16);
  const uint8_t* src = x + (int64_t)t * row_bytes;
  for (int v = lane; v < nvec; v += 64) {
    const u128 val = ld128(src + (int64_t)v * 16);
    for (int r = 0; r < k; ++r) {
      const int s = slot[(int64_t)t * k + r];
      if (s >= 0) st128(x_perm + (int64_t)s * row_bytes + (int64_t)v * 16, val);
    }
  }
}

// Per-chunk histograms of the allocation-free dispatch: a file-scope device
// array, one copy per GPU, held until the process ends. Its host-side name is a
// stand-in, not a device address: kernels get the address that
// hipGetSymbolAddress returns for the device (cached per device below).
static __device__ __align__(256) int32_t scratch[kDispatchScratchInts];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];

// Device address of `scratch` on the device `st` belongs to (the current device
// for the null stream); looked up once per device with that device current.
hipError_t scratch_address(hipStream_t st, int32_t** out) {
  int dev = -1;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(p, std::memory_order_release);  // racing lookups store the same address
  }
  *out = reinterpret_cast<int32_t*>(p);
  return hipSuccess;
}

}  // namespace

bool dispatch_fits_scratch(int T, int k, int E) {
  return (int64_t)dispatch_num_chunks(T, k) * E <= kDispatchScratchInts;
}

hipError_t launch_dispatch_noalloc(const DispatchArgs& a_in, hipStream_t st) {
  if (!dispatch_fits_scratch(a_in.T, a_in.k, a_in.E)) return hipErrorInvalidValue;
  DispatchArgs a = a_in;
  hipError_t e = scratch_address(st, &a.ws_chunk);
  if (e != hipSuccess) return e;
  // every histogram entry the launch reads is written by it first: nothing to clear
  return launch_dispatch(a, st);
}

int dispatch_num_chunks(int T, int k) {
  const int64_t total = (int64_t)T * k;
  return (int)((total + kChunk - 1) / kChunk);
}

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t st) {
  const int total = a.T * a.k;
  const int nch = dispatch_num_chunks(a.T, a.k);
  if (nch > 0)
    hipLaunchKernelGGL(hist_kernel, dim3(nch), dim3(256), a.E * sizeof(int32_t), st, a.topk_idx, total,
                       a.E, a.ws_chunk);
  if (a.E > kScanThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, st, a.ws_chunk, nch, a.E, a.capacity,
                     a.counts, a.offsets);
  if (nch == 0) return hipGetLastError();  // no tokens: counts and offsets are all zero
  hipLaunchKernelGGL(assign_kernel, dim3(nch), dim3(256), 4 * a.E * sizeof(int32_t), st, a.topk_idx,
                     total, a.k, a.E, a.capacity, a.ws_chunk, a.offsets, a.slot, a.row_token);
  if (a.x_perm)  // without x_perm the matmuls read the rows through row_token
    hipLaunchKernelGGL(scatter_rows_kernel, dim3((a.T + 3) / 4), dim3(256), 0, st,
                       (const uint8_t*)a.x, a.slot, a.T, a.k, (int64_t)a.d * a.elem_bytes,
                       (uint8_t*)a.x_perm);
  return hipGetLastError();
}

}  // namespace moe
