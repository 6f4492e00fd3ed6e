// bf16 grouped matmuls on the gfx950 matrix cores, over ragged expert groups.
//
// [LRMOE] (ai-cafe.club LRMoE item, "この記事のポイント"): compacted
// expert-contiguous rows make the expert FFNs one variable-size grouped GEMM.
// [SW] ("Mixture of Experts (MoE) を1から解説 — Switch Transformerのルーティングと負荷分散",
// ta-paperlens.web.app), section on replacing the FFN by N expert copies.
//
// One kernel template covers the six matmuls of the layer:
//   ragged-M (forward, and the input gradients): the row count of each group
//     comes from the device offsets; the workgroup id is decoded in-kernel into
//     (group, row tile, column tile), so no host round trip is needed.
//   ragged-K (weight gradients): a fixed [M, N] output per group, contracted
//     over that group's rows; a group without rows writes zeros. Groups with
//     rows run largest first, the ones without spread between them
//     (rank_groups_by_rows).
//
// Main loop: an NS-stage pipeline over BK-deep K steps. Every step is
// brought into LDS with direct global->LDS 16-byte loads (each wave fills
// 1 KB blocks; lane i of a load lands at +16*i, so the XOR swizzle of the LDS
// layout is applied by choosing which global chunk each lane fetches). Up to
// NS-1 steps are in flight while the matrix cores work on the current one; a
// per-wave vmcnt wait plus one barrier per step publishes a stage. A partial
// last K step loads clamped addresses and zeroes what lies past K in LDS.
//   K-contiguous operand ([rows][K] in memory): LDS rows of BK k, with the
//     16-byte chunks XOR-swizzled by row (mfma_tile.h); fragments read with
//     ds_read_b128.
//   MN-contiguous operand ([K][rows] in memory, the gradient matmuls): LDS
//     k-rows as in memory with the chunks swizzled by k-row; fragments read
//     with the gfx950 LDS transpose read (ds_read_b64_tr_b16), which turns a
//     4(k) x 16(mn) block into per-lane k-vectors.
// Two wave rows by WGN wave columns (4 or 8 waves), each wave computing its
// sub-tile with v_mfma_f32_32x32x16_bf16 (fp32 accumulation). Rows or
// columns past the end of a group read clamped (finite) data and are never
// stored. The epilogue stages the fp32 tile in LDS (half at a time) and
// writes 16-byte rows, fusing the activation (forward) or its derivative
// (backward), or the unpermute of the input gradient.
#include <type_traits>

#include "gemm_common.h"
#include "mfma_tile.h"

namespace moe {

namespace {


// ------------------------------------------------------------ direct loads
// A pointer every lane holds the same value of, returned as a wave-uniform
// value (two readfirstlanes, each half widened through uint32_t), so that
// arithmetic on it stays on the scalar unit.
__device__ __forceinline__ const uint16_t* uniform_ptr(const uint16_t* p) {
  const uint64_t b = (uint64_t)(uintptr_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return reinterpret_cast<const uint16_t*>((uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 16-byte global->LDS load per lane; the 64 lanes of the wave fill the
// 1 KB block at LDS byte address `lds_block` (wave-uniform), lane i at +16*i.
// The global address is a per-lane 32-bit byte offset (VGPR) plus a
// wave-uniform 64-bit base (SGPR pair), so a K step only moves the base.
// M0 holds the LDS address for the instruction and is restored afterwards.
// NT: non-temporal (streaming) cache policy, for data read once.
template <bool NT = false>
__device__ __forceinline__ void dma16s(uint32_t voff, const void* base, uint32_t lds_block) {
  // readfirstlane returns int: widen through uint32_t, never sign-extend a half
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  uint32_t saved;
  if (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_block))
        : "memory");
  else
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds_block))
        : "memory");
}

// One 4-byte global->LDS load per lane: lane i lands at `lds` + 4*i.
__device__ __forceinline__ void dma4s(uint32_t voff, const void* base, uint32_t lds) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sb), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait until at most `steps` later pipeline steps (L loads each) of this wave
// are in flight
template <int L>
__device__ __forceinline__ void wait_steps(int steps) {
  if (steps <= 0) wait_vm<0>();
  else if (steps == 1) wait_vm<L>();
  else if (steps == 2) wait_vm<2 * L>();
  else if (steps == 3) wait_vm<3 * L>();
  else wait_vm<4 * L>();
}

// Per-lane byte offsets of the direct loads of one tile, computed once per
// workgroup (they depend on the tile, not on the K step).
template <int R, int BK, int NW>
struct DmaPlan {
  static constexpr int NB = R * BK * 2 / 1024;  // 1 KB blocks in the tile
  static constexpr int Q = NB / NW;              // blocks per wave
  uint32_t voff[Q];
  // K-contiguous: rowidx(r) = source row (clamped / remapped) of tile row r
  template <typename RowIdx>
  __device__ void make_kc(int wave, int lane, int64_t ld, RowIdx rowidx) {
    constexpr int CPR = BK / 8;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int p = (wave * Q + q) * 64 + lane;
      const int r = p / CPR, pc = p % CPR;
      const int c = pc ^ kc_swz<BK>(r);
      voff[q] = (uint32_t)(((int64_t)rowidx(r) * ld + 8 * c) * 2);
    }
  }
  // MN-contiguous: k-row kr at kr * ld, column chunks clamped to cvalid
  __device__ void make_mn(int wave, int lane, int64_t ld, int cvalid) {
    constexpr int CPR = R / 8;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int p = (wave * Q + q) * 64 + lane;
      const int kr = p / CPR, pc = p % CPR;
      const int c = mn_chunk<R>(kr, pc);  // the swizzle is an involution
      const int cc = c < cvalid ? c : cvalid - 1;
      voff[q] = (uint32_t)(((int64_t)kr * ld + 8 * cc) * 2);
    }
  }
  template <bool NT>
  __device__ void issue(const uint16_t* base, uint32_t lds_tile, int wave) const {
#pragma unroll
    for (int q = 0; q < Q; ++q) dma16s<NT>(voff[q], base, lds_tile + (wave * Q + q) * 1024);
  }
  // The partial last step of a K-contiguous operand (make_kc plan): 16-byte
  // chunks at or past kv (kv a multiple of 8, 0 < kv < BK) read chunk 0 of
  // their row instead; the caller zeroes them in LDS.
  template <bool NT>
  __device__ void issue_kc_tail(const uint16_t* base, uint32_t lds_tile, int wave, int lane, int kv) const {
    constexpr int CPR = BK / 8;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int p = (wave * Q + q) * 64 + lane;
      const int r = p / CPR;
      const int c = (p % CPR) ^ kc_swz<BK>(r);
      const uint32_t v = 8 * c < kv ? voff[q] : voff[q] - (uint32_t)(16 * c);
      dma16s<NT>(v, base, lds_tile + (wave * Q + q) * 1024);
    }
  }
  // An MN-contiguous operand whose k-rows are gathered: the k-row of load q
  // of this lane is row rowq[q] of the operand (past the end of K the last
  // row again, which the caller zeroes in LDS); column chunks clamped to
  // cvalid as in make_mn.
  template <bool NT>
  __device__ void issue_mn_rows(const uint16_t* base, uint32_t lds_tile, int wave, int lane, const int (&rowq)[Q],
                                int64_t ld, int cvalid) const {
    constexpr int CPR = R / 8;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int p = (wave * Q + q) * 64 + lane;
      const int c = mn_chunk<R>(p / CPR, p % CPR);
      const int cc = c < cvalid ? c : cvalid - 1;
      dma16s<NT>((uint32_t)(((int64_t)rowq[q] * ld + 8 * cc) * 2), base, lds_tile + (wave * Q + q) * 1024);
    }
  }
  // the k-row (within the step) of load q of this lane
  __device__ static int mn_krow(int wave, int lane, int q) { return ((wave * Q + q) * 64 + lane) / (R / 8); }
  // The partial last step of an MN-contiguous operand (make_mn plan): k-rows
  // at or past kv (1 <= kv < BK) read k-row kv-1 instead, so every address
  // stays inside the group; the caller zeroes those k-rows in LDS.
  template <bool NT>
  __device__ void issue_mn_tail(const uint16_t* base, uint32_t lds_tile, int wave, int lane, int kv,
                                int64_t ld) const {
    constexpr int CPR = R / 8;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int kr = ((wave * Q + q) * 64 + lane) / CPR;
      const uint32_t v = kr < kv ? voff[q] : voff[q] - (uint32_t)((int64_t)(kr - kv + 1) * ld * 2);
      dma16s<NT>(v, base, lds_tile + (wave * Q + q) * 1024);
    }
  }
};

// The top-1 combine of a token whose only choice was dropped: y = x bit for
// bit. Wave w (counted over the copy workgroups) takes the 64 tokens from
// 64 w, finds the dropped ones with one ballot and copies their rows, 16 bytes
// per lane.
__device__ __forceinline__ void copy_dropped_rows(const GemmArgs& a, int wave_global, int lane) {
  const int t0 = wave_global * 64;
  if (t0 >= a.copy_tokens) return;
  const int t = t0 + lane;
  uint64_t mask = __ballot(t < a.copy_tokens && a.slot[t] < 0);
  const uint16_t* X = reinterpret_cast<const uint16_t*>(a.X);
  uint16_t* Y = reinterpret_cast<uint16_t*>(a.Yc);
  const int nv = a.N / 8;
  while (mask) {
    const int j = __builtin_ctzll(mask);
    mask &= mask - 1;
    const int64_t off = (int64_t)(t0 + j) * a.ldx;
    for (int v = lane; v < nv; v += 64) st128_nt(Y + off + 8 * v, ld128(X + off + 8 * v));
  }
}

// ------------------------------------------------------------ kernel
// WGN waves along N (2 along M): 4 waves for 128x128 tiles, or 8 waves for
// 256x256 tiles with 128x64 per wave (two waves per SIMD, so one wave's matrix
// work covers the other's waits). Row-ragged 128x128 tiles are held to the
// registers of three workgroups per CU (their 64 KB of LDS admits two);
// weight-gradient tiles fit 128 registers (four workgroups per CU): their
// short contractions are latency-bound, so more of them in flight pays.
template <int WGN, int KIND>
constexpr int waves_per_simd() { return WGN == 4 ? 2 : (KIND == 1 ? 4 : 3); }

// GB (weight gradients): B's k-rows of the routed groups are gathered through
// GemmArgs::b_rows. Each wave brings the row indices of a step into its own
// two-slot LDS ring with one more direct load, issued with the operand loads
// two steps earlier, and reads its lanes' indices into registers one step
// before the operand loads that use them go out.
template <int BM, int BN, int BK, int NS, int KIND, int B_KC, int EPI, int WGN, int GB>
__global__ __launch_bounds__(128 * WGN, 1) __attribute__((amdgpu_waves_per_eu(waves_per_simd<WGN, KIND>(), waves_per_simd<WGN, KIND>()))) void gemm_bf16_kernel(
    GemmArgs a) {
  constexpr int kBK = BK;
  constexpr int NW = 2 * WGN, NTH = 64 * NW;  // waves, threads
  constexpr int WM = BM / 2, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int A_KC = (KIND == 0);
  constexpr int B_IS_KC = (KIND == 0) && B_KC;
  constexpr int kStage = (BM + BN) * kBK;  // elements
  constexpr int kOperandBytes = NS * kStage * 2;
  constexpr int CP = BN + 8;  // padded row of the staged fp32 tile
  constexpr int HM = BM / 2;  // the fp32 tile is staged half (one wave row) at a time
  constexpr int kStageBytes = HM * CP * 4;
  constexpr int kRingOff = kOperandBytes;            // GB: index rings (512 bytes per wave), after the stages
  constexpr int kLoopBytes = kOperandBytes + (GB ? NW * 512 : 0);
  constexpr int kLds = kLoopBytes > kStageBytes ? kLoopBytes : kStageBytes;
  constexpr int L = (BM + BN) * BK * 2 / 1024 / NW + GB;  // direct loads per wave per K step
  static_assert(!GB || (KIND == 1 && BK <= 64 && NS == 2), "row gathers are for the weight gradients");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kLds];
  __shared__ __attribute__((aligned(16))) int info[12];

  uint16_t* stages = reinterpret_cast<uint16_t*>(smem);
  const uint32_t lds0 = lds_addr(smem);

  const int tid = threadIdx.x;
  // the wave index is the same in every lane: as a scalar, the LDS block
  // addresses of the direct loads are scalar arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int wm = wave / WGN, wn = wave % WGN;

  if constexpr (EPI == EPI_COMBINE1) {
    if ((int64_t)blockIdx.x >= a.copy_base) {
      copy_dropped_rows(a, (int)((int64_t)blockIdx.x - a.copy_base) * NW + wave, lane);
      return;
    }
  }

  // ---- locate the tile
  int g, rows, mrow0 = 0, nb, mb = 0;
  int64_t r0;
  if (KIND == 0) {
    const int ncols = (EPI == EPI_SWIGLU_FWD) ? a.f : a.N;
    const int bn = (EPI == EPI_SWIGLU_FWD) ? BN / 2 : BN;
    TileInfo ti;
    if (!locate_ragged_m<BM>(a, (ncols + bn - 1) / bn, 4, info, ti, nb)) return;
    g = ti.g; r0 = ti.r0; rows = ti.rows; mrow0 = ti.m0;
  } else {
    // groups in the given order (largest first), tiles of one group
    // consecutive. 128x128 tiles (short, weight-streaming contractions) are
    // placed on the XCDs by k_tile; 256x256 tiles (compute-bound) keep the row
    // block fastest (in bands of 4 row blocks for the gathered kind).
    const int nM = (a.M + BM - 1) / BM, nN = (a.N + BN - 1) / BN;
    const uint32_t per_g = (uint32_t)((BM < 256) ? ragged_k_per_group(nM, nN) : (int64_t)nM * nN);
    const int rank = (int)(blockIdx.x / per_g);
    if (BM < 256) {
      if (!k_tile(blockIdx.x % per_g, nM, nN, mb, nb)) return;
    } else {
      const int t = (int)(blockIdx.x % per_g);
      if constexpr (GB) {
        // the up projection's weight gradient (x's rows gathered): bands of 4
        // row blocks across all column blocks, row block fastest inside a band,
        // so each row block's panel sits in two XCDs' L2s and each gathered
        // column panel in four (1-2 % faster than one band of all row blocks)
        constexpr int GMW = 4;
        const int gsz = GMW * nN, first = (t / gsz) * GMW, gm = min(GMW, nM - first), local = t % gsz;
        mb = first + local % gm;
        nb = local / gm;
      } else {
        mb = t % nM;
        nb = t / nM;
      }
    }
    g = a.order ? a.order[rank] : rank;
    if (g < a.E) {
      r0 = a.offsets[g];
      rows = a.offsets[g + 1] - a.offsets[g];
    } else {
      r0 = 0;
      rows = a.shared_rows;
    }
    if (!group_in_part(a, rows)) return;  // the other launch of a split matmul
    if (EPI == EPI_STORE && rows == 0) {
      // a group without rows: its weight gradient is zero, stored straight from
      // registers (no operand loads, no LDS staging)
      uint16_t* Cg = reinterpret_cast<uint16_t*>(g < a.E ? a.C : a.C_sh) + (g < a.E ? (int64_t)g * a.strideC : 0);
      for (int u = threadIdx.x; u < BM * BN / 8; u += 128 * WGN) {
        const int mm = mb * BM + u / (BN / 8), nn = nb * BN + (u % (BN / 8)) * 8;
        if (mm < a.M && nn < a.N) st128_nt(Cg + (int64_t)mm * a.ldc + nn, zero128());
      }
      return;
    }
  }
  const bool sh = g >= a.E;
  const uint16_t* Ab = reinterpret_cast<const uint16_t*>(sh ? a.A_sh : a.A);
  const uint16_t* Bb = reinterpret_cast<const uint16_t*>(sh ? a.B_sh : a.B);
  if (!sh && KIND == 0) Bb += (int64_t)g * a.strideB;

  // K extent, operand origins and valid extents
  const int K = (KIND == 0) ? a.K : rows;
  const uint16_t* Aorig;
  const uint16_t* Borig;
  int a_valid, b_valid;  // KC: valid rows of the tile; MN: valid 8-column chunks
  // routed rows of A read in place through the row map (ragged-M)
  const bool ga = KIND == 0 && a.a_rows && !sh;
  // routed k-rows of B gathered through the row map (ragged-K)
  const bool gb = GB && !sh;
  if (KIND == 0) {
    Aorig = ga ? Ab : Ab + (r0 + mrow0) * a.lda;
    a_valid = min(rows - mrow0, BM);
    if (B_KC) {
      Borig = Bb;
      b_valid = (EPI == EPI_SWIGLU_FWD) ? 0 : min(a.N - nb * BN, BN);
    } else {
      Borig = Bb + (int64_t)nb * BN;  // [K][N]
      b_valid = min(a.N - nb * BN, BN) / 8;
    }
  } else {
    Aorig = Ab + r0 * a.lda + (int64_t)mb * BM;                  // [rows][M]
    Borig = Bb + (gb ? 0 : r0 * a.ldb) + (int64_t)nb * BN;  // [rows][N]
    a_valid = min(a.M - mb * BM, BM) / 8;
    b_valid = min(a.N - nb * BN, BN) / 8;
  }
  const int h0 = nb * (BN / 2);  // SwiGLU: first h column of this tile

  // the operand origins are the same for the whole workgroup (the tile decode
  // reaches every lane through LDS): as scalars, each K step moves a scalar base
  Aorig = uniform_ptr(Aorig);
  Borig = uniform_ptr(Borig);
  DmaPlan<BM, BK, NW> pa;
  DmaPlan<BN, BK, NW> pb;
  if (A_KC)
    pa.make_kc(wave, lane, a.lda, [&](int r) {
      const int rr = r < a_valid ? r : a_valid - 1;
      return ga ? a.a_rows[r0 + mrow0 + rr] : rr;
    });
  else pa.make_mn(wave, lane, a.lda, a_valid);
  if (B_IS_KC)
    pb.make_kc(wave, lane, a.ldb, [&](int r) {
      if (EPI == EPI_SWIGLU_FWD) {
        const int hc0 = h0 + (r < BN / 2 ? r : r - BN / 2);
        const int hc = hc0 < a.f ? hc0 : a.f - 1;
        return r < BN / 2 ? hc : a.f + hc;
      }
      return nb * BN + (r < b_valid ? r : b_valid - 1);
    });
  else pb.make_mn(wave, lane, a.ldb, b_valid);
  // Row-ragged 128x128 launches (groups under 256 rows on average): each
  // group's weight slab is read by one or two row tiles, adjacent in time, so
  // the weight loads stream past the caches (non-temporal) and leave L2 to the
  // activation tiles, which every column tile re-reads.
  constexpr bool kStreamB = KIND == 0 && BM < 256;
  // GB: the row indices of step k, in slot k & 1 of this wave's ring, and
  // this lane's rows of the next step to be issued
  auto ring = [&](int k) { return reinterpret_cast<const int32_t*>(smem + kRingOff + wave * 512 + (k & 1) * 256); };
  int growq[GB ? DmaPlan<BN, BK, NW>::Q : 1];
  auto prefetch_rows = [&](int k) {
    if constexpr (GB) {
      if (gb) {
#pragma unroll
        for (int q = 0; q < DmaPlan<BN, BK, NW>::Q; ++q) growq[q] = ring(k)[DmaPlan<BN, BK, NW>::mn_krow(wave, lane, q)];
      }
    }
  };
  auto dma_idx = [&](int k) {
    if constexpr (GB) {
      const uint32_t slot = lds0 + kRingOff + wave * 512 + (k & 1) * 256;
      // rows past K repeat the last one; the shared group (rows in place)
      // loads a placeholder, so every wave issues the same loads per step
      if (gb) dma4s((uint32_t)min(k * kBK + lane, K - 1) * 4u, a.b_rows + r0, slot);
      else dma4s(0u, Borig, slot);
    }
  };
  // B's k-rows through the row map (GB); true when it issued them
  auto dma_rows = [&](uint32_t sb) {
    if constexpr (GB) {
      if (gb) {
        pb.template issue_mn_rows<kStreamB>(Borig, sb, wave, lane, growq, a.ldb, b_valid);
        return true;
      }
    }
    return false;
  };
  auto dma_step = [&](int stage, int k0) {
    const uint32_t sa = lds0 + stage * kStage * 2;
    const uint32_t sb = sa + BM * kBK * 2;
    pa.template issue<false>(A_KC ? Aorig + k0 : Aorig + (int64_t)k0 * a.lda, sa, wave);
    if (!dma_rows(sb)) pb.template issue<kStreamB>(B_IS_KC ? Borig + k0 : Borig + (int64_t)k0 * a.ldb, sb, wave);
  };
  // the partial last step as one more direct-load step with clamped addresses
  auto dma_tail = [&](int stage, int k0) {
    const uint32_t sa = lds0 + stage * kStage * 2;
    const uint32_t sb = sa + BM * kBK * 2;
    if (A_KC) pa.template issue_kc_tail<false>(Aorig + k0, sa, wave, lane, K - k0);
    else pa.template issue_mn_tail<false>(Aorig + (int64_t)k0 * a.lda, sa, wave, lane, K - k0, a.lda);
    if (dma_rows(sb)) return;
    if (B_IS_KC) pb.template issue_kc_tail<kStreamB>(Borig + k0, sb, wave, lane, K - k0);
    else pb.template issue_mn_tail<kStreamB>(Borig + (int64_t)k0 * a.ldb, sb, wave, lane, K - k0, a.ldb);
  };
  // A partial last K step (k >= K reads as zero; weight gradients have one in
  // almost every group, row-ragged matmuls only when K is not a multiple of
  // BK) is one more pipelined direct-load step with clamped addresses (k-rows
  // of an MN-contiguous operand, 16-byte chunks of a K-contiguous one), whose
  // parts past K are zeroed in LDS once it lands. No registers are held across
  // the loop for it.

  floatx16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Main loop, pipelined at the granularity of one 16-deep MFMA sub-step: while
  // the MFMAs of sub-step (k, s) run, the fragments of the next sub-step are
  // read from LDS into the other register set, so the matrix cores do not wait
  // on LDS. Before the first fragments of step k+1 are read, that step is
  // published (its direct loads waited for, one barrier); the LDS slot of step
  // k is then free (all its fragments are in registers) and receives step k+NS.
  // 128x128 tiles free it one barrier earlier, right after the sub-steps that
  // read it, so NS-1 later steps are in flight while step k+1 is waited for.
  //
  // 128x128 tiles: the wave's 32-row blocks interleave with the other wave
  // row's (block i of wave row wm holds tile rows (2i + wm) * 32 .. +32), so
  // the valid rows of a short group split evenly over the SIMDs. 256x256
  // tiles: wave row wm holds rows wm * 128 .. +128. In the row-ragged kinds the
  // blocks wholly past the group's rows skip their fragment reads and matrix
  // work: the loop runs with FMV = the count of live blocks (a compile-time
  // value per instantiation), every instantiation with the same barriers.
  constexpr bool kInterleave = BM < 256;
  auto brow = [&](int i) { return kInterleave ? (2 * i + wm) * 32 : wm * WM + i * 32; };
  constexpr int SUB = kBK / 16;  // even: sub-step s always uses register set s & 1
  bf16x8 fa[2][FM], fb[2][FN];
  auto read_frags = [&](auto fmv, auto set, int stage, int s) {
    constexpr int FMV = decltype(fmv)::value;
    constexpr int S = decltype(set)::value;
    const uint16_t* ta = stages + stage * kStage;
    const uint16_t* tb = ta + BM * kBK;
#pragma unroll
    for (int i = 0; i < FMV; ++i)
      fa[S][i] = A_KC ? frag_kc<BK>(ta, brow(i), s, lane) : frag_mn<BM>(ta, brow(i), s, lane);
    if (FMV > 0) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
        fb[S][j] = B_IS_KC ? frag_kc<BK>(tb, wn * WN + j * 32, s, lane) : frag_mn<BN>(tb, wn * WN + j * 32, s, lane);
    }
  };
  auto mfmas = [&](auto fmv, auto set) {
    constexpr int FMV = decltype(fmv)::value;
    constexpr int S = decltype(set)::value;
#pragma unroll
    for (int i = 0; i < FMV; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[S][i], fb[S][j], acc[i][j], 0, 0, 0);
  };
  auto interleave = [&](auto fmv) {
    constexpr int FMV = decltype(fmv)::value;
    constexpr int RD = FMV == 0 ? 0 : FMV * (A_KC ? 1 : 2) + FN * (B_IS_KC ? 1 : 2);  // LDS reads per sub-step
    constexpr int MF = FMV * FN;                                                      // MFMAs per sub-step
    if constexpr (A_KC && B_IS_KC) {
      // both operands K-contiguous (one 16-byte read per fragment): every read of
      // the next sub-step first, then this sub-step's MFMAs. The two register
      // sets then stay distinct, and the reads have the whole sub-step to land
      // (mixing them in let the compiler reuse the current set's registers, so
      // each sub-step's first MFMAs waited for reads issued just before them).
      if (RD > 0) {
        __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
      }
    } else {
      // transposed reads (two per fragment): one LDS read, then a share of the MFMAs, RD times
#pragma unroll
      for (int r = 0; r < RD; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, (MF + RD - 1) / (RD > 0 ? RD : 1), 0);
      }
    }
  };

  const int nfull = K / kBK;
  const int nk = nfull + ((K % kBK) ? 1 : 0);
  const bool has_tail = nk > nfull;
  // 128x128 tiles (weight-streaming shapes) refill a slot as soon as every
  // wave has read it, one barrier earlier than the publish of the next step;
  // 256x256 tiles (matrix-bound) save that barrier
  constexpr bool kEarly = BM < 256;
  // GB: after a step's operand loads (whose rows were read from the ring a
  // step earlier) the indices of step k+2 go into the slot those rows came
  // from. Each publish then also waits for the indices loaded with the step
  // before the one it publishes, so prefetch_rows(k + NS + 1) may follow
  // publish(k + 1) in both pipelines (the one-step-in-flight wait of the
  // 128x128 tiles leaves out only the last step's operand and index loads).
  auto issue_step = [&](int stage, int k) {
    if (k < nfull) dma_step(stage, k * kBK);
    else dma_tail(stage, k * kBK);
    dma_idx(k + 2);
  };
  // Direct loads issued before publish(k): steps 0 .. min(NS-1, nk-1) for
  // k = 0 (prologue); steps 0 .. min(k+NS-2, nk-1) for k >= 1. The wait lets
  // the later ones stay in flight.
  auto publish = [&](int k) {
    wait_steps<L>(kEarly || k == 0 ? min(NS - 1, nk - 1 - k) : min(NS - 2, nk - 1 - k));
    __syncthreads();
    if (k == nfull && has_tail) {
      // zero what the clamped loads brought in past K, in both operands
      const int kv = K - nfull * kBK;
      uint16_t* ta = stages + (k % NS) * kStage;
      uint16_t* tb = ta + BM * kBK;
      for (int u = tid; u < kBK * BM / 8; u += NTH) {
        if (A_KC) {
          if (8 * (u % (BK / 8)) >= kv) st128(ta + kc_off<BK>(u / (BK / 8), u % (BK / 8)), zero128());
        } else if (u / (BM / 8) >= kv) {
          st128(ta + mn_off<BM>(u / (BM / 8), u % (BM / 8)), zero128());
        }
      }
      for (int u = tid; u < kBK * BN / 8; u += NTH) {
        if (B_IS_KC) {
          if (8 * (u % (BK / 8)) >= kv) st128(tb + kc_off<BK>(u / (BK / 8), u % (BK / 8)), zero128());
        } else if (u / (BN / 8) >= kv) {
          st128(tb + mn_off<BN>(u / (BN / 8), u % (BN / 8)), zero128());
        }
      }
      __syncthreads();
    }
  };
  if (GB && nk > 0) {
    dma_idx(0);
    dma_idx(1);
    wait_vm<0>();
  }
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < nk) {
      prefetch_rows(s);
      issue_step(s, s);
    }
  using Set0 = std::integral_constant<int, 0>;
  using Set1 = std::integral_constant<int, 1>;
  // sub-steps 0 .. SUB-2 of the current step (no barrier inside)
  auto inner = [&](auto fmv, int stage) {
#pragma unroll
    for (int s = 0; s + 1 < SUB; ++s) {
      if (s & 1) {
        read_frags(fmv, Set0(), stage, s + 1);
        mfmas(fmv, Set1());
      } else {
        read_frags(fmv, Set1(), stage, s + 1);
        mfmas(fmv, Set0());
      }
      interleave(fmv);
    }
  };
  auto main_loop = [&](auto fmv) {
    publish(0);
    if (NS < nk) prefetch_rows(NS);
    read_frags(fmv, Set0(), 0, 0);
    for (int k = 0; k + 1 < nk; ++k) {
      const int stage = k % NS;
      inner(fmv, stage);
      // every fragment of step k is in registers once all waves pass this
      // barrier (it waits for the wave's LDS reads): its slot takes step k+NS
      // before step k+1 is waited for, so NS-1 later steps stay in flight
      if (kEarly && k + NS < nk) {
        __syncthreads();
        issue_step(stage, k + NS);
      }
      // last sub-step of step k (set 1, SUB is even) overlaps the first reads of step k+1
      publish(k + 1);
      if (!kEarly && k + NS < nk) issue_step(stage, k + NS);
      if (k + NS + 1 < nk) prefetch_rows(k + NS + 1);
      read_frags(fmv, Set0(), (k + 1) % NS, 0);
      mfmas(fmv, Set1());
      interleave(fmv);
    }
    inner(fmv, (nk - 1) % NS);
    mfmas(fmv, Set1());
  };
  if (nk > 0) {
    // live 32-row blocks of this wave: those with brow(i) < a_valid, a prefix
    // of its FM blocks in both layouts
    if constexpr (KIND == 0 && kInterleave && FM == 2) {
      const int nvb = __builtin_amdgcn_readfirstlane(a_valid > 64 + wm * 32 ? 2 : (a_valid > wm * 32 ? 1 : 0));
      if (nvb == 2) main_loop(std::integral_constant<int, 2>());
      else if (nvb == 1) main_loop(std::integral_constant<int, 1>());
      else main_loop(std::integral_constant<int, 0>());
    } else if constexpr (KIND == 0 && !kInterleave && FM == 4) {
      const int lv = a_valid - wm * WM;  // valid rows from this wave row's first
      const int nvb = __builtin_amdgcn_readfirstlane(lv <= 0 ? 0 : (lv >= 128 ? 4 : (lv + 31) / 32));
      if (nvb == 4) main_loop(std::integral_constant<int, 4>());
      else if (nvb == 3) main_loop(std::integral_constant<int, 3>());
      else if (nvb == 2) main_loop(std::integral_constant<int, 2>());
      else if (nvb == 1) main_loop(std::integral_constant<int, 1>());
      else main_loop(std::integral_constant<int, 0>());
    } else {
      main_loop(std::integral_constant<int, FM>());
    }
  }
  __syncthreads();

  if constexpr ((EPI == EPI_STORE || EPI == EPI_COMBINE1) && (BM == 256 || KIND == 0)) {
    // A plain bf16 output: the tile is staged in LDS as the bf16 values it is
    // stored as (the same rounding of the same accumulators), all of it in one
    // pass: half the LDS bytes of fp32 staging, and one barrier instead of three.
    // (Not for the 128x128 weight-gradient tiles: there the conversions of
    // every accumulator at once cost the registers of their fourth workgroup
    // per CU.)
    constexpr int CB = BN + 8;  // padded bf16 row
    static_assert(BM * CB * 2 <= kLds, "the bf16 tile fits the LDS of the main loop");
    uint16_t* Cb = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = brow(i) + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const int n = wn * WN + j * 32 + (lane & 31);
          Cb[m * CB + n] = f2bf(acc[i][j][e]);
        }
    __syncthreads();
    uint16_t* C = reinterpret_cast<uint16_t*>(sh ? a.C_sh : a.C);
    if constexpr (EPI == EPI_COMBINE1) {
      // y_perm as above, and the combine of each row's token in the order of
      // the separate pass (x, then the weighted expert row; one rounding). The
      // tokens, their weights and x's vectors of all of a thread's outputs go
      // out before any is used: three dependent loads per output.
      constexpr int IT1 = BM * BN / 8 / NTH;
      static_assert((BM * BN / 8) % NTH == 0, "every thread writes the same number of vectors");
      const uint16_t* X = reinterpret_cast<const uint16_t*>(a.X);
      uint16_t* Y = reinterpret_cast<uint16_t*>(a.Yc);
      int tok[IT1];
      float w[IT1];
      u128 xv[IT1];
#pragma unroll
      for (int it = 0; it < IT1; ++it) {
        const int u = tid + it * NTH, m = u / (BN / 8), col = nb * BN + (u % (BN / 8)) * 8;
        tok[it] = (m < rows - mrow0 && col < a.N) ? a.row_tok[r0 + mrow0 + m] : -1;
      }
#pragma unroll
      for (int it = 0; it < IT1; ++it) {
        const int u = tid + it * NTH, col = nb * BN + (u % (BN / 8)) * 8;
        if (tok[it] >= 0) {
          w[it] = a.tok_w[tok[it]];
          xv[it] = ld128(X + (int64_t)tok[it] * a.ldx + col);
        }
      }
#pragma unroll
      for (int it = 0; it < IT1; ++it) {
        if (tok[it] < 0) continue;
        const int u = tid + it * NTH, m = u / (BN / 8), n = (u % (BN / 8)) * 8, col = nb * BN + n;
        const u128 v = ld128(Cb + m * CB + n);
        st128(C + (r0 + mrow0 + m) * a.ldc + col, v);
        float yp[8], o[8];
        Elem<uint16_t>::unpack(v, yp);
        Elem<uint16_t>::unpack(xv[it], o);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf(w[it], yp[e], o[e]);
        st128_nt(Y + (int64_t)tok[it] * a.ldx + col, Elem<uint16_t>::pack(o));
      }
      return;
    }
    for (int u = tid; u < BM * BN / 8; u += NTH) {
      const int m = u / (BN / 8), n = (u % (BN / 8)) * 8;
      const u128 v = ld128(Cb + m * CB + n);
      if (KIND == 1) {
        // weight gradients are written once and not read in this pass
        const int mm = mb * BM + m, nn = nb * BN + n;
        if (mm >= a.M || nn >= a.N) continue;
        uint16_t* Cg = sh ? C : C + (int64_t)g * a.strideC;
        st128_nt(Cg + (int64_t)mm * a.ldc + nn, v);
      } else {
        const int col = nb * BN + n;
        if (m >= rows - mrow0 || col >= a.N) continue;
        st128(C + (r0 + mrow0 + m) * a.ldc + col, v);
      }
    }
    return;
  }

  // ---- epilogue: stage the fp32 tile in LDS one half (the rows of one wave
  // row) at a time, then write 16-byte row vectors. The epilogues that read
  // other tensors issue those loads for a whole half together instead of one
  // output vector at a time: the saved pre-activations before the half is
  // staged (their latency overlaps the staging), the unpermute's slots before
  // it and the rows they name after it, in batches.
  float* Cs = reinterpret_cast<float*>(smem);
  uint16_t* C = reinterpret_cast<uint16_t*>(sh ? a.C_sh : a.C);
  uint16_t* C2 = reinterpret_cast<uint16_t*>(sh ? a.C2_sh : a.C2);
  const uint16_t* X = reinterpret_cast<const uint16_t*>(sh ? a.X_sh : a.X);
  constexpr int U = HM * BN / 8;  // 16-byte output vectors of a half
  constexpr int IT = U / NTH;     // per thread
  static_assert(U % NTH == 0, "every thread writes the same number of vectors");
  constexpr bool kReadsX = EPI == EPI_RELU_BWD || EPI == EPI_SWIGLU_BWD || EPI == EPI_UNPERMUTE;
  constexpr int kUK = 2;  // unpermute: kept rows per token loaded ahead (it runs for k <= 2)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int mbase = half * HM;  // tile row of Cs row 0
    // the output vector of iteration it: tile row m, column col, and whether it is stored
    auto unit = [&](int it, int& m, int& n, int& col) {
      const int u = tid + it * NTH;
      m = mbase + u / (BN / 8);
      n = (u % (BN / 8)) * 8;
      col = nb * BN + n;
      return m < rows - mrow0 && col < a.N;
    };
    // (the unpermute loads only its slots here; dy comes with the rows below)
    u128 xa[kReadsX && EPI != EPI_UNPERMUTE ? IT : 1], xb[EPI == EPI_SWIGLU_BWD ? IT : 1];
    int sl[EPI == EPI_UNPERMUTE ? IT * kUK : 1];
    if constexpr (kReadsX) {
#pragma unroll
      for (int it = 0; it < IT; ++it) {
        int m, n, col;
        const bool ok = unit(it, m, n, col);
        // vectors that are not stored read the tile's first one (always inside the tensors)
        const int64_t row = r0 + mrow0 + (ok ? m : 0);
        const int cc = ok ? col : 0;
        if constexpr (EPI != EPI_UNPERMUTE) xa[it] = ld128(X + row * a.ldx + cc);
        if constexpr (EPI == EPI_SWIGLU_BWD) xb[it] = ld128(X + row * a.ldx + a.f + cc);
        if constexpr (EPI == EPI_UNPERMUTE) {
#pragma unroll
          for (int r = 0; r < kUK; ++r) sl[it * kUK + r] = (ok && r < a.slot_k) ? a.slot[row * a.slot_k + r] : -1;
        }
      }
    }
    // the blocks (of every wave, or of wave row `half`) whose rows fall in this half
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (kInterleave ? (i < half * FM / 2 || i >= (half + 1) * FM / 2) : wm != half) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = brow(i) - half * HM + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          const int n = wn * WN + j * 32 + (lane & 31);
          Cs[m * CP + n] = acc[i][j][e];
        }
    }
    __syncthreads();
    if (EPI == EPI_SWIGLU_FWD) {
      // columns [0, BN/2) hold gate, [BN/2, BN) up, for h columns h0 + j
      for (int u = tid; u < U / 2; u += NTH) {
        const int ml = u / (BN / 16);
        const int j = (u % (BN / 16)) * 8;
        const int m = mbase + ml;
        const int hc = h0 + j;
        if (m >= rows - mrow0 || hc >= a.f) continue;
        const int64_t row = r0 + mrow0 + m;
        float gv[8], uv[8], hv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          gv[e] = Cs[ml * CP + j + e];
          uv[e] = Cs[ml * CP + BN / 2 + j + e];
          hv[e] = silu_f(gv[e]) * uv[e];
        }
        st128(C + row * a.ldc + hc, Elem<uint16_t>::pack(gv));
        st128(C + row * a.ldc + a.f + hc, Elem<uint16_t>::pack(uv));
        st128(C2 + row * a.ldc2 + hc, Elem<uint16_t>::pack(hv));
      }
    } else {
      // unpermute: the kept rows' vectors (and the shared expert's) of CH
      // iterations, loaded together once the slots are in. CH bounds the
      // registers they hold while the other wave row's accumulators are still
      // live (the first half of a 256x256 tile); in the second half every
      // accumulator is in LDS and all of them go out at once.
      const int CH = (EPI == EPI_UNPERMUTE && IT > 4 && half == 0) ? 2 : IT;
#pragma unroll
      for (int c0 = 0; c0 < IT; c0 += CH) {
        u128 xc[EPI == EPI_UNPERMUTE ? IT : 1], yr[EPI == EPI_UNPERMUTE ? IT * kUK : 1], ys[EPI == EPI_UNPERMUTE ? IT : 1];
        if constexpr (EPI == EPI_UNPERMUTE) {
          const uint16_t* Yp = reinterpret_cast<const uint16_t*>(a.Y);
          const uint16_t* Ys = reinterpret_cast<const uint16_t*>(a.Y_sh);
#pragma unroll
          for (int c = 0; c < CH; ++c) {
            int m, n, col;
            if (!unit(c0 + c, m, n, col)) continue;
            xc[c] = ld128(X + (r0 + mrow0 + m) * a.ldx + col);
#pragma unroll
            for (int r = 0; r < kUK; ++r) {
              const int q = sl[(c0 + c) * kUK + r];
              if (q >= 0) yr[c * kUK + r] = ld128(Yp + (int64_t)q * a.N + col);
            }
            if (Ys) ys[c] = ld128(Ys + (r0 + mrow0 + m) * a.N + col);
          }
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int it = c0 + c;
          int m, n, col;
          const bool ok = unit(it, m, n, col);
          const int ml = m - mbase;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = Cs[ml * CP + n + e];
          if (KIND == 1) {
            const int mm = mb * BM + m, nn = nb * BN + n;
            if (mm >= a.M || nn >= a.N) continue;
            if (EPI == EPI_STORE_F32) {
              float* Cf = reinterpret_cast<float*>(a.C) + (int64_t)g * a.strideC + (int64_t)mm * a.ldc + nn;
              reinterpret_cast<float4*>(Cf)[0] = make_float4(v[0], v[1], v[2], v[3]);
              reinterpret_cast<float4*>(Cf)[1] = make_float4(v[4], v[5], v[6], v[7]);
              continue;
            }
            // weight gradients are written once and not read in this pass
            uint16_t* Cg = sh ? C : C + (int64_t)g * a.strideC;
            st128_nt(Cg + (int64_t)mm * a.ldc + nn, Elem<uint16_t>::pack(v));
            continue;
          }
          if (!ok) continue;
          const int64_t row = r0 + mrow0 + m;
          if (EPI == EPI_STORE) {
            st128(C + row * a.ldc + col, Elem<uint16_t>::pack(v));
          } else if (EPI == EPI_STORE_F32) {
            float* Cf = reinterpret_cast<float*>(sh ? a.C_sh : a.C) + row * a.ldc + col;
            reinterpret_cast<float4*>(Cf)[0] = make_float4(v[0], v[1], v[2], v[3]);
            reinterpret_cast<float4*>(Cf)[1] = make_float4(v[4], v[5], v[6], v[7]);
          } else if (EPI == EPI_RELU_FWD) {
            float h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = fmaxf(v[e], 0.0f);
            if (C) st128(C + row * a.ldc + col, Elem<uint16_t>::pack(v));  // pre-activation only if asked for
            st128(C2 + row * a.ldc2 + col, Elem<uint16_t>::pack(h));
          } else if (EPI == EPI_RELU_BWD) {
            float xs[8];
            Elem<uint16_t>::unpack(xa[it], xs);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = xs[e] > 0.0f ? v[e] : 0.0f;
            st128(C + row * a.ldc + col, Elem<uint16_t>::pack(v));
          } else if (EPI == EPI_UNPERMUTE) {
            // same order as the separate pass: dy, kept expert rows in r order,
            // router term, shared expert
            float o[8], tmp[8];
            Elem<uint16_t>::unpack(xc[c], o);
#pragma unroll
            for (int r = 0; r < kUK; ++r) {
              if (sl[it * kUK + r] < 0) continue;
              Elem<uint16_t>::unpack(yr[c * kUK + r], tmp);
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] += tmp[e];
            }
            // rows past the ones loaded ahead (not used by the layer: k <= 2)
            for (int r = kUK; r < a.slot_k; ++r) {
              const int s2 = a.slot[row * a.slot_k + r];
              if (s2 < 0) continue;
              Elem<uint16_t>::unpack(ld128(reinterpret_cast<const uint16_t*>(a.Y) + (int64_t)s2 * a.N + col), tmp);
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] += tmp[e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] += v[e];
            if (a.Y_sh) {
              Elem<uint16_t>::unpack(ys[c], tmp);
#pragma unroll
              for (int e = 0; e < 8; ++e) o[e] += tmp[e];
            }
            st128(C + row * a.ldc + col, Elem<uint16_t>::pack(o));
          } else if (EPI == EPI_SWIGLU_BWD) {
            float gs[8], us[8], dg[8], du[8];
            Elem<uint16_t>::unpack(xa[it], gs);
            Elem<uint16_t>::unpack(xb[it], us);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float s = act_sigmoid(gs[e]);
              du[e] = v[e] * gs[e] * s;
              dg[e] = v[e] * us[e] * s * (1.0f + gs[e] * (1.0f - s));
            }
            st128(C + row * a.ldc + col, Elem<uint16_t>::pack(dg));
            st128(C + row * a.ldc + a.f + col, Elem<uint16_t>::pack(du));
          }
        }
      }
    }
    if (half == 0) __syncthreads();
  }
}

template <int BM, int BN, int BK, int NS, int KIND, int B_KC, int EPI, int WGN = 2, int GB = 0>
hipError_t launch_t(const GemmArgs& a, hipStream_t st) {
  int64_t n;
  if (KIND == 0) {
    const int ncols = (EPI == EPI_SWIGLU_FWD) ? a.f : a.N;
    const int bn = (EPI == EPI_SWIGLU_FWD) ? BN / 2 : BN;
    n = raster_grid(row_tile_bound(a, BM), (ncols + bn - 1) / bn);
  } else {
    const int ng = a.E + (a.has_shared ? 1 : 0);
    const int nM = (a.M + BM - 1) / BM, nN = (a.N + BN - 1) / BN;
    n = (int64_t)ng * ((BM < 256) ? ragged_k_per_group(nM, nN) : (int64_t)nM * nN);
  }
  GemmArgs b = a;
  if constexpr (EPI == EPI_COMBINE1) {
    // the dropped tokens' copies: one wave per 64 tokens, after the tiles
    b.copy_base = n;
    n += (a.copy_tokens + 128 * WGN - 1) / (128 * WGN);
  }
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BK, NS, KIND, B_KC, EPI, WGN, GB>), dim3((unsigned)n), dim3(128 * WGN), 0,
                     st, b);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int NS, int WGN = 2>
hipError_t launch_tiles(const GemmArgs& a, hipStream_t st) {
  // the direct loads address each operand as base + 32-bit per-lane byte offset
  // (gathered rows: anywhere in the mapped operand)
  const int64_t lim = int64_t(1) << 32;
  int64_t b_span = a.kind == 0 && a.b_kcontig ? (a.epi == EPI_SWIGLU_FWD ? 2 * (int64_t)a.f : a.N) : BK;
  int64_t a_span = a.kind == 0 ? BM : BK;
  if (a.kind == 0 && a.a_rows) a_span = a.src_rows;
  if (a.kind == 1 && a.b_rows) b_span = a.src_rows;
  if (a_span * a.lda * 2 >= lim || b_span * a.ldb * 2 >= lim) return hipErrorInvalidValue;
  if (a.kind == 1) {
    if (a.epi == EPI_STORE_F32) return launch_t<BM, BN, BK, NS, 1, 0, EPI_STORE_F32, WGN>(a, st);
    return a.b_rows ? launch_t<BM, BN, BK, NS, 1, 0, EPI_STORE, WGN, 1>(a, st)
                    : launch_t<BM, BN, BK, NS, 1, 0, EPI_STORE, WGN>(a, st);
  }
  if (a.b_kcontig) {
    switch (a.epi) {
      case EPI_STORE: return launch_t<BM, BN, BK, NS, 0, 1, EPI_STORE, WGN>(a, st);
      case EPI_RELU_FWD: return launch_t<BM, BN, BK, NS, 0, 1, EPI_RELU_FWD, WGN>(a, st);
      case EPI_SWIGLU_FWD: return launch_t<BM, BN, BK, NS, 0, 1, EPI_SWIGLU_FWD, WGN>(a, st);
      case EPI_COMBINE1: return launch_t<BM, BN, BK, NS, 0, 1, EPI_COMBINE1, WGN>(a, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (a.epi) {
    case EPI_STORE: return launch_t<BM, BN, BK, NS, 0, 0, EPI_STORE, WGN>(a, st);
    case EPI_RELU_BWD: return launch_t<BM, BN, BK, NS, 0, 0, EPI_RELU_BWD, WGN>(a, st);
    case EPI_SWIGLU_BWD: return launch_t<BM, BN, BK, NS, 0, 0, EPI_SWIGLU_BWD, WGN>(a, st);
    case EPI_STORE_F32: return launch_t<BM, BN, BK, NS, 0, 0, EPI_STORE_F32, WGN>(a, st);
    case EPI_UNPERMUTE: return launch_t<BM, BN, BK, NS, 0, 0, EPI_UNPERMUTE, WGN>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// Group ranking alone (batches without tokens; otherwise the combine backward
// launch does it in an extra workgroup).
__global__ __launch_bounds__(512) void group_order_kernel(const int32_t* __restrict__ offsets, int E,
                                                         int shared_rows, int has_shared,
                                                         int32_t* __restrict__ order) {
  __shared__ int rows_s[1025];
  rank_groups_by_rows(offsets, E, shared_rows, has_shared, order, rows_s, 512);
}

}  // namespace

hipError_t launch_group_order(const int32_t* offsets, int E, int shared_rows, int has_shared, int32_t* order,
                              hipStream_t st) {
  hipLaunchKernelGGL(group_order_kernel, dim3(1), dim3(512), 0, st, offsets, E, shared_rows, has_shared, order);
  return hipGetLastError();
}

// Tile choice: 256x256 on eight waves (128x64 each, two waves per SIMD;
// 64-deep K steps, two stages, one workgroup per CU) when the groups are large
// enough to fill it on average. Otherwise 128x128 on four waves: row-ragged
// matmuls with 64-deep steps and two stages (two workgroups per CU, a full
// 128-byte line per weight row and step), weight gradients with 32-deep steps
// and two stages (four workgroups per CU: their one to three steps per tile
// are latency-bound). Those are the small expert batches, where the weights
// stream from HBM and the row tile is mostly padding.
hipError_t launch_gemm_bf16(const GemmArgs& a, hipStream_t st) {
  const int64_t groups = a.E > 0 ? a.E : 1;
  const int64_t avg_rows = a.max_rows / groups;
  // 256x256 tiles also need enough of them to give every CU a workgroup
  const int64_t big_tiles = a.kind == 0 ? ((a.max_rows + 255) / 256) * ((a.N + 255) / 256)
                                        : (groups + (a.has_shared ? 1 : 0)) * ((a.M + 255) / 256) * ((a.N + 255) / 256);
  const bool big = avg_rows >= 256 && (a.kind == 0 ? a.N >= 256 : (a.M >= 256 && a.N >= 256)) &&
                   big_tiles >= 256;
  // short contractions (one or two K steps per tile): two stages suffice
  auto small_tiles = [&](const GemmArgs& s) { return s.kind == 1 ? launch_tiles<128, 128, 32, 2>(s, st) : launch_tiles<128, 128, 64, 2>(s, st); };
  if (!big) return small_tiles(a);
  // Groups capped at 512 rows or fewer (expert capacity): the host knows only
  // the cap, and the realised groups range from full (expert choice, balanced
  // routing) to mostly empty (skewed routing that drops most assignments). A
  // row-ragged matmul then runs as two launches over the groups, each deciding
  // on the device from the group's row count: kSplitRows (64) rows or more on
  // 256x256 tiles (a group of 64-255 rows reads each weight slab once, and the
  // waves past its rows skip their matrix work), the others (and empty ones)
  // on the weight-streaming 128x128 tiles. Below 64 rows a group's few
  // 256-wide column tiles each stream a long weight slab alone. Dropless layers keep one launch: there the
  // zero-fill of empty experts overlaps the big groups' matrix work, which a
  // second launch would serialise.
  const bool capped = a.row_cap > 0 && a.row_cap <= 512 && a.E > 1;
  // A capped layer's weight gradients contract over at most 512 rows (eight
  // 64-deep steps): the short-contraction 128x128 tiles, four workgroups per
  // CU, run them faster than the 256x256 pipeline.
  if (capped && a.kind == 1) return small_tiles(a);
  if (!capped) return launch_tiles<256, 256, 64, 2, 4>(a, st);
  constexpr int kSplitRows = 64;
  GemmArgs b = a;
  b.split_part = 1;
  b.split_rows = kSplitRows;
  b.copy_tokens = 0;  // the dropped tokens of a fused combine are copied by the second launch
  const hipError_t e = launch_tiles<256, 256, 64, 2, 4>(b, st);
  if (e != hipSuccess) return e;
  GemmArgs sm = a;
  sm.split_part = 2;
  sm.split_rows = kSplitRows;
  return small_tiles(sm);
}

}  // namespace moe
