// Grouped bf16 expert GEMMs for batches with many rows per expert (prefill-
// shaped and skewed batches): gate/up with a fused SwiGLU epilogue, and down.
//
// Built around what gfx950 executes fastest:
//  * v_mfma_f32_32x32x16_bf16: one wave keeps the matrix pipe busy with only
//    a few independent accumulators (the 16x16x32 form needs many waves or
//    accumulators per SIMD to hide its latency).  A 16-byte chunk of an
//    operand row is the 8 bf16 one lane supplies; lanes 0-31 and 32-63 take
//    neighbouring chunks, so a stage row of CK chunks feeds CK/2 MFMA K-steps.
//  * Operand tiles move HBM -> LDS with the direct-to-LDS load
//    (global_load_lds_dwordx4): no staging registers or ds_write.  One wave
//    instruction fills a contiguous KiB of stage rows, so each lane fetches
//    the chunk that the row's XOR swizzle places in its slot; the swizzle
//    keeps the 32-row fragment reads free of bank conflicts.
//  * NS named LDS stages (one array each, K-steps of 32 or 64) and a K loop
//    unrolled by NS, NS-1 stages in flight: the
//    compiler can then prove that the stage being read is not the one being
//    filled, and no vmcnt wait separates them.  Each K-step waits (vmcnt)
//    only for its own stage, then one s_barrier.
//  * Balanced tile heights: an expert with m rows gets ceil(m / BM) tiles of
//    equal height, so a tile never holds a lone remainder of a few rows.
//  * 256 x 256 tiles over 8 waves (2 per SIMD) of 128 x 64: one wave's MFMAs
//    run while the other waits on LDS or DMA.
//  * Persistent grid, device-side tile list, XCD-contiguous tile order (as in
//    gemm.hip).

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBigMaxGroups = 1024;

// s_waitcnt with only vmcnt constrained (expcnt, lgkmcnt left at their max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Swizzle of the 16-byte chunk c of tile row r inside a stage whose rows hold
// CK chunks: 8-chunk rows XOR with (r ^ (r >> 3)) & 7, 4-chunk rows with
// ((r >> 1) ^ (r >> 3)) & 3.  Either keeps every 8-lane group (32 banks) and
// every 16-lane group (64 banks) of a 32-row fragment read on distinct banks.
template <int CK>
__device__ __forceinline__ int swz(int r, int c) {
  if (CK == 8) return c ^ ((r ^ (r >> 3)) & 7);
  return c ^ (((r >> 1) ^ (r >> 3)) & 3);
}

template <int MODE, int BM, int BN, int WM, int WN, int NS, int CK, int MG>
__global__ void __launch_bounds__(64 * WM * WN, 1)
grouped_gemm_big_kernel(GemmArgs g) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int RB = CK * 16;                       // bytes per stage row
  constexpr int RPK = 1024 / RB;                    // rows per KiB
  constexpr int KS = CK * 8;                        // K elements per stage
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;       // 32x32 blocks per wave
  constexpr int HN = (MODE == 1) ? BN / 2 : BN;     // output columns per tile
  constexpr int A_KB = BM / RPK, B_KB = BN / RPK;    // KiB chunks per stage
  static_assert(A_KB % NW == 0 && B_KB % NW == 0, "chunks per wave");
  constexpr int A_PW = A_KB / NW, B_PW = B_KB / NW;  // DMA instructions per wave
  constexpr int L = A_PW + B_PW;
  static_assert(NS >= 2 && NS <= 4, "two to four stages");
  static_assert(CK == 4 || CK == 8, "64- or 128-byte stage rows");
  static_assert(L * (NS - 1) < 64, "vmcnt range");
  static_assert(MODE != 1 || NB % 2 == 0, "gate/up pairing");

  // One array per stage (see the header comment).
  __shared__ __attribute__((aligned(1024))) char s_a0[BM * RB];
  __shared__ __attribute__((aligned(1024))) char s_a1[BM * RB];
  __shared__ __attribute__((aligned(1024))) char s_a2[NS >= 3 ? BM * RB : 16];
  __shared__ __attribute__((aligned(1024))) char s_a3[NS >= 4 ? BM * RB : 16];
  __shared__ __attribute__((aligned(1024))) char s_b0[BN * RB];
  __shared__ __attribute__((aligned(1024))) char s_b1[BN * RB];
  __shared__ __attribute__((aligned(1024))) char s_b2[NS >= 3 ? BN * RB : 16];
  __shared__ __attribute__((aligned(1024))) char s_b3[NS >= 4 ? BN * RB : 16];
  __shared__ int s_mt[kBigMaxGroups + 1];
  __shared__ int s_tmp[NT / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r32 = lane & 31, kg = lane >> 5;
  const int ngroups = g.ngroups;

  // ---- per-group tile counts -> prefix sums in LDS
  {
    constexpr int PER = (kBigMaxGroups + NT - 1) / NT;
    int loc[PER];
    int run = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int gi = tid * PER + i;
      int mt = 0;
      if (gi < ngroups) mt = (g.offsets[gi + 1] - g.offsets[gi] + BM - 1) / BM;
      run += mt;
      loc[i] = run;
    }
    const int incl = block_inclusive_scan<NT>(run, s_tmp);
    const int base = incl - run;
    if (tid == 0) s_mt[0] = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int gi = tid * PER + i;
      if (gi < ngroups) s_mt[gi + 1] = base + loc[i];
    }
    __syncthreads();
  }
  const int ntiles = (g.N + HN - 1) / HN;
  const long total = (long)s_mt[ngroups] * ntiles;
  const int G = gridDim.x, b = blockIdx.x;
  const int vid = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int nK = g.K / KS;  // the host guarantees nK % NS == 0
  const size_t row_bytes = (size_t)g.K * 2;

  // DMA lane geometry: lane fills slot (lane % CK) of row (lane / CK) of a
  // KiB and fetches the logical chunk that the swizzle of that tile row
  // stores in the slot (the swizzle is an involution in c for a fixed row).
  const int dma_row = lane / CK;
  const int dma_slot = lane % CK;

  for (long t = vid; t < total; t += G) {
    int lo = 0, hi = ngroups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((long)s_mt[mid] * ntiles <= t) lo = mid; else hi = mid - 1;
    }
    const int grp = lo;
    const int mt_g = s_mt[grp + 1] - s_mt[grp];
    const long local = t - (long)s_mt[grp] * ntiles;
    // Within an expert, tiles go in groups of MG m-tiles x all n-tiles (n-tile
    // major inside a group), so the tiles that run together on one XCD share
    // both their token-row slices and their weight slices in L2.
    const int grp_m0 = (int)(local / ((long)MG * ntiles)) * MG;
    const int mg = min(MG, mt_g - grp_m0);
    const int in_grp = (int)(local - (long)grp_m0 * ntiles);
    const int nt = in_grp / mg, mi = grp_m0 + in_grp % mg;
    const int row0 = g.offsets[grp];
    const int cnt = g.offsets[grp + 1] - row0;
    const int h = ((cnt + mt_g - 1) / mt_g + 31) & ~31;  // balanced tile height
    const int m0 = mi * h;
    const int m_end = min(cnt, m0 + h);                  // rows [m0, m_end)
    const int n0 = nt * HN;

    // ---- per-lane DMA source offsets (32-bit; bases are wave-uniform)
    const char* a_base = (const char*)g.a;
    uint32_t a_off[A_PW];
#pragma unroll
    for (int q = 0; q < A_PW; ++q) {
      const int r = (wave + q * NW) * RPK + dma_row;  // tile row
      int rr = m0 + r;
      if (rr > m_end - 1) rr = m_end - 1;
      long src_row;
      if (MODE == 1 && g.perm != nullptr) {
        src_row = g.perm[row0 + rr] / g.top_k;  // gather token rows on load
        if (src_row < 0 || src_row >= g.M) src_row = 0;
      } else {
        src_row = row0 + rr;
      }
      a_off[q] = (uint32_t)(src_row * row_bytes) + swz<CK>(r, dma_slot) * 16;
    }
    const char* b_base0 = (const char*)g.b0 + (size_t)grp * g.N * row_bytes;
    const char* b_base1 =
        (MODE == 1) ? (const char*)g.b1 + (size_t)grp * g.N * row_bytes : b_base0;
    uint32_t b_off[B_PW];
#pragma unroll
    for (int q = 0; q < B_PW; ++q) {
      const int r = (wave + q * NW) * RPK + dma_row;
      int n = (MODE == 1 && r >= HN) ? n0 + r - HN : n0 + r;
      if (n > g.N - 1) n = g.N - 1;
      b_off[q] = (uint32_t)(n * row_bytes) + swz<CK>(r, dma_slot) * 16;
    }

    f32x16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x16_t{};

    auto stage_a = [&](auto bufc) -> char* {
      constexpr int BUF = decltype(bufc)::value;
      return BUF == 0 ? s_a0 : (BUF == 1 ? s_a1 : (BUF == 2 ? s_a2 : s_a3));
    };
    auto stage_b = [&](auto bufc) -> char* {
      constexpr int BUF = decltype(bufc)::value;
      return BUF == 0 ? s_b0 : (BUF == 1 ? s_b1 : (BUF == 2 ? s_b2 : s_b3));
    };

    // every stage issues exactly L loads per wave (the vmcnt waits count on
    // it); rows past the tile were clamped to its last row above
    auto issue = [&](auto bufc, int ks) {
      char* sa = stage_a(bufc);
      char* sb = stage_b(bufc);
      const size_t off = (size_t)ks * RB;
#pragma unroll
      for (int q = 0; q < A_PW; ++q) {
        const int kb = wave + q * NW;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(a_base + a_off[q] + off),
                                         (lds_void_t*)(sa + kb * 1024), 16, 0, 0);
      }
#pragma unroll
      for (int q = 0; q < B_PW; ++q) {
        const int kb = wave + q * NW;
        // gate rows fill the first half of the B tile, up rows the second
        const char* bb = (MODE == 1 && kb * RPK >= HN) ? b_base1 : b_base0;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(bb + b_off[q] + off),
                                         (lds_void_t*)(sb + kb * 1024), 16, 0, 0);
      }
    };

    auto brow = [&](int j) {
      if (MODE == 1)
        return (j < NB / 2) ? wn * (WTN / 2) + j * 32 + r32
                            : HN + wn * (WTN / 2) + (j - NB / 2) * 32 + r32;
      return wn * WTN + j * 32 + r32;
    };

    // One K-step of 64: wait for this stage's DMA (newer stages may stay in
    // flight), barrier, start the DMA NS-1 steps ahead into the stage freed
    // by the previous step, then 4 MFMA K-slices of 16 with the fragments of
    // slice kk+1 read from LDS while slice kk computes.
    auto kstep = [&](auto bufc, int ks) {
      constexpr int BUF = decltype(bufc)::value;
      const char* sa = stage_a(bufc);
      const char* sb = stage_b(bufc);
      // stages newer than this one that may still be in flight
      const int ahead = min(NS - 2, nK - 1 - ks);
      if (NS >= 4 && ahead >= 2) wait_vmcnt<(NS >= 4 ? 2 * L : 0)>();
      else if (NS >= 3 && ahead >= 1) wait_vmcnt<(NS >= 3 ? L : 0)>();
      else wait_vmcnt<0>();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      if (ks + NS - 1 < nK) issue(std::integral_constant<int, (BUF + NS - 1) % NS>{}, ks + NS - 1);
      // favour this wave's MFMA issue over the other wave on the SIMD
      __builtin_amdgcn_s_setprio(1);
      u32x4_t af[2][MB], bfr[2][NB];
      auto load = [&](int set, int kk) {
        const int c = kk * 2 + kg;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int r = (i * WM + wm) * 32 + r32;
          af[set][i] = *reinterpret_cast<const u32x4_t*>(&sa[r * RB + (swz<CK>(r, c) << 4)]);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int r = brow(j);
          bfr[set][j] = *reinterpret_cast<const u32x4_t*>(&sb[r * RB + (swz<CK>(r, c) << 4)]);
        }
      };
      constexpr int NKK = CK / 2;  // MFMA K-slices of 16 per stage
      load(0, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + 1 < NKK) load((kk + 1) & 1, kk + 1);
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, bfr[kk & 1][j]),
                __builtin_bit_cast(bf16x8_t, af[kk & 1][i]), acc[i][j], 0, 0, 0);
      }
      // Pin the schedule (the default one sinks every LDS read next to its
      // first use and stalls on it): the first slice's reads, then each
      // slice's MFMAs with the next slice's reads interleaved 1:1 at the
      // front, so they have landed before that slice starts.
      constexpr int NR = MB + NB;        // LDS reads per slice
      constexpr int NM = MB * NB;        // MFMAs per slice
      static_assert(NM >= NR, "read/MFMA interleave");
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
      for (int kk = 0; kk + 1 < NKK; ++kk) {
#pragma unroll
        for (int q = 0; q < NR; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
      __builtin_amdgcn_s_setprio(0);
    };

    // previous tile's epilogue stores and LDS reads must be done before the
    // stage buffers are refilled and before vmcnt counts only this tile's DMA
    wait_vmcnt<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    issue(std::integral_constant<int, 0>{}, 0);
    if (NS >= 3 && nK > 1) issue(std::integral_constant<int, 1>{}, 1);
    if (NS >= 4 && nK > 2) issue(std::integral_constant<int, 2>{}, 2);
    for (int ks = 0; ks < nK; ks += NS) {
      kstep(std::integral_constant<int, 0>{}, ks);
      kstep(std::integral_constant<int, 1>{}, ks + 1);
      if (NS >= 3) kstep(std::integral_constant<int, (NS >= 3 ? 2 : 0)>{}, ks + 2);
      if (NS >= 4) kstep(std::integral_constant<int, (NS >= 4 ? 3 : 0)>{}, ks + 3);
    }

    // ---- epilogue.  Weights were the MFMA row operand, so block (i, j) is
    // C^T: lane (r32, kg) holds, for quad q = v / 4, the 4 consecutive output
    // columns 8q + 4kg + {0..3} of token row r32 -> one packed 8-byte store.
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r = m0 + (i * WM + wm) * 32 + r32;
      if (r < m_end) {
        char* crow = (char*)g.c + (size_t)(row0 + r) * g.N * 2;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (MODE == 1) {
#pragma unroll
            for (int j = 0; j < NB / 2; ++j) {
              const int col = n0 + wn * (WTN / 2) + j * 32 + 8 * q + 4 * kg;
              float hv[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float z = acc[i][j][4 * q + e];
                // silu(z) = z * sigmoid(z) with hardware exp2 / reciprocal
                // (H is rounded to bf16 right after)
                const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504f));
                hv[e] = z * sg * acc[i][j + NB / 2][4 * q + e];
              }
              if (col + 3 < g.N) {
                const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hv[0]) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hv[1]) << 16);
                const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hv[2]) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hv[3]) << 16);
                *reinterpret_cast<uint2*>(crow + col * 2) = make_uint2(lo, hi);
              }
            }
          } else {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const int col = n0 + wn * WTN + j * 32 + 8 * q + 4 * kg;
              if (col + 3 < g.N) {
                const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[i][j][4 * q]) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[i][j][4 * q + 1]) << 16);
                const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[i][j][4 * q + 2]) |
                                    ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)acc[i][j][4 * q + 3]) << 16);
                *reinterpret_cast<uint2*>(crow + col * 2) = make_uint2(lo, hi);
              }
            }
          }
        }
      }
    }
  }
}

#ifndef MOE_HUGE_TILE
#define MOE_HUGE_TILE 256, 256, 2, 4, 2, 8, 4
#endif

template <int BM, int BN, int WM, int WN, int NS, int CK, int MG>
struct BigCfg {
  static constexpr int KSTEP_MULT = NS * CK * 8;  // K must be a multiple of this
  static constexpr int NT = 64 * WM * WN;
};

template <int MODE>
static int launch_big_mode(const GemmArgs& g, hipStream_t st) {
  auto kern = grouped_gemm_big_kernel<MODE, MOE_HUGE_TILE>;
  const int cus = device_cu_count();
  if (cus <= 0) return MOE_EHIP;
  int grid = cus;  // one workgroup per CU (LDS bound)
  grid -= grid % 8;
  if (grid < 8) grid = 8;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(BigCfg<MOE_HUGE_TILE>::NT), 0, st, g);
  return check_launch();
}

int launch_gemm_big(int mode, const GemmArgs& g, hipStream_t st) {
  return mode == 1 ? launch_big_mode<1>(g, st) : launch_big_mode<2>(g, st);
}

}  // namespace moe
