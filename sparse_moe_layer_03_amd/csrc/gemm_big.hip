// Grouped bf16 expert GEMMs for batches with many rows per expert (prefill-
// shaped and skewed batches): gate/up with a fused SwiGLU epilogue, and down.
// The same kernel (mode 0) runs the router GEMM of a many-token batch with
// more than 128 experts: one group of T rows, fp32 partial logits, its K
// loop split into ksplit ranges so that (split, tile) items fill the chip.
//
// Built around what gfx950 executes fastest:
//  * v_mfma_f32_32x32x16_bf16: one wave keeps the matrix pipe busy with only
//    a few independent accumulators (the 16x16x32 form needs many waves or
//    accumulators per SIMD to hide its latency).  A 16-byte chunk of an
//    operand row is the 8 bf16 one lane supplies; lanes 0-31 and 32-63 take
//    neighbouring chunks, so a 128-byte stage row feeds 4 MFMA K-slices.
//  * Operand tiles move HBM -> LDS with the direct-to-LDS load
//    (global_load_lds_dwordx4): no staging registers or ds_write.  One wave
//    instruction fills a contiguous KiB of stage rows, so each lane fetches
//    the chunk that the row's XOR swizzle places in its slot; the swizzle
//    keeps the 32-row fragment reads free of bank conflicts.
//  * Two rings of named LDS stages (one array each, K-steps of 64): token
//    rows in 2 stages, weights in 3.  Token rows are re-read by every n-tile
//    of an expert and mostly hit L2, so one step of lead hides them; the
//    weight slice of a step usually comes from HBM and is issued two steps
//    ahead.  2 x 32 KiB + 3 x 32 KiB fill the 160 KiB of LDS.  The K loop is
//    unrolled by 6 (both ring positions static), so the compiler can prove
//    that the stage being read is not one being filled and emits no vmcnt
//    wait between them.  Each K-step waits (vmcnt) only for its own stages,
//    then one s_barrier.
//  * The direct-to-LDS loads of a main-loop step are issued two per MFMA
//    K-slice (token rows in the first two slices, weights in the last two),
//    not all after the barrier: their issue stalls until earlier ones have
//    drained into LDS, and eight waves issuing at once had kept every SIMD's
//    MFMAs waiting for about a third of each step.
//  * Balanced tile heights: an expert with m rows gets ceil(m / 256) tiles of
//    equal height (a multiple of 32).  A wave runs the MFMAs of only the
//    32-row blocks that hold rows: the K loop exists once per count of
//    active blocks, chosen per tile, so a 160-row tile does 5/8 of the MFMA
//    work of a full one (its DMA and barriers cost the same).
//  * A last round of the persistent grid that is at most half full has its
//    tiles cut into row slices (at least 32 rows each) over the idle CUs.
//  * 256 x 256 tiles over 8 waves (2 per SIMD) of 128 x 64: one wave's MFMAs
//    run while the other waits on LDS or DMA.
//  * Persistent grid, XCD-contiguous tile order (as in gemm.hip); each
//    workgroup finds the experts of its own tiles at the start.

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace moe {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// s_waitcnt with only vmcnt constrained (expcnt, lgkmcnt left at their max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4) | (0x0 << 8));
}

// Swizzle of the 16-byte chunk c of tile row r in a 128-byte stage row:
// XOR with (r ^ (r >> 3)) & 7 keeps every 8-lane group (32 banks) and every
// 16-lane group (64 banks) of a 32-row fragment read on distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r ^ (r >> 3)) & 7); }

constexpr int kBigMaxGroups = 1024;

template <int MODE, int MG>
__global__ void __launch_bounds__(512, 1)
grouped_gemm_big_kernel(GemmArgs g) {
  constexpr int BM = kBigTileRows, BN = 256, WM = 2, WN = 4, NW = WM * WN, NT = 64 * NW;
  constexpr int RB = 128;                           // bytes per stage row
  constexpr int RPK = 1024 / RB;                    // stage rows per KiB
  constexpr int KS = RB / 2;                        // K elements per stage
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 32, NB = WTN / 32;       // 32x32 blocks per wave
  constexpr int HN = (MODE == 1) ? BN / 2 : BN;     // output columns per tile
  constexpr int A_PW = BM / RPK / NW;               // DMA instructions per wave
  constexpr int B_PW = BN / RPK / NW;
  constexpr int NKK = KS / 16;                      // MFMA K-slices per stage
  static_assert(MODE != 1 || NB % 2 == 0, "gate/up pairing");
  static_assert(A_PW + 2 * B_PW < 64, "vmcnt range");

  // One array per stage (see the header comment).
  __shared__ __attribute__((aligned(1024))) char s_a0[BM * RB];
  __shared__ __attribute__((aligned(1024))) char s_a1[BM * RB];
  __shared__ __attribute__((aligned(1024))) char s_b0[BN * RB];
  __shared__ __attribute__((aligned(1024))) char s_b1[BN * RB];
  __shared__ __attribute__((aligned(1024))) char s_b2[BN * RB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wave / WN, wn = wave % WN;
  const int r32 = lane & 31, kg = lane >> 5;

  const int ngroups = g.ngroups;
  const int ntiles = (g.N + HN - 1) / HN;
  const int G = gridDim.x, b = blockIdx.x;
  const int vid = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;

  // ---- this workgroup's tiles.  The per-group m-tile prefix is built in the
  // first token-row stage (no DMA has started yet); lane l of every wave then
  // looks up the group of tiles vid + l*G and vid + (64 + l)*G and keeps it,
  // packed with the group's first m-tile, in one register each (the host
  // guarantees at most 128 tiles per workgroup); the tile loop reads them
  // back with readlane.
  int* s_pref = reinterpret_cast<int*>(s_a0);  // ngroups + 1 <= 1025 ints
  int* s_scan = reinterpret_cast<int*>(s_a1);  // NT / 64 ints
  {
    constexpr int PER = (kBigMaxGroups + NT - 1) / NT;
    int loc[PER];
    int run = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int gi = tid * PER + i;
      int mt = 0;
      if (gi < ngroups)
        mt = ((MODE == 0 ? g.M : g.offsets[gi + 1] - g.offsets[gi]) + BM - 1) / BM;
      run += mt;
      loc[i] = run;
    }
    const int incl = block_inclusive_scan<NT>(run, s_scan);
    const int base = incl - run;
    if (tid == 0) s_pref[0] = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int gi = tid * PER + i;
      if (gi < ngroups) s_pref[gi + 1] = base + loc[i];
    }
    __syncthreads();
  }
  // the router (mode 0) splits its K loop: work item t is split t / tiles
  // of tile t % tiles, so the tiles running together share a K range
  const int ksplit = (MODE == 0) ? g.ksplit : 1;
  const int tiles = s_pref[ngroups] * ntiles;
  // Tail split (expert modes): when the last round of the persistent grid
  // is at most half full, each of its tiles is cut into f row slices, so
  // the slices spread over the idle CUs.  Items below `full` are whole
  // tiles; item full + j is slice j % f of tile full + j / f.
  const int full = tiles - tiles % G;
  const int rem = tiles - full;
  const int f = (MODE != 0 && rem > 0 && 2 * rem <= G) ? min(8, G / rem) : 1;
  const int total = (full + rem * f) * ksplit;
  auto tile_of = [&](int it) { return it < full ? it : full + (it - full) / f; };
  auto find = [&](int t) -> uint32_t {  // (first m-tile << 10) | group
    if (t >= tiles) return 0;
    const int m = t / ntiles;
    int lo = 0, hi = ngroups - 1;  // last group with s_pref[grp] <= m
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pref[mid] <= m) lo = mid; else hi = mid - 1;
    }
    return ((uint32_t)s_pref[lo] << 10) | (uint32_t)lo;
  };
  const uint32_t tdesc0 = (MODE == 0) ? 0u : find(tile_of(vid + lane * G));
  const uint32_t tdesc1 = (MODE == 0) ? 0u : find(tile_of(vid + (64 + lane) * G));
  __syncthreads();  // the prefix is dead before the first DMA into s_a0
  const int nK = g.K / KS / ksplit;  // per split; the host guarantees an even count
  const size_t row_bytes = (size_t)g.K * 2;

  // DMA lane geometry: lane fills slot (lane % 8) of row (lane / 8) of a KiB
  // and fetches the logical chunk that the swizzle of that tile row stores
  // in the slot (the swizzle is an involution in c for a fixed row).
  const int dma_row = lane / 8;
  const int dma_slot = lane % 8;

  for (int k = 0; vid + k * G < total; ++k) {
    const int tsplit = (MODE == 0) ? (vid + k * G) / tiles : 0;
    const int it = vid + k * G - tsplit * tiles;  // item (== tile unless sliced)
    const int t = tile_of(it);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane(
        (int)(k < 64 ? tdesc0 : tdesc1), k & 63);
    const int grp = (MODE == 0) ? 0 : (int)(d & 1023u);
    const int tp0 = (MODE == 0) ? 0 : (int)(d >> 10);
    const int cnt_g = (MODE == 0) ? g.M : g.offsets[grp + 1] - g.offsets[grp];
    const int mt_g = (cnt_g + BM - 1) / BM;
    const int local = t - tp0 * ntiles;
    // Within an expert, tiles go in groups of MG m-tiles x all n-tiles (n-tile
    // major inside a group), so the tiles that run together on one XCD share
    // both their token-row slices and their weight slices in L2.
    const int grp_m0 = (local / (MG * ntiles)) * MG;
    const int mg = min(MG, mt_g - grp_m0);
    const int in_grp = local - grp_m0 * ntiles;
    const int nt = in_grp / mg, mi = grp_m0 + in_grp % mg;
    const int row0 = (MODE == 0) ? 0 : g.offsets[grp];
    const int cnt = cnt_g;
    const int h = ((cnt + mt_g - 1) / mt_g + 31) & ~31;  // balanced tile height
    int m0 = mi * h;
    int m_end = min(cnt, m0 + h);                        // rows [m0, m_end)
    if (it >= full && f > 1) {
      // slice (it - full) % f of the tile: at least 32 rows each; an empty
      // slice (short tile) is skipped by the whole workgroup
      const int hs = max(32, ((m_end - m0 + f - 1) / f + 31) & ~31);
      const int s0 = m0 + ((it - full) % f) * hs;
      m_end = min(m_end, s0 + hs);
      m0 = s0;
      if (m0 >= m_end) continue;
    }
    const int n0 = nt * HN;
    // 32-row blocks of this wave that hold rows: i with (i*WM + wm)*32 < rows
    const int nrb = (m_end - m0 + 31) / 32;
    const int mba = min(MB, (nrb - wm + WM - 1) / WM);

    // ---- per-lane DMA source offsets (32-bit; bases are wave-uniform),
    // starting at this split's K range
    const uint32_t k_base = (uint32_t)(tsplit * nK * RB);
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
      a_off[q] = (uint32_t)(src_row * row_bytes) + k_base + swz(r, dma_slot) * 16;
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
      b_off[q] = (uint32_t)(n * row_bytes) + k_base + swz(r, dma_slot) * 16;
    }

    f32x16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x16_t{};

    auto stage_a = [&](auto sc) -> char* {
      constexpr int S = decltype(sc)::value;
      return S == 0 ? s_a0 : s_a1;
    };
    auto stage_b = [&](auto sc) -> char* {
      constexpr int S = decltype(sc)::value;
      return S == 0 ? s_b0 : (S == 1 ? s_b1 : s_b2);
    };

    // Every stage issues exactly A_PW (token rows) or B_PW (weights) loads
    // per wave, whatever the tile height (the vmcnt waits count on it); rows
    // past the tile were clamped to its last row above.
    auto issue_a = [&](auto sc, int ks) {
      char* sa = stage_a(sc);
      const size_t off = (size_t)ks * RB;
#pragma unroll
      for (int q = 0; q < A_PW; ++q)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(a_base + a_off[q] + off),
                                         (lds_void_t*)(sa + (wave + q * NW) * 1024), 16, 0, 0);
    };
    auto issue_b = [&](auto sc, int ks) {
      char* sb = stage_b(sc);
      const size_t off = (size_t)ks * RB;
#pragma unroll
      for (int q = 0; q < B_PW; ++q) {
        // gate rows fill the first half of the B tile, up rows the second
        // (wave < NW, so the half is fixed per q)
        const char* bb = (MODE == 1 && (q * NW) * RPK >= HN) ? b_base1 : b_base0;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(bb + b_off[q] + off),
                                         (lds_void_t*)(sb + (wave + q * NW) * 1024), 16, 0, 0);
      }
    };
    static_assert(MODE != 1 || (HN % (NW * RPK) == 0), "gate/up halves align with q");

    auto brow = [&](int j) {
      if (MODE == 1)
        return (j < NB / 2) ? wn * (WTN / 2) + j * 32 + r32
                            : HN + wn * (WTN / 2) + (j - NB / 2) * 32 + r32;
      return wn * WTN + j * 32 + r32;
    };

    // One K-step of 64 on token-row stage AS and weight stage BS, with MBA
    // active 32-row blocks: wait for this step's stages (the weight stage of
    // the next step may stay in flight), barrier, then 4 MFMA K-slices of 16
    // with the fragments of slice kk+1 read from LDS while slice kk computes,
    // refilling the stages the previous step read (token rows one step
    // ahead, weights two) — spread over the slices in the main loop, right
    // after the barrier in the tail.  nac / nbc: whether the step issues the token
    // rows of step ks+1 / the weights of step ks+2.  In the main loop they
    // are compile-time true, so the compiler knows exactly which DMA is still
    // in flight and adds no wait of its own.
    auto kstep = [&](auto mbac, auto asc, auto bsc, auto nac, auto nbc, int ks) {
      constexpr int MBA = decltype(mbac)::value;
      constexpr int AS = decltype(asc)::value, BS = decltype(bsc)::value;
      const bool next_a = nac, next_b = nbc;
      const char* sa = stage_a(asc);
      const char* sb = stage_b(bsc);
      // the weights of step ks+1 were issued by the previous step iff this
      // step issues the token rows of step ks+1
      if (next_a) wait_vmcnt<B_PW>();
      else wait_vmcnt<0>();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      // Keep the DMA lane offsets 32-bit: left alone, the compiler hoists
      // their 64-bit extensions out of the K loop, doubling their registers.
#pragma unroll
      for (int q = 0; q < A_PW; ++q) asm volatile("" : "+v"(a_off[q]));
#pragma unroll
      for (int q = 0; q < B_PW; ++q) asm volatile("" : "+v"(b_off[q]));
      // Main-loop steps (both refills compile-time true) spread their DMA
      // issue over the MFMA slices: a direct-to-LDS load can block issue
      // until earlier ones drain, and all waves issuing theirs at the step
      // start would stall their MFMAs together.  Token rows go first (the
      // step-start vmcnt wait allows only the weights to be in flight).
      constexpr bool SPREAD = std::is_same_v<decltype(nac), std::true_type> &&
                              std::is_same_v<decltype(nbc), std::true_type>;
      if constexpr (!SPREAD) {
        if (next_a) issue_a(std::integral_constant<int, (AS + 1) % 2>{}, ks + 1);
        if (next_b) issue_b(std::integral_constant<int, (BS + 2) % 3>{}, ks + 2);
      }
      // favour this wave's MFMA issue over the other wave on the SIMD
      __builtin_amdgcn_s_setprio(1);
      u32x4_t af[2][MBA], bfr[2][NB];
      auto load = [&](int set, int kk) {
        const int c = kk * 2 + kg;
#pragma unroll
        for (int i = 0; i < MBA; ++i) {
          const int r = (i * WM + wm) * 32 + r32;
          af[set][i] = *reinterpret_cast<const u32x4_t*>(&sa[r * RB + (swz(r, c) << 4)]);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int r = brow(j);
          bfr[set][j] = *reinterpret_cast<const u32x4_t*>(&sb[r * RB + (swz(r, c) << 4)]);
        }
      };
      // DMA pieces of slice kk: A loads 2kk, 2kk+1 (kk < 2), B loads 2(kk-2), 2(kk-2)+1
      auto dma_piece = [&](int kk) {
        if (kk < 2) {
          char* sa2 = stage_a(std::integral_constant<int, (AS + 1) % 2>{});
          const size_t off = (size_t)(ks + 1) * RB;
#pragma unroll
          for (int q = 2 * kk; q < 2 * kk + 2; ++q)
            __builtin_amdgcn_global_load_lds((glb_void_t*)(a_base + a_off[q] + off),
                                             (lds_void_t*)(sa2 + (wave + q * NW) * 1024), 16, 0, 0);
        } else {
          char* sb2 = stage_b(std::integral_constant<int, (BS + 2) % 3>{});
          const size_t off = (size_t)(ks + 2) * RB;
#pragma unroll
          for (int q = 2 * (kk - 2); q < 2 * (kk - 2) + 2; ++q) {
            const char* bb = (MODE == 1 && (q * NW) * RPK >= HN) ? b_base1 : b_base0;
            __builtin_amdgcn_global_load_lds((glb_void_t*)(bb + b_off[q] + off),
                                             (lds_void_t*)(sb2 + (wave + q * NW) * 1024), 16, 0, 0);
          }
        }
      };
      static_assert(!SPREAD || (A_PW == 4 && B_PW == 4 && NKK == 4), "two DMA loads per slice");
      // Pin the schedule (the default one sinks every LDS read next to its
      // first use and stalls on it): the first slice's reads, then each
      // slice's MFMAs with the next slice's reads interleaved 1:1 at the
      // front, so they have landed before that slice starts.  Main-loop
      // steps place one DMA load before each half of a slice's pairs; a
      // scheduling fence after every slice keeps the token-row loads ahead of
      // the weight loads, which the step-start vmcnt wait relies on.
      constexpr int NR = MBA + NB;       // LDS reads per slice
      constexpr int NM = MBA * NB;       // MFMAs per slice
      constexpr int NP = NR < NM ? NR : NM;
      constexpr int H1 = NP / 2;
      load(0, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + 1 < NKK) load((kk + 1) & 1, kk + 1);
        if constexpr (SPREAD) dma_piece(kk);
#pragma unroll
        for (int i = 0; i < MBA; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8_t, bfr[kk & 1][j]),
                __builtin_bit_cast(bf16x8_t, af[kk & 1][i]), acc[i][j], 0, 0, 0);
        if (kk + 1 < NKK) {
          if constexpr (SPREAD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
#pragma unroll
          for (int q = 0; q < H1; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
          if constexpr (SPREAD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
#pragma unroll
          for (int q = H1; q < NP; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          }
          if constexpr (NR > NP) __builtin_amdgcn_sched_group_barrier(0x100, NR - NP, 0);
          if constexpr (NM > NP) __builtin_amdgcn_sched_group_barrier(0x008, NM - NP, 0);
        } else {
          if constexpr (SPREAD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NM / 2, 0);
          if constexpr (SPREAD) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, NM - NM / 2, 0);
        }
        if constexpr (SPREAD) __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using T = std::true_type;
    // The K loop for MBA active blocks up to the tail: both ring positions
    // repeat every 6 steps, and the loop runs while every step in it has both
    // refills to issue (ks + 8 <= nK); K is a multiple of 128, so 2, 4 or 6
    // steps remain for the tail.  Returns the first tail step.
    auto kloop = [&](auto mbac) {
      // previous tile's epilogue stores and LDS reads must be done before the
      // stages are refilled and before vmcnt counts only this tile's DMA
      wait_vmcnt<0>();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      issue_a(I0{}, 0);
      issue_b(I0{}, 0);
      issue_b(I1{}, 1);  // nK >= 2
      int ks = 0;
      for (; ks + 8 <= nK; ks += 6) {
        kstep(mbac, I0{}, I0{}, T{}, T{}, ks);
        kstep(mbac, I1{}, I1{}, T{}, T{}, ks + 1);
        kstep(mbac, I0{}, I2{}, T{}, T{}, ks + 2);
        kstep(mbac, I1{}, I0{}, T{}, T{}, ks + 3);
        kstep(mbac, I0{}, I1{}, T{}, T{}, ks + 4);
        kstep(mbac, I1{}, I2{}, T{}, T{}, ks + 5);
      }
      return ks;
    };
    // a wave with no rows (mba == 0) still loads and waits with the others;
    // its one block of clamped rows is never stored
    int ks;
    if (mba >= 4) ks = kloop(std::integral_constant<int, 4>{});
    else if (mba == 3) ks = kloop(std::integral_constant<int, 3>{});
    else if (mba == 2) ks = kloop(std::integral_constant<int, 2>{});
    else ks = kloop(std::integral_constant<int, 1>{});
    // The last 2, 4 or 6 steps run every block (one copy of the code; blocks
    // without rows are never stored) with refills decided at run time.
    {
      using M4 = std::integral_constant<int, 4>;
      kstep(M4{}, I0{}, I0{}, ks + 1 < nK, ks + 2 < nK, ks);
      kstep(M4{}, I1{}, I1{}, ks + 2 < nK, ks + 3 < nK, ks + 1);
      if (ks + 4 <= nK) {
        kstep(M4{}, I0{}, I2{}, ks + 3 < nK, ks + 4 < nK, ks + 2);
        kstep(M4{}, I1{}, I0{}, ks + 4 < nK, ks + 5 < nK, ks + 3);
      }
      if (ks + 6 <= nK) {
        kstep(M4{}, I0{}, I1{}, ks + 5 < nK, ks + 6 < nK, ks + 4);
        kstep(M4{}, I1{}, I2{}, false, false, ks + 5);
      }
    }

    // ---- epilogue.  Weights were the MFMA row operand, so block (i, j) is
    // C^T: lane (r32, kg) holds, for quad q = v / 4, the 4 consecutive output
    // columns 8q + 4kg + {0..3} of token row r32 -> one packed 8-byte store.
    // Blocks past the wave's active ones hold rows >= m_end and are skipped.
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r = m0 + (i * WM + wm) * 32 + r32;
      if (r < m_end) {
        char* crow = (char*)g.c + (size_t)(row0 + r) * g.N * 2;
        float* prow = (float*)g.c + ((size_t)tsplit * g.M + r) * g.N;  // mode 0
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (MODE == 0) {
            // fp32 partial logits of this K split, [split][T][E]
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const int col = n0 + wn * WTN + j * 32 + 8 * q + 4 * kg;
              if ((g.N & 3) == 0 && col + 3 < g.N) {
                *reinterpret_cast<float4*>(prow + col) =
                    make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                acc[i][j][4 * q + 3]);
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (col + e < g.N) prow[col + e] = acc[i][j][4 * q + e];
              }
            }
          } else if (MODE == 1) {
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

#ifndef MOE_BIG_MG
#define MOE_BIG_MG 4
#endif

int big_grid() {
  int grid = device_cu_count();  // one workgroup per CU (LDS bound)
  grid -= grid % 8;
  return grid < 8 ? 8 : grid;
}

template <int MODE>
static int launch_big_mode(const GemmArgs& g, hipStream_t st) {
  auto kern = grouped_gemm_big_kernel<MODE, MOE_BIG_MG>;
  if (device_cu_count() <= 0) return MOE_EHIP;
  hipLaunchKernelGGL(kern, dim3(big_grid()), dim3(512), 0, st, g);
  return check_launch();
}

int launch_gemm_big(int mode, const GemmArgs& g, hipStream_t st) {
  if (g.K % 128 != 0 || g.ngroups < 1 || g.ngroups > kBigMaxGroups) return MOE_EINVAL;
  if (mode == 0) {
    // each split covers an even number (>= 2) of 64-wide K-steps
    if (g.ngroups != 1 || g.ksplit < 1 || (g.K / 64) % (2 * g.ksplit) != 0) return MOE_EINVAL;
    return launch_big_mode<0>(g, st);
  }
  return mode == 1 ? launch_big_mode<1>(g, st) : launch_big_mode<2>(g, st);
}

}  // namespace moe
