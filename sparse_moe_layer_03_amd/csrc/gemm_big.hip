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
//  * A second tile shape, 320 x 192 on 16x16x32 MFMAs, takes the experts of
//    257..320 rows in one tile (a batch averaging 256 rows per expert has
//    about half of them there); split into two 256-row tiles, each would
//    stream the expert's whole weight slice through LDS.  Its own launch
//    runs before the 256-row one, when those experts fill four rounds of the
//    grid.  The down GEMM's 256 x 256 tiles run on 16x16x32 MFMAs as well
//    (16-row blocks: half the padding of the 32-row ones).
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
#include "plan.h"

namespace moe {

// cache-policy operand of a load: non-temporal
constexpr int kCpolNT = 2;

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
constexpr int kGateUp16MinK = 4096;  // gate/up's 256 x 256 tiles on 16x16x32 MFMAs from here
constexpr int kBigDescRegs = 4;  // tile descriptors: 64 per register
static_assert(64 * kBigDescRegs == plan::kBigMaxTilesPerWg, "host bound on items per workgroup");
static_assert(kBigMaxGroups == plan::kBigMaxGroups && kBigTileRows == plan::kBigTileRows,
              "host plan matches the kernel");
static_assert(plan::kR320Lo > kBigTileRows && plan::kR320Hi <= 320, "320-row tiles");

// The tile shapes.
//  0: 256 x 256 on 32x32x16 MFMAs, 8 waves of 128 x 64: the router, and the
//     gate/up experts outside 257..320 rows when d_model < 4096.
//  1: 320 x 192 on 16x16x32 MFMAs, 8 waves of 80 x 96 (120 accumulators per
//     lane, 152 KiB of LDS): an expert with 257..320 rows in one tile
//     instead of two, so its weight slice passes through LDS once.
//  2: 256 x 256 on 16x16x32 MFMAs, 8 waves of 64 x 128: the down experts
//     outside 257..320 rows, and the gate/up ones when d_model >= 4096.
//     Rows come in blocks of 16, so a tile's last block carries 8 padding
//     rows on average instead of 16; it ran faster than shape 0 for down on
//     every workload (prefill 3.83 -> 3.73 ms).  Its fragments are read
//     once per K-slice (a second set does not fit next to 128
//     accumulators).
template <int SHAPE>
struct BigShape {
  static constexpr int BM = SHAPE == 1 ? 320 : 256, BN = SHAPE == 1 ? 192 : 256;
  static constexpr int WM = SHAPE == 0 ? 2 : 4, WN = SHAPE == 0 ? 4 : 2;
  static constexpr int BLK = SHAPE == 0 ? 32 : 16;  // rows and weight rows per MFMA block
  static constexpr int KSL = SHAPE == 0 ? 16 : 32;  // K per MFMA
};

// Whether a group of `cnt` rows runs on the 320-row kernel (both kernels
// decide alike, so every group runs on exactly one of them).
__device__ __forceinline__ bool rows320(const GemmArgs& g, int cnt) {
  return g.r320_hi > 0 && cnt >= g.r320_lo && cnt <= g.r320_hi && cnt <= 320;
}

template <int MODE, int MG, int SHAPE>
__global__ void __launch_bounds__(512, 1)
grouped_gemm_big_kernel(GemmArgs g) {
  constexpr bool R320 = SHAPE == 1;
  using SH = BigShape<SHAPE>;
  constexpr int BM = SH::BM, BN = SH::BN, WM = SH::WM, WN = SH::WN, NW = WM * WN, NT = 64 * NW;
  constexpr int BLK = SH::BLK;
  constexpr int RB = 128;                           // bytes per stage row
  constexpr int RPK = 1024 / RB;                    // stage rows per KiB
  constexpr int KS = RB / 2;                        // K elements per stage
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / BLK, NB = WTN / BLK;     // MFMA blocks per wave
  constexpr int HN = (MODE == 1) ? BN / 2 : BN;     // output columns per tile
  constexpr int A_PW = BM / RPK / NW;               // DMA instructions per wave
  constexpr int B_PW = BN / RPK / NW;
  constexpr int NKK = KS / SH::KSL;                 // MFMA K-slices per stage
  constexpr int DPS = (A_PW + B_PW) / NKK;          // DMA instructions per slice
  constexpr bool B16 = SH::BLK == 16;  // 16x16x32 MFMAs, all K-steps in kloop
  using acc_t = std::conditional_t<B16, f32x4_t, f32x16_t>;
  static_assert(MODE != 1 || NB % 2 == 0, "gate/up pairing");
  static_assert(A_PW + 2 * B_PW < 64, "vmcnt range");
  static_assert(DPS * NKK == A_PW + B_PW, "DMA spread evenly over the slices");
  static_assert(!B16 || MODE != 0, "16x16 tiles: experts only");
  static_assert(HN % RPK == 0, "one DMA instruction's rows lie in one gate/up half");
  static_assert(BM * RB * 2 + BN * RB * 3 <= 160 * 1024, "LDS");

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
  const int rin = lane & (BLK - 1);  // row of an MFMA block this lane supplies
  const int kg = lane / BLK;         // its 16-byte K chunk within the K-slice

  const int ngroups = g.ngroups;
  const int ntiles = (g.N + HN - 1) / HN;
  const int G = gridDim.x, b = blockIdx.x;
  const int vid = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;

  // ---- this workgroup's tiles.  The per-group m-tile prefix is built in the
  // first token-row stage (no DMA has started yet); lane l of every wave then
  // looks up the group of tiles vid + (64 j + l)*G, j < kBigDescRegs, and
  // keeps it, packed with the group's first m-tile, in register j (the host
  // guarantees at most 64 * kBigDescRegs tiles per workgroup); the tile loop
  // reads them back with readlane.
  int* s_pref = reinterpret_cast<int*>(s_a0);  // ngroups + 1 <= 1025 ints
  int* s_scan = reinterpret_cast<int*>(s_a1);  // NT / 64 + 1 ints
  constexpr int PER = (kBigMaxGroups + NT - 1) / NT;
  // The 320-row tiles are used only when they fill at least four rounds of
  // the grid (their launch's partly idle last round costs up to one round);
  // both tile shapes count the groups alike.
  bool use320 = false;
  if (MODE != 0 && g.r320_hi > 0) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int gi = tid * PER + i;
      if (gi < ngroups && rows320(g, g.offsets[gi + 1] - g.offsets[gi])) ++n;
    }
    const int incl = block_inclusive_scan<NT>(n, s_scan);
    if (tid == NT - 1) s_scan[NT / 64] = incl;
    __syncthreads();
    constexpr int HN320 = MODE == 1 ? BigShape<true>::BN / 2 : BigShape<true>::BN;
    // (four rounds of one workgroup per CU: the grid is grid_mult of them)
    use320 = s_scan[NT / 64] * ((g.N + HN320 - 1) / HN320) >=
             4 * (int)gridDim.x / max(1, g.grid_mult);
  }
  // m-tiles of a group of cnt rows on this kernel (none for the groups the
  // other tile shape runs)
  auto mtiles = [&](int cnt) -> int {
    if (MODE == 0) return (cnt + BM - 1) / BM;
    const bool r = use320 && rows320(g, cnt);
    if constexpr (R320) return r ? 1 : 0;
    else return r ? 0 : (cnt + BM - 1) / BM;
  };
  {
    int loc[PER];
    int run = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int gi = tid * PER + i;
      int mt = 0;
      if (gi < ngroups)
        mt = mtiles(MODE == 0 ? g.M : g.offsets[gi + 1] - g.offsets[gi]);
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
  uint32_t tdesc[kBigDescRegs];
#pragma unroll
  for (int j = 0; j < kBigDescRegs; ++j)
    tdesc[j] = (MODE == 0) ? 0u : find(tile_of(vid + (64 * j + lane) * G));
  __syncthreads();  // the prefix is dead before the first DMA into s_a0
  const int nK = g.K / KS / ksplit;  // per split; the host guarantees an even count
  const size_t row_bytes = (size_t)g.K * 2;

  // DMA lane geometry: lane fills slot (lane % 8) of row (lane / 8) of a KiB
  // and fetches the logical chunk that the swizzle of that tile row stores
  // in the slot (the swizzle is an involution in c for a fixed row).
  const int dma_row = lane / 8;
  const int dma_slot = lane % 8;

  for (int k = 0; vid + k * G < total; ++k) {
    // the host bounds the items per workgroup by 64 * kBigDescRegs (the
    // descriptor registers); never read past them
    MOE_CHECK(MODE == 0 || k < 64 * kBigDescRegs, MOE_CHECK_GEMM_ITEMS);
    if (MODE != 0 && k >= 64 * kBigDescRegs) break;
    const int tsplit = (MODE == 0) ? (vid + k * G) / tiles : 0;
    const int it = vid + k * G - tsplit * tiles;  // item (== tile unless sliced)
    const int t = tile_of(it);
    uint32_t dreg = tdesc[0];
#pragma unroll
    for (int j = 1; j < kBigDescRegs; ++j)
      if ((k >> 6) == j) dreg = tdesc[j];
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)dreg, k & 63);
    const int grp = (MODE == 0) ? 0 : (int)(d & 1023u);
    const int tp0 = (MODE == 0) ? 0 : (int)(d >> 10);
    const int cnt_g = (MODE == 0) ? g.M : g.offsets[grp + 1] - g.offsets[grp];
    const int mt_g = mtiles(cnt_g);
    const int local = t - tp0 * ntiles;
    // Within an expert, tiles go in groups of MG m-tiles x all n-tiles (n-tile
    // major inside a group), so the tiles that run together on one XCD share
    // both their token-row slices and their weight slices in L2.
    const int grp_m0 = (local / (MG * ntiles)) * MG;
    const int mg = max(1, min(MG, mt_g - grp_m0));
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
    // Down tiles walk their K range from a step rotated by (expert, n-tile):
    // the rows of W_down lie 4 KiB apart, and tiles that all read the same
    // K-step of their weight rows crowd the same HBM channels (prefill down
    // 4.02 -> 3.84 ms; gate/up, rows 12 KiB apart, gained nothing).  All
    // m-tiles of one (expert, n-tile) share the rotation, and so their weight
    // stages in L2; a tile's accumulation order depends only on its (expert,
    // n-tile), so results stay deterministic.
    const int rot = (MODE == 2) ? (int)(((long)grp * ntiles + nt) % nK) : 0;
    auto kofs = [&](int kstep) -> size_t {
      if constexpr (MODE == 2) {
        int kr = kstep + rot;
        if (kr >= nK) kr -= nK;
        return (size_t)kr * RB;
      } else {
        return (size_t)kstep * RB;
      }
    };
    MOE_CHECK(grp < ngroups && mi < mt_g && m0 < m_end && m_end <= cnt && n0 < g.N &&
                  m_end - m0 <= BM,
              MOE_CHECK_GEMM_TILE);
    // row blocks of this wave that hold rows: i with (i*WM + wm)*BLK < rows
    const int nrb = (m_end - m0 + BLK - 1) / BLK;
    const int mba = min(MB, (nrb - wm + WM - 1) / WM);

    // ---- per-lane DMA source offsets (32-bit; bases are wave-uniform, and
    // 64-bit), starting at this split's K range.  Gathered token rows can be
    // anywhere in x: their base is x (the host keeps x below 4 GiB).  Other
    // token rows (x_perm, H, the router's x) are contiguous: their base is
    // the tile's first row, so no offset exceeds 256 rows.
    const uint32_t k_base = (uint32_t)(tsplit * nK * RB);
    const bool gather = (MODE == 1 && g.perm != nullptr);
    const char* a_base = (const char*)g.a + (gather ? 0 : (size_t)(row0 + m0) * row_bytes);
    uint32_t a_off[A_PW];
#pragma unroll
    for (int q = 0; q < A_PW; ++q) {
      const int r = (wave + q * NW) * RPK + dma_row;  // tile row
      int rr = m0 + r;
      if (rr > m_end - 1) rr = m_end - 1;
      long src_row;
      if (gather) {
        src_row = g.perm[row0 + rr] / g.top_k;  // gather token rows on load
        MOE_CHECK(src_row >= 0 && src_row < g.M, MOE_CHECK_GEMM_ROW);
        if (src_row < 0 || src_row >= g.M) src_row = 0;
      } else {
        src_row = rr - m0;
      }
      a_off[q] = (uint32_t)(src_row * row_bytes) + k_base + swz(r, dma_slot) * 16;
    }
    const char* b_base0 = (const char*)g.b0 + (size_t)grp * g.N * row_bytes;
    const char* b_base1 =
        (MODE == 1) ? (const char*)g.b1 + (size_t)grp * g.N * row_bytes : b_base0;
    // gate rows fill the first half of a gate/up weight tile, up rows the
    // second; the 8 rows one DMA instruction fills lie in one half (with 256
    // rows the half is fixed per q, with 192 it depends on the wave)
    auto up_half = [&](int q) {
      return MODE == 1 && (HN % (NW * RPK) != 0 ? (wave + q * NW) * RPK >= HN
                                                 : (q * NW) * RPK >= HN);
    };
    uint32_t b_off[B_PW];
#pragma unroll
    for (int q = 0; q < B_PW; ++q) {
      const int r = (wave + q * NW) * RPK + dma_row;
      int n = up_half(q) ? n0 + r - HN : n0 + r;
      if (n > g.N - 1) n = g.N - 1;
      b_off[q] = (uint32_t)(n * row_bytes) + k_base + swz(r, dma_slot) * 16;
    }

    acc_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = acc_t{};

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
      const size_t off = kofs(ks);
#pragma unroll
      for (int q = 0; q < A_PW; ++q)
        __builtin_amdgcn_global_load_lds((glb_void_t*)(a_base + a_off[q] + off),
                                         (lds_void_t*)(sa + (wave + q * NW) * 1024), 16, 0, 0);
    };
    // ntc: whether the weight loads are non-temporal (an expert's weight
    // slice read by one m-tile only)
    auto issue_b = [&](auto sc, int ks, auto ntc) {
      constexpr int CP = decltype(ntc)::value ? kCpolNT : 0;
      char* sb = stage_b(sc);
      const size_t off = kofs(ks);
#pragma unroll
      for (int q = 0; q < B_PW; ++q) {
        const char* bb = up_half(q) ? b_base1 : b_base0;
        __builtin_amdgcn_global_load_lds((glb_void_t*)(bb + b_off[q] + off),
                                         (lds_void_t*)(sb + (wave + q * NW) * 1024), 16, 0, CP);
      }
    };

    auto brow = [&](int j) {
      if (MODE == 1)
        return (j < NB / 2) ? wn * (WTN / 2) + j * BLK + rin
                            : HN + wn * (WTN / 2) + (j - NB / 2) * BLK + rin;
      return wn * WTN + j * BLK + rin;
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
    auto kstep = [&](auto mbac, auto ntc, auto asc, auto bsc, auto nac, auto nbc, int ks) {
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
        if (next_b) issue_b(std::integral_constant<int, (BS + 2) % 3>{}, ks + 2, ntc);
      }
      // favour this wave's MFMA issue over the other wave on the SIMD
      __builtin_amdgcn_s_setprio(1);
      // DMA load L of a main-loop step: token rows of step ks+1 for
      // L < A_PW, then weights of step ks+2; slice kk issues loads
      // kk*DPS .. kk*DPS + DPS-1, so token rows always go first
      auto dma_one = [&](int L) {
        if (L < A_PW) {
          char* sa2 = stage_a(std::integral_constant<int, (AS + 1) % 2>{});
          const size_t off = kofs(B16 ? min(ks + 1, nK - 1) : ks + 1);
          __builtin_amdgcn_global_load_lds((glb_void_t*)(a_base + a_off[L] + off),
                                           (lds_void_t*)(sa2 + (wave + L * NW) * 1024), 16, 0, 0);
        } else {
          const int q = L - A_PW;
          char* sb2 = stage_b(std::integral_constant<int, (BS + 2) % 3>{});
          const size_t off = kofs(B16 ? min(ks + 2, nK - 1) : ks + 2);
          const char* bb = up_half(q) ? b_base1 : b_base0;
          constexpr int CP = decltype(ntc)::value ? kCpolNT : 0;
          __builtin_amdgcn_global_load_lds((glb_void_t*)(bb + b_off[q] + off),
                                           (lds_void_t*)(sb2 + (wave + q * NW) * 1024), 16, 0, CP);
        }
      };
      auto dma_piece = [&](int kk) {
#pragma unroll
        for (int L = kk * DPS; L < kk * DPS + DPS; ++L) dma_one(L);
      };
      auto frag = [&](const char* base, int r, int c) {
        return *reinterpret_cast<const u32x4_t*>(&base[r * RB + (swz(r, c) << 4)]);
      };
      if constexpr (B16) {
        // Two K-slices of 32 per stage, MFMAs token-row block by block
        // (i-major), a scheduling fence closing every block's group, the
        // slice's DMA loads spread over the groups.
        // Shape 1: slice 0's fragments are read after the barrier, slice 1's
        // under slice 0's MFMAs: each token-row fragment once slice 0's last
        // MFMA on that block has issued, the weight fragments one by one in
        // the last block, so each can take the registers of the fragment it
        // replaces (120 accumulators leave no room for a second set).
        // Shape 2 (128 accumulators, 12 fragments per slice): each slice
        // reads its fragments, then runs its MFMAs.
        if constexpr (SHAPE == 1) {
        u32x4_t a0[MBA], a1[MBA], w0[NB], w1[NB];
#pragma unroll
        for (int i = 0; i < MBA; ++i) a0[i] = frag(sa, (i * WM + wm) * BLK + rin, kg);
#pragma unroll
        for (int j = 0; j < NB; ++j) w0[j] = frag(sb, brow(j), kg);
        __builtin_amdgcn_sched_group_barrier(0x100, MBA + NB, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
          for (int i = 0; i < MBA; ++i) {
            const int d_lo = (i * DPS + MBA - 1) / MBA, d_hi = ((i + 1) * DPS + MBA - 1) / MBA;
            if constexpr (SPREAD) {
#pragma unroll
              for (int d = d_lo; d < d_hi; ++d) dma_one(kk * DPS + d);
            }
            const bool last = kk == 0 && i == MBA - 1;
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, kk == 0 ? w0[j] : w1[j]),
                  __builtin_bit_cast(bf16x8_t, kk == 0 ? a0[i] : a1[i]), acc[i][j], 0, 0, 0);
              if (last) w1[j] = frag(sb, brow(j), 4 + kg);
            }
            if (kk == 0) a1[i] = frag(sa, (i * WM + wm) * BLK + rin, 4 + kg);
            if constexpr (SPREAD) {
#pragma unroll
              for (int d = d_lo; d < d_hi; ++d) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
            if (last) {
#pragma unroll
              for (int j = 0; j < NB; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
              }
            } else {
              __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
            }
            if (kk == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        } else {
        u32x4_t a0[MBA], w0[NB];
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
          for (int i = 0; i < MBA; ++i) a0[i] = frag(sa, (i * WM + wm) * BLK + rin, 4 * kk + kg);
#pragma unroll
          for (int j = 0; j < NB; ++j) w0[j] = frag(sb, brow(j), 4 * kk + kg);
          __builtin_amdgcn_sched_group_barrier(0x100, MBA + NB, 0);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < MBA; ++i) {
            const int d_lo = (i * DPS + MBA - 1) / MBA, d_hi = ((i + 1) * DPS + MBA - 1) / MBA;
            if constexpr (SPREAD) {
#pragma unroll
              for (int d = d_lo; d < d_hi; ++d) dma_one(kk * DPS + d);
            }
#pragma unroll
            for (int j = 0; j < NB; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8_t, w0[j]), __builtin_bit_cast(bf16x8_t, a0[i]),
                  acc[i][j], 0, 0, 0);
            if constexpr (SPREAD) {
#pragma unroll
              for (int d = d_lo; d < d_hi; ++d) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, NB, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        }
      } else {
      u32x4_t af[2][MBA], bfr[2][NB];
      auto load = [&](int set, int kk) {
        const int c = kk * 2 + kg;
#pragma unroll
        for (int i = 0; i < MBA; ++i) af[set][i] = frag(sa, (i * WM + wm) * BLK + rin, c);
#pragma unroll
        for (int j = 0; j < NB; ++j) bfr[set][j] = frag(sb, brow(j), c);
      };
      static_assert(B16 || !SPREAD || (A_PW == 4 && B_PW == 4 && NKK == 4), "two DMA loads per slice");
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
    auto kloop = [&](auto mbac, auto ntc) {
      // previous tile's epilogue stores and LDS reads must be done before the
      // stages are refilled and before vmcnt counts only this tile's DMA
      wait_vmcnt<0>();
      wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      issue_a(I0{}, 0);
      issue_b(I0{}, 0, ntc);
      issue_b(I1{}, 1, ntc);  // nK >= 2
      int ks = 0;
      // 320-row tiles run every step here, the last ones refilling stages
      // that are never read (the refill K-step is clamped to the last one)
      for (; ks + (B16 ? 6 : 8) <= nK; ks += 6) {
        kstep(mbac, ntc, I0{}, I0{}, T{}, T{}, ks);
        kstep(mbac, ntc, I1{}, I1{}, T{}, T{}, ks + 1);
        kstep(mbac, ntc, I0{}, I2{}, T{}, T{}, ks + 2);
        kstep(mbac, ntc, I1{}, I0{}, T{}, T{}, ks + 3);
        kstep(mbac, ntc, I0{}, I1{}, T{}, T{}, ks + 4);
        kstep(mbac, ntc, I1{}, I2{}, T{}, T{}, ks + 5);
      }
      if constexpr (B16) {
        // nK is even: 0, 2 or 4 steps remain
        if (ks + 2 <= nK) {
          kstep(mbac, ntc, I0{}, I0{}, T{}, T{}, ks);
          kstep(mbac, ntc, I1{}, I1{}, T{}, T{}, ks + 1);
        }
        if (ks + 4 <= nK) {
          kstep(mbac, ntc, I0{}, I2{}, T{}, T{}, ks + 2);
          kstep(mbac, ntc, I1{}, I0{}, T{}, T{}, ks + 3);
        }
      }
      return ks;
    };
    // a wave with no rows (mba == 0) still loads and waits with the others;
    // its one block of clamped rows is never stored
    auto run = [&](auto ntc) {
      int ks;
      if (MB >= 5 && mba >= 5) ks = kloop(std::integral_constant<int, MB >= 5 ? 5 : 4>{}, ntc);
      else if (mba >= 4) ks = kloop(std::integral_constant<int, 4>{}, ntc);
      else if (mba == 3) ks = kloop(std::integral_constant<int, 3>{}, ntc);
      else if (mba == 2) ks = kloop(std::integral_constant<int, 2>{}, ntc);
      else ks = kloop(std::integral_constant<int, 1>{}, ntc);
      // The last 2, 4 or 6 steps run every block (one copy of the code;
      // blocks without rows are never stored) with refills decided at run
      // time.
      if constexpr (!B16) {
        using M4 = std::integral_constant<int, MB>;
        kstep(M4{}, ntc, I0{}, I0{}, ks + 1 < nK, ks + 2 < nK, ks);
        kstep(M4{}, ntc, I1{}, I1{}, ks + 2 < nK, ks + 3 < nK, ks + 1);
        if (ks + 4 <= nK) {
          kstep(M4{}, ntc, I0{}, I2{}, ks + 3 < nK, ks + 4 < nK, ks + 2);
          kstep(M4{}, ntc, I1{}, I0{}, ks + 4 < nK, ks + 5 < nK, ks + 3);
        }
        if (ks + 6 <= nK) {
          kstep(M4{}, ntc, I0{}, I1{}, ks + 5 < nK, ks + 6 < nK, ks + 4);
          kstep(M4{}, ntc, I1{}, I2{}, false, false, ks + 5);
        }
      }
    };
    // Gate/up weight loads are non-temporal when the expert has one m-tile:
    // no other tile reads its weight slice, which then need not displace
    // cached token rows (prefill step 11.00 -> 10.87 ms, gate/up 6.76 ->
    // 6.65 ms; non-temporal loads for every tile had made the small and
    // skewed batches, whose experts' m-tiles share the slice, 1-3% slower;
    // for down they gained nothing)
    using NT0 = std::false_type;
    using NT1 = std::true_type;
    if constexpr (MODE == 1 && SHAPE == 1) run(NT1{});
    else if constexpr (MODE == 1) {
      if (mt_g == 1) run(NT1{});
      else run(NT0{});
    } else {
      run(NT0{});
    }

    // ---- epilogue.  Weights were the MFMA row operand, so block (i, j) is
    // C^T.  32x32 blocks: lane (r32, kg) holds, for quad q = v / 4, the 4
    // consecutive output columns 8q + 4kg + {0..3} of token row r32.  16x16
    // blocks: lane (r16, kg) holds columns 4kg + {0..3} of token row r16.
    // Either way one packed 8-byte store per 4 columns.  Blocks past the
    // wave's active ones hold rows >= m_end and are skipped.
    auto bf16x4 = [](float v0, float v1, float v2, float v3) {
      const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v0) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v1) << 16);
      const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v2) |
                          ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v3) << 16);
      return make_uint2(lo, hi);
    };
    // silu(z) = z * sigmoid(z) with hardware exp2 / reciprocal (H is
    // rounded to bf16 right after)
    auto swiglu = [](float z, float u) {
      const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * 1.44269504f));
      return z * sg * u;
    };
    if constexpr (B16) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int r = m0 + (i * WM + wm) * BLK + rin;
        if (r < m_end) {
          char* crow = (char*)g.c + (size_t)(row0 + r) * g.N * 2;
          if (MODE == 1) {
#pragma unroll
          for (int j = 0; j < NB / 2; ++j) {
            const int col = n0 + wn * (WTN / 2) + j * BLK + 4 * kg;
            const acc_t& z = acc[i][j];
            const acc_t& u = acc[i][j + NB / 2];
            if (col + 3 < g.N)
              *reinterpret_cast<uint2*>(crow + col * 2) =
                  bf16x4(swiglu(z[0], u[0]), swiglu(z[1], u[1]), swiglu(z[2], u[2]),
                         swiglu(z[3], u[3]));
          }
          } else {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const int col = n0 + wn * WTN + j * BLK + 4 * kg;
              const acc_t& v = acc[i][j];
              if (col + 3 < g.N)
                *reinterpret_cast<uint2*>(crow + col * 2) = bf16x4(v[0], v[1], v[2], v[3]);
            }
          }
        }
      }
    } else {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int r = m0 + (i * WM + wm) * 32 + rin;
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
              for (int e = 0; e < 4; ++e) hv[e] = swiglu(acc[i][j][4 * q + e], acc[i][j + NB / 2][4 * q + e]);
              if (col + 3 < g.N)
                *reinterpret_cast<uint2*>(crow + col * 2) = bf16x4(hv[0], hv[1], hv[2], hv[3]);
            }
          } else {
#pragma unroll
            for (int j = 0; j < NB; ++j) {
              const int col = n0 + wn * WTN + j * 32 + 8 * q + 4 * kg;
              if (col + 3 < g.N)
                *reinterpret_cast<uint2*>(crow + col * 2) =
                    bf16x4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                           acc[i][j][4 * q + 3]);
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


MOE_CHECK_ACCESSOR(check_word_gemm_big)

int big_grid(hipStream_t st) {
  int grid = st == nullptr ? device_cu_count() : stream_cu_count(st);  // one workgroup per CU
  grid -= grid % 8;                                                    // (LDS bound)
  return grid < 8 ? 8 : grid;
}

template <int MODE, int SHAPE>
static int launch_big_mode(const GemmArgs& g, hipStream_t st) {
  auto kern = grouped_gemm_big_kernel<MODE, MOE_BIG_MG, SHAPE>;
  if (device_cu_count() <= 0) return MOE_EHIP;
  // expert modes: grid_mult waves of one workgroup per CU (plan::big_grid_mult)
  const int mult = (MODE != 0 && g.grid_mult > 1) ? g.grid_mult : 1;
  hipLaunchKernelGGL(kern, dim3(big_grid(st) * mult), dim3(512), 0, st, g);
  return check_launch();
}

// Expert modes: the groups of r320_lo..r320_hi rows on 320 x 192 tiles, the
// others on 256 x 256 tiles (two launches on the same stream; they write
// disjoint rows).  Down's 256 x 256 tiles always run on 16x16x32 MFMAs;
// gate/up's do when d_model (its K) is at least kGateUp16MinK: then the
// whole layer step was faster (prefill 10.73-10.85 -> 10.63 ms, skewed
// 1.69 -> 1.65 ms: gate/up about even, the down GEMM after it 2-4% faster),
// with d_model 2048 slower (small 0.41 -> 0.42 ms).
template <int MODE>
static int launch_big_expert(const GemmArgs& g, hipStream_t st) {
  if (g.r320_hi > 0) {
    const int rc = launch_big_mode<MODE, 1>(g, st);
    if (rc != MOE_OK) return rc;
  }
  if (MODE == 2 || g.K >= kGateUp16MinK) return launch_big_mode<MODE, 2>(g, st);
  return launch_big_mode<MODE, 0>(g, st);
}

int launch_gemm_big(int mode, const GemmArgs& g, hipStream_t st) {
  if (g.K % 128 != 0 || g.ngroups < 1 || g.ngroups > kBigMaxGroups) return MOE_EINVAL;
  if (mode == 0) {
    // each split covers an even number (>= 2) of 64-wide K-steps
    if (g.ngroups != 1 || g.ksplit < 1 || (g.K / 64) % (2 * g.ksplit) != 0) return MOE_EINVAL;
    return launch_big_mode<0, 0>(g, st);
  }
  if (g.r320_hi > 0 && (g.r320_lo < 1 || g.r320_hi > 320)) return MOE_EINVAL;
  if (g.grid_mult < 0 || g.grid_mult > plan::kBigMaxGridMult) return MOE_EINVAL;
  return mode == 1 ? launch_big_expert<1>(g, st) : launch_big_expert<2>(g, st);
}

}  // namespace moe
