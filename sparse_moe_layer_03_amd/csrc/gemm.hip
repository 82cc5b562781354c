// Grouped GEMM on gfx950 MFMA for the MoE layer: the router classifier, the
// experts' gate/up projections with a fused SwiGLU epilogue, and the experts'
// down projections.
//
// Every operand has its reduction dimension contiguous (x rows, H rows and
// the out-major weights), so a 16-byte chunk of one row is exactly the
// 8 bf16 (or 4 fp32) values one lane feeds to a 16x16 MFMA.  Tiles of A
// (token rows) and B (weight rows) are staged in LDS as 128-byte rows per
// K-step, with the chunk index XOR-swizzled by (row & 7) so that both the
// row-wise global->LDS stores and the fragment reads are bank-conflict free.
// Two LDS stages and two register sets: while one stage feeds the MFMAs,
// the next K-step waits in the other stage and the global loads of the one
// after it are in flight into registers.
//
// Work is a persistent loop over (group, n-tile, m-tile) tiles.  Each
// workgroup derives the tile list itself from the group offsets, so no host
// synchronisation is needed to learn how many rows each expert received.
// Workgroup ids are remapped so that consecutive tiles land on the same XCD
// (dispatch is round-robin over the 8 XCDs), which keeps an expert's weight
// tile and its token rows in that XCD's L2 while its m-tiles run.

#include "common.h"
#include "internal.h"

namespace moe {

enum { MODE_ROUTER = 0, MODE_GATE_UP = 1, MODE_DOWN = 2 };

constexpr int kMaxGroups = 1024;

__device__ __forceinline__ float silu_f(float z) { return z / (1.0f + expf(-z)); }

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
  // one 16-byte chunk per lane = the whole K=32 slice of a 16x16x32 MFMA
  static __device__ __forceinline__ f32x4_t step(u32x4_t a, u32x4_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  // a 16-byte chunk holds 4 K values: four 16x16x4 fp32 MFMAs
  static __device__ __forceinline__ f32x4_t step(u32x4_t a, u32x4_t b, f32x4_t c) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[s]), __uint_as_float(b[s]), c, 0, 0, 0);
    return c;
  }
};

template <typename T, int MODE, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_kernel(GemmArgs g) {
  constexpr int NT = 64 * WM * WN;
  constexpr int CE = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int BK = 8 * CE;                // elements per K-step (128 bytes)
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int MB = WTM / 16, NB = WTN / 16;
  constexpr int HN = (MODE == MODE_GATE_UP) ? BN / 2 : BN;  // output cols per tile
  static_assert(MB >= 1 && NB >= 1, "wave tile too small");
  static_assert(MODE != MODE_GATE_UP || NB % 2 == 0, "gate/up pairing");
  constexpr int A_CH = BM * 8, B_CH = BN * 8;
  constexpr int A_IT = (A_CH + NT - 1) / NT, B_IT = (B_CH + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) char s_a[2][BM * 128];
  __shared__ __attribute__((aligned(16))) char s_b[2][BN * 128];
  // chunks that threads past a tile's chunk count load but never use land
  // here, so every thread stores unconditionally (no branch around the
  // stores, which would make the compiler drain the loads in flight)
  constexpr bool A_SPARE = A_IT * NT > A_CH, B_SPARE = B_IT * NT > B_CH;
  __shared__ __attribute__((aligned(16))) char s_junk[(A_SPARE || B_SPARE) ? NT * 16 : 16];
  __shared__ int s_mt[kMaxGroups + 1];
  __shared__ int s_tmp[NT / 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int r16 = lane & 15, kg = lane >> 4;

  // ---- tile list: per-group m-tile prefix sums in LDS
  const int ngroups = (MODE == MODE_ROUTER) ? 1 : g.ngroups;
  {
    constexpr int PER = (kMaxGroups + NT - 1) / NT;
    int loc[PER];
    int run = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int gi = tid * PER + i;
      int mt = 0;
      if (gi < ngroups) {
        const int cnt = (MODE == MODE_ROUTER) ? g.M : (g.offsets[gi + 1] - g.offsets[gi]);
        mt = (cnt + BM - 1) / BM;
      }
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
  const int ksplit = (MODE == MODE_ROUTER) ? g.ksplit : 1;
  const long total = (long)s_mt[ngroups] * ntiles * ksplit;
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int vid = (G % 8 == 0) ? (b % 8) * (G / 8) + b / 8 : b;
  const int nK = g.K / BK / ksplit;  // K-steps per split (the host divides evenly)
  const size_t a_row_bytes = (size_t)g.K * sizeof(T);

  // LDS slots of this thread's chunks (the same in every tile)
  int a_lds[A_IT], b_lds[B_IT];
#pragma unroll
  for (int it = 0; it < A_IT; ++it) {
    const int q = tid + it * NT, r = q >> 3, c = q & 7;
    a_lds[it] = r * 128 + ((c ^ (r & 7)) << 4);
  }
#pragma unroll
  for (int it = 0; it < B_IT; ++it) {
    const int q = tid + it * NT, r = q >> 3, c = q & 7;
    b_lds[it] = r * 128 + ((c ^ (r & 7)) << 4);
  }

  // Few-row expert tiles stream their weights once; each walks its K range
  // starting at a K-step rotated by (expert, n-tile), so the tiles running
  // at one time read different columns of their weight rows.  Rows of the
  // down projection lie 4 KiB apart, and tiles all starting at K-step 0
  // crowd the same HBM channels (decode down 1.74 -> 1.67 ms; gate/up, rows
  // 12 KiB apart, unchanged).  All m-tiles of one (expert, n-tile) share the
  // rotation and so their weight slices in L2.  The accumulation order of a
  // tile depends only on its (expert, n-tile): results stay deterministic.
  constexpr bool K_ROTATE = MODE != MODE_ROUTER && BM <= 32;
  // A tile: its place in the output and this thread's source chunks (at the
  // start of its K range)
  struct Tile {
    int split, row0, rows, m0, n0, rot;
    const char* a[A_IT];
    const char* b[B_IT];
  };
  auto setup = [&](long tt, Tile& tl) {
    const int split = (int)(tt % ksplit);
    const long t = tt / ksplit;
    const size_t k_off = (size_t)split * nK * 128;  // byte offset of this split's K range
    // locate group: last gi with s_mt[gi] * ntiles <= t
    int lo = 0, hi = ngroups - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((long)s_mt[mid] * ntiles <= t) lo = mid; else hi = mid - 1;
    }
    const int grp = lo;
    const int mt_g = s_mt[grp + 1] - s_mt[grp];
    const long local = t - (long)s_mt[grp] * ntiles;
    // groups of 4 m-tiles x all n-tiles, n-tile major inside a group, so
    // tiles running together on one XCD share rows and weights in L2
    constexpr int MG = 4;
    const int grp_m0 = (int)(local / ((long)MG * ntiles)) * MG;
    const int mg = min(MG, mt_g - grp_m0);
    const int in_grp = (int)(local - (long)grp_m0 * ntiles);
    const int nt = in_grp / mg, mi = grp_m0 + in_grp % mg;
    const int row0 = (MODE == MODE_ROUTER) ? 0 : g.offsets[grp];
    const int rows = (MODE == MODE_ROUTER) ? g.M : (g.offsets[grp + 1] - row0);
    const int m0 = mi * BM;
    const int n0 = nt * HN;
    MOE_CHECK(grp < ngroups && mi < mt_g && m0 < rows && n0 < g.N, MOE_CHECK_GEMM_TILE);
    tl.split = split;
    tl.rot = K_ROTATE ? (int)(((long)grp * ntiles + nt) % nK) : 0;
    tl.row0 = row0;
    tl.rows = rows;
    tl.m0 = m0;
    tl.n0 = n0;
#pragma unroll
    for (int it = 0; it < A_IT; ++it) {
      const int q = tid + it * NT;
      const int r = q >> 3, c = q & 7;
      int rr = m0 + r;
      if (rr > rows - 1) rr = rows - 1;  // ragged tail: reload a valid row
      long src_row;
      if (q >= A_CH)
        src_row = 0;  // a thread past the tile loads row 0 (valid in every mode), never stored
      else if (MODE == MODE_GATE_UP && g.perm != nullptr)
      {
        src_row = g.perm[row0 + rr] / g.top_k;  // gather token rows on load
        MOE_CHECK(src_row >= 0 && src_row < g.M, MOE_CHECK_GEMM_ROW);
        if (src_row < 0 || src_row >= g.M) src_row = 0;
      }
      else
        src_row = row0 + rr;
      tl.a[it] = (const char*)g.a + src_row * a_row_bytes + k_off + c * 16;
    }
#pragma unroll
    for (int it = 0; it < B_IT; ++it) {
      const int q = tid + it * NT;
      const int r = q >> 3, c = q & 7;
      const char* base;
      int n;
      if (MODE == MODE_GATE_UP) {
        const bool up = r >= HN;
        n = n0 + (up ? r - HN : r);
        if (n > g.N - 1) n = g.N - 1;
        base = (const char*)(up ? g.b1 : g.b0) + (size_t)grp * g.N * a_row_bytes;
      } else {
        n = n0 + r;
        if (n > g.N - 1) n = g.N - 1;
        base = (const char*)g.b0 + (MODE == MODE_DOWN ? (size_t)grp * g.N * a_row_bytes : 0);
      }
      tl.b[it] = base + (size_t)n * a_row_bytes + k_off + c * 16;  // q >= B_CH: loaded, not stored
    }
  };

  // The last two K-steps of a tile load the first two of the workgroup's
  // next tile (nK even), so its loads, its group lookup and its gather
  // indices are in flight under this tile's MFMAs and epilogue; without a
  // next tile they repeat the last step.
  const bool chain = nK % 2 == 0;
  Tile cur, nxt;
  bool pre = false;  // cur was set up by the previous tile, which also loaded
                     // its step 0 into LDS stage 0 and step 1 into register set 1

  // Expert weights in the few-rows-per-expert tiles are read by one row
  // tile each and never again in the step: they are loaded non-temporal
  // (decode gate/up 3.65 -> 3.32 ms, down 1.88 -> 1.80).  The router matrix
  // is re-read by every row tile and stays cached.
  constexpr bool B_STREAM = MODE != MODE_ROUTER && BM <= 32;
  u32x4_t ra0[A_IT], rb0[B_IT], ra1[A_IT], rb1[B_IT];

  for (long tt = vid; tt < total; tt += G) {
    if (!pre) setup(tt, cur);
    const bool more = chain && tt + G < total;
    if (more) setup(tt + G, nxt);
    else nxt = cur;

    f32x4_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Two register sets carry the global loads of the next two K-steps, so a
    // load has two K-steps of MFMA work to arrive before it is written to LDS.
    // Every thread loads every step (steps past the end come from the next
    // tile or repeat the last one, threads past the tile's chunks repeat a
    // valid chunk): a load under a condition makes the compiler drain all
    // loads in flight at that point.
    auto gload = [&](u32x4_t* ra, u32x4_t* rb, int ks) {
      const bool past = ks >= nK;
      const int kl = past ? (more ? ks - nK : nK - 1) : ks;  // K-step of the tile
      const int rot = past ? nxt.rot : cur.rot;
      const int kr = kl + rot >= nK ? kl + rot - nK : kl + rot;
      const size_t off = (size_t)kr * 128;
#pragma unroll
      for (int it = 0; it < A_IT; ++it) ra[it] = ld16((past ? nxt.a[it] : cur.a[it]) + off);
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const char* p = (past ? nxt.b[it] : cur.b[it]) + off;
        rb[it] = B_STREAM ? __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p))
                          : ld16(p);
      }
    };
    auto lstore = [&](const u32x4_t* ra, const u32x4_t* rb, int buf) {
#pragma unroll
      for (int it = 0; it < A_IT; ++it) {
        char* dst = (!A_SPARE || tid + it * NT < A_CH) ? &s_a[buf][a_lds[it]] : &s_junk[tid * 16];
        *reinterpret_cast<u32x4_t*>(dst) = ra[it];
      }
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        char* dst = (!B_SPARE || tid + it * NT < B_CH) ? &s_b[buf][b_lds[it]] : &s_junk[tid * 16];
        *reinterpret_cast<u32x4_t*>(dst) = rb[it];
      }
    };
    auto compute = [&](int buf) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int c = kk * 4 + kg;
        u32x4_t af[MB], bfr[NB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const int r = wm * WTM + i * 16 + r16;
          af[i] = *reinterpret_cast<const u32x4_t*>(&s_a[buf][r * 128 + ((c ^ (r & 7)) << 4)]);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          int r;
          if (MODE == MODE_GATE_UP)
            r = (j < NB / 2) ? wn * (WTN / 2) + j * 16 + r16
                             : HN + wn * (WTN / 2) + (j - NB / 2) * 16 + r16;
          else
            r = wn * WTN + j * 16 + r16;
          bfr[j] = *reinterpret_cast<const u32x4_t*>(&s_b[buf][r * 128 + ((c ^ (r & 7)) << 4)]);
        }
#pragma unroll
        for (int i = 0; i < MB; ++i)
#pragma unroll
          for (int j = 0; j < NB; ++j) acc[i][j] = Mfma<T>::step(af[i], bfr[j], acc[i][j]);
      }
    };

    if (!pre) {
      gload(ra0, rb0, 0);
      gload(ra1, rb1, 1);
      lstore(ra0, rb0, 0);
      __syncthreads();
    }
    for (int ks = 0; ks < nK; ks += 2) {
      // LDS stage 0 holds step ks; registers set 1 hold step ks+1 (in flight)
      gload(ra0, rb0, ks + 2);
      compute(0);
      lstore(ra1, rb1, 1);  // past the end: a repeated step, never computed
      __syncthreads();
      if (ks + 1 >= nK) break;
      // LDS stage 1 holds step ks+1; registers set 0 hold step ks+2
      gload(ra1, rb1, ks + 3);
      compute(1);
      lstore(ra0, rb0, 0);  // past the end: the next tile's step 0
      __syncthreads();
    }

    // ---- epilogue: lane holds C[4*kg + v][r16] of each 16x16 block
    const int m0 = cur.m0, n0 = cur.n0, rows = cur.rows, row0 = cur.row0, split = cur.split;
    (void)split;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = m0 + wm * WTM + i * 16 + 4 * kg + v;
        if (r >= rows) continue;
        if (MODE == MODE_GATE_UP) {
#pragma unroll
          for (int j = 0; j < NB / 2; ++j) {
            const int col = n0 + wn * (WTN / 2) + j * 16 + r16;
            if (col < g.N) {
              const float h = silu_f(acc[i][j][v]) * acc[i][j + NB / 2][v];
              ((T*)g.c)[(size_t)(row0 + r) * g.N + col] = ElemOps<T>::from_f(h);
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            const int col = n0 + wn * WTN + j * 16 + r16;
            if (col < g.N) {
              if (MODE == MODE_ROUTER)  // partial sum of this K split
                ((float*)g.c)[((size_t)split * g.M + r) * g.N + col] = acc[i][j][v];
              else
                ((T*)g.c)[(size_t)(row0 + r) * g.N + col] = ElemOps<T>::from_f(acc[i][j][v]);
            }
          }
        }
      }
    }
    cur = nxt;
    pre = more;
  }
}

// ---------------------------------------------------------------- launch --

MOE_CHECK_ACCESSOR(check_word_gemm)

template <typename T, int MODE, int BM, int BN, int WM, int WN>
static int launch_cfg(const GemmArgs& g, hipStream_t st) {
  auto kern = grouped_gemm_kernel<T, MODE, BM, BN, WM, WN>;
  constexpr int NT = 64 * WM * WN;
  // occupancy of this instantiation, queried once (thread-safe static
  // initialisation; every device this library runs on is a gfx950)
  static const int per_cu = [kern] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, NT, 0) != hipSuccess || n < 1) n = 1;
    return n;
  }();
  const int cus = stream_cu_count(st);
  if (cus <= 0) return MOE_EHIP;
  int grid = cus * per_cu;
  grid -= grid % 8;
  if (grid < 8) grid = 8;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, g);
  return check_launch();
}

// Tile shapes (rows x weight-rows, waves along M x N).  Overridable at build
// time for tuning sweeps.
#ifndef MOE_BIG_TILE
#define MOE_BIG_TILE 128, 128, 2, 2
#endif
#ifndef MOE_SMALL_TILE
#define MOE_SMALL_TILE 16, 128, 1, 4
#endif
// Gate/up streams 256 weight rows (128 gate + 128 up) per few-row tile: half
// the tiles, each token-row chunk loaded once per 256 weight rows; two
// workgroups per CU.  Decode gate/up 3.34-3.37 -> 3.21 ms (whole step 5.13-5.17
// -> 4.99-5.00 ms); down and the router are no faster with it.
#ifndef MOE_SMALL_TILE_GATE_UP
#define MOE_SMALL_TILE_GATE_UP 16, 256, 1, 4
#endif
#ifndef MOE_SMALL_TILE_DOWN
#define MOE_SMALL_TILE_DOWN MOE_SMALL_TILE
#endif

template <typename T>
static int launch_typed(int mode, int big, const GemmArgs& g, hipStream_t st) {
  if (big) {
    switch (mode) {
      case MODE_ROUTER: return launch_cfg<T, MODE_ROUTER, MOE_BIG_TILE>(g, st);
      case MODE_GATE_UP: return launch_cfg<T, MODE_GATE_UP, MOE_BIG_TILE>(g, st);
      default: return launch_cfg<T, MODE_DOWN, MOE_BIG_TILE>(g, st);
    }
  }
  switch (mode) {
    case MODE_ROUTER: return launch_cfg<T, MODE_ROUTER, MOE_SMALL_TILE>(g, st);
    case MODE_GATE_UP: return launch_cfg<T, MODE_GATE_UP, MOE_SMALL_TILE_GATE_UP>(g, st);
    default: return launch_cfg<T, MODE_DOWN, MOE_SMALL_TILE_DOWN>(g, st);
  }
}

int launch_gemm(int dtype, int mode, int big, const GemmArgs& g, hipStream_t st) {
  if (dtype == MOE_BF16) return launch_typed<__bf16>(mode, big, g, st);
  return launch_typed<float>(mode, big, g, st);
}

}  // namespace moe
