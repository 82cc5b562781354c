// Router softmax, biased top-k and gates; and, for at most 128 experts in
// bf16, the router GEMM fused with them (router_topk_kernel).
//
// LongCat-2.0 data sheet (archdb), table "Mixture of experts": the router
// scores FFN and identity experts together and selects the top k by score
// plus e_score_correction_bias; the gates are the unbiased scores times the
// routed scaling factor, not renormalised.
//
// Selection runs in one wave64 per token, or per few tokens at once: each
// lane holds experts lane, lane+64, ... in registers (E <= 1024 -> at most 16
// per lane).  The softmax max and sum are butterfly reductions over the wave
// in a fixed order, so the result is deterministic.  The top k are found by
// a radix select on the fp32 keys mapped to order-preserving integers: the
// k-th largest key is built bit by bit with ballot counts, then every key
// above it and the keys equal to it in ascending expert id are taken (larger
// key wins, equal keys go to the lower expert id).  The chosen set is
// emitted in ascending expert id with a ballot per register slot.

#include <math.h>

#include "common.h"
#include "internal.h"

namespace moe {

// Softmax, biased top-k and gates of NT tokens held by one wave (lane holds
// experts lane + 64 i of each; m[n] is the lane's partial max of token n;
// bias must be readable at [0, 64 PL), e.g. a copy in LDS padded past E);
// writes token t[n]'s k slots of idx / gate in ascending expert id, for the
// tokens with t[n] >= 0.  The NT tokens' reductions are independent chains
// interleaved step by step, so their shuffle latencies overlap.
template <int PL, int NT>
__device__ __forceinline__ void select_topk(float (&l)[NT][PL], float (&m)[NT],
                                            const float* __restrict__ bias, int E, int k,
                                            float scaling, const int (&t)[NT],
                                            int32_t* __restrict__ idx, float* __restrict__ gate) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
#pragma unroll
    for (int n = 0; n < NT; ++n) m[n] = fmaxf(m[n], __shfl_xor(m[n], o, kWave));
  float s[NT], p[NT][PL];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    s[n] = 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + 64 * i;
      p[n][i] = (e < E) ? expf(l[n][i] - m[n]) : 0.f;
      s[n] += p[n][i];
    }
  }
  // same butterfly order as wave_sum
#pragma unroll
  for (int o = 32; o > 0; o >>= 1)
#pragma unroll
    for (int n = 0; n < NT; ++n) s[n] += __shfl_xor(s[n], o, kWave);
  // Selection key p + bias in fp32, mapped to an unsigned integer with the
  // same order (NaN ranks as -inf, -0 as +0); experts past E map to 0,
  // below every real key.
  uint32_t u[NT][PL];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + 64 * i;
      p[n][i] = p[n][i] / s[n];
      const float bv = bias[lane + 64 * i];  // readable for every slot
      if (e < E) {
        float key = p[n][i] + bv;
        if (key != key) key = -INFINITY;
        key += 0.0f;  // -0 -> +0
        const uint32_t b = __float_as_uint(key);
        u[n][i] = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
      } else {
        u[n][i] = 0u;
      }
    }
  // The k-th largest mapped key, found bit by bit from the top: keep bit b
  // if at least k keys are >= the threshold with it set.  Counts are wave
  // ballots, so no lane exchanges data.
  uint32_t thr[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) thr[n] = 0u;
  for (int b = 31; b >= 0; --b) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint32_t cand = thr[n] | (1u << b);
      int cnt = 0;
#pragma unroll
      for (int i = 0; i < PL; ++i) cnt += __popcll(__ballot(u[n][i] >= cand));
      if (cnt >= k) thr[n] = cand;
    }
  }
  // Selected: every key above the threshold, then the keys equal to it in
  // ascending expert id (slot i holds ids 64 i + lane) until k are chosen.
  bool sel[NT][PL];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    int above = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) above += __popcll(__ballot(u[n][i] > thr[n]));
    int ties_before = 0;
    const int need = k - above;  // >= 1
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const uint64_t tie = __ballot(u[n][i] == thr[n]);
      const int rank = ties_before + __popcll(tie & lanemask_lt());
      sel[n][i] = u[n][i] > thr[n] || (u[n][i] == thr[n] && rank < need);
      ties_before += __popcll(tie);
    }
  }

#pragma unroll
  for (int n = 0; n < NT; ++n) {
    int pos = 0;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const uint64_t bal = __ballot(sel[n][i]);
      if (sel[n][i] && t[n] >= 0) {
        const int o = t[n] * k + pos + __popcll(bal & lanemask_lt());
        MOE_CHECK(lane + 64 * i < E, MOE_CHECK_ROUTE_ID);
        if (MOE_GUARD(o < (t[n] + 1) * k, MOE_CHECK_ROUTE_ID)) {  // at most k per token
          idx[o] = lane + 64 * i;
          gate[o] = scaling * p[n][i];
        }
      }
      pos += __popcll(bal);
    }
  }
}

template <int PL, int U>
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ partials, int nsplit, const float* __restrict__ col_bias,
            float* __restrict__ logits_out, const float* __restrict__ bias, int T, int E,
            int k, float scaling, int32_t* __restrict__ idx, float* __restrict__ gate) {
  // selection bias and classifier offset in LDS, zero past E, so every slot
  // reads them unconditionally
  __shared__ float s_bias[64 * PL], s_cb[64 * PL];
  for (int e = threadIdx.x; e < 64 * PL; e += blockDim.x) {
    s_bias[e] = e < E ? bias[e] : 0.f;
    s_cb[e] = (col_bias != nullptr && e < E) ? col_bias[e] : 0.f;
  }
  __syncthreads();
  const int lane = lane_id();
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave

  // logits = sum of the K-split partials ([split][T][E]) in split order.  A
  // lane reads experts lane + 64 i of its row for every slot: the slots past
  // E read into the next row or, for the last row, into the workspace's
  // slack, and are discarded below.
  const float* row = partials + (size_t)t * E + lane;
  const size_t sstride = (size_t)T * E;
  float l[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) l[i] = row[64 * i];
  if constexpr (U == 1) {
    for (int sp = 1; sp < nsplit; ++sp)
#pragma unroll
      for (int i = 0; i < PL; ++i) l[i] += row[sp * sstride + 64 * i];
  } else {
    // many splits and few tokens: read U splits at a time so the loads overlap
    int sp = 1;
    for (; sp + U <= nsplit; sp += U) {
      float v[U][PL];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < PL; ++i) v[u][i] = row[(sp + u) * sstride + 64 * i];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < PL; ++i) l[i] += v[u][i];
    }
    for (; sp < nsplit; ++sp)
#pragma unroll
      for (int i = 0; i < PL; ++i) l[i] += row[sp * sstride + 64 * i];
  }
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + 64 * i;
    l[i] += s_cb[e];  // + 0 without a classifier offset
    if (e < E) {
      if (logits_out != nullptr) logits_out[(size_t)t * E + e] = l[i];
    } else {
      l[i] = -INFINITY;
    }
    m = fmaxf(m, l[i]);
  }
  float l1[1][PL], m1[1] = {m};
#pragma unroll
  for (int i = 0; i < PL; ++i) l1[0][i] = l[i];
  const int t1[1] = {t};
  select_topk<PL, 1>(l1, m1, s_bias, E, k, scaling, t1, idx, gate);
}

// The router matrix in the operand order of v_mfma_f32_16x16x32_bf16, so
// that each load of the fused kernel reads 1 KiB whole (in row order every
// instruction touched 16 rows x 64 bytes, half a cache line each, and the
// K loop was bound by the request count): block (K-step ks of 32, column
// block c) holds, for lane l, expert 16c + (l % 16) (rows past E repeat row
// E - 1) and K elements 32 ks + 8 (l / 16) .. + 7.  Written into the
// workspace on every call (the library keeps nothing between calls).
__global__ void __launch_bounds__(256)
pack_router_kernel(const __bf16* __restrict__ wr, int E, int d, int ncb,
                   u32x4_t* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;  // (ks, c, lane)
  if (i >= (d / 32) * ncb * 64) return;
  const int lane = i & 63, c = (i >> 6) % ncb, ks = (i >> 6) / ncb;
  const int e = min(16 * c + (lane & 15), E - 1);
  out[i] = *reinterpret_cast<const u32x4_t*>(wr + (size_t)e * d + 32 * ks + 8 * (lane >> 4));
}

// Router GEMM and top-k in one launch, for at most 128 experts in bf16
// (d_model a multiple of 128 * NW).  A workgroup takes 16 tokens and all
// experts (in ceil(E / 16) column blocks of 16).  Wave w of NW multiplies them by the router over the K slice w
// with v_mfma_f32_16x16x32_bf16, operands loaded straight from global memory
// (x by rows, the router matrix packed as above) into registers with P
// K-steps of 32 in flight; the slices' products are
// summed in LDS in slice order, and each wave then selects for 16/NW of the
// tokens at once.  Every workgroup reads the whole router matrix, so the
// limit is how many loads each CU keeps in flight: hence NW waves.
template <int NCB, int NW>
__global__ void __launch_bounds__(64 * NW)
router_topk_kernel(const __bf16* __restrict__ x, const u32x4_t* __restrict__ wr_packed,
                   const float* __restrict__ col_bias, float* __restrict__ logits_out,
                   const float* __restrict__ bias, int T, int E, int d, int k, float scaling,
                   int32_t* __restrict__ idx, float* __restrict__ gate) {
  // NCB 16-expert column blocks (E <= 16 NCB); PL experts per lane in the
  // selection
  constexpr int PL = (NCB * 16 + 63) / 64;
  constexpr int BT = 16;            // tokens per workgroup
  constexpr int TPW = BT / NW;      // tokens selected per wave
  constexpr int P = 4;              // K-steps in flight
  constexpr int LDP = NCB * 16 + 4; // LDS row pitch (floats): conflict-free stores
  static_assert(BT % NW == 0, "tokens per wave");
  __shared__ float s_part[NW][BT][LDP];
  __shared__ float s_bias[64 * PL];  // selection bias, zero past E
  typedef float f32x4 __attribute__((ext_vector_type(4)));

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < 64 * PL; e += 64 * NW) s_bias[e] = e < E ? bias[e] : 0.f;
  const int t0 = blockIdx.x * BT;
  const int r16 = lane & 15, oct = lane >> 4;  // operand row / col, K octet
  const int kq = d / NW;                       // K per wave
  const int nsteps = kq / 32;                  // multiple of P (host: d % (128 NW) == 0)

  // lane's operand rows: token t0 + r16 (A), expert 16c + r16 (B); rows past
  // the end are clamped (their products are never used)
  const int xr = min(t0 + r16, T - 1);
  const char* xa = (const char*)x + ((size_t)xr * d + (size_t)w * kq + oct * 8) * 2;
  // this wave's first packed block (global K-step w * nsteps, column 0)
  const u32x4_t* wpk = wr_packed + (size_t)w * nsteps * NCB * 64 + lane;

  f32x4 acc[NCB];
#pragma unroll
  for (int c = 0; c < NCB; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4_t fx[P], fw[P][NCB];
  auto fetch = [&](int slot, int st) __attribute__((always_inline)) {
    fx[slot] = *reinterpret_cast<const u32x4_t*>(xa + st * 64);
#pragma unroll
    for (int c = 0; c < NCB; ++c)
      fw[slot][c] = wpk[((size_t)st * NCB + c) * 64];
  };
#pragma unroll
  for (int u = 0; u < P; ++u) fetch(u, u);
  for (int st = 0; st < nsteps; st += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
#pragma unroll
      for (int c = 0; c < NCB; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, fx[u]), __builtin_bit_cast(bf16x8_t, fw[u][c]),
            acc[c], 0, 0, 0);
      // unconditional (clamped past the end, never used): a conditional load
      // makes the compiler drain every load in flight at the loop head
      fetch(u, min(st + u + P, nsteps - 1));
    }
  }
  // lane holds C[4 oct + i][r16] of each column block: tokens 4 oct + i
#pragma unroll
  for (int c = 0; c < NCB; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_part[w][4 * oct + i][16 * c + r16] = acc[c][i];
  __syncthreads();

  // wave w selects for tokens TPW w .. TPW w + TPW - 1 together
  float l[TPW][PL], m[TPW];
  int tk[TPW];
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int tt = TPW * w + q, t = t0 + tt;
    tk[q] = t < T ? t : -1;
    m[q] = -INFINITY;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        float v = s_part[0][tt][e];
#pragma unroll
        for (int ww = 1; ww < NW; ++ww) v += s_part[ww][tt][e];
        if (col_bias != nullptr) v += col_bias[e];
        if (logits_out != nullptr && t < T) logits_out[(size_t)t * E + e] = v;
        l[q][i] = v;
      } else {
        l[q][i] = -INFINITY;
      }
      m[q] = fmaxf(m[q], l[q][i]);
    }
  }
  select_topk<PL, TPW>(l, m, s_bias, E, k, scaling, tk, idx, gate);
}

#ifndef MOE_ROUTER_WAVES
#define MOE_ROUTER_WAVES 8
#endif

bool router_topk_fused_ok(int T, int E, int d_model, int dtype) {
  return dtype == MOE_BF16 && E <= 128 && d_model % (128 * MOE_ROUTER_WAVES) == 0 && T >= 1;
}

size_t router_packed_bytes(int E, int d_model) {
  return (size_t)((E + 15) / 16) * 16 * d_model * 2;
}

int launch_router_topk(const void* x, const void* wr, void* wr_packed, const float* col_bias,
                       float* logits_out, const float* bias, int T, int E, int d, int k,
                       float scaling, int32_t* idx, float* gate, hipStream_t st) {
  constexpr int NW = MOE_ROUTER_WAVES;
  const dim3 grid((T + 15) / 16), block(64 * NW);
  const int ncb = (E + 15) / 16;  // <= 8
  const int npack = (d / 32) * ncb * 64;
  hipLaunchKernelGGL(pack_router_kernel, dim3((npack + 255) / 256), dim3(256), 0, st,
                     (const __bf16*)wr, E, d, ncb, (u32x4_t*)wr_packed);
#define MOE_RT(NCB)                                                                         \
  hipLaunchKernelGGL((router_topk_kernel<NCB, NW>), grid, block, 0, st, (const __bf16*)x,    \
                     (const u32x4_t*)wr_packed, col_bias, logits_out, bias, T, E, d, k,      \
                     scaling, idx, gate)
  switch ((E + 15) / 16) {
    case 1: MOE_RT(1); break;
    case 2: MOE_RT(2); break;
    case 3: MOE_RT(3); break;
    case 4: MOE_RT(4); break;
    case 5: MOE_RT(5); break;
    case 6: MOE_RT(6); break;
    case 7: MOE_RT(7); break;
    default: MOE_RT(8); break;
  }
#undef MOE_RT
  return check_launch();
}

int launch_topk(const float* partials, int nsplit, const float* col_bias, float* logits_out,
                const float* bias, int T, int E, int k, float scaling, int32_t* idx, float* gate,
                hipStream_t st) {
  // few tokens (decode): one wave per workgroup, spread over more CUs
  const int wpb = T < 2048 ? 1 : 4;
  const dim3 grid((T + wpb - 1) / wpb), block(64 * wpb);
#define MOE_TOPK_ARGS partials, nsplit, col_bias, logits_out, bias, T, E, k, scaling, idx, gate
#define MOE_TOPK(PL)                                                                   \
  do {                                                                                \
    if (nsplit >= 4)                                                                  \
      hipLaunchKernelGGL((topk_kernel<PL, 4>), grid, block, 0, st, MOE_TOPK_ARGS);    \
    else                                                                              \
      hipLaunchKernelGGL((topk_kernel<PL, 1>), grid, block, 0, st, MOE_TOPK_ARGS);    \
  } while (0)
  if (E <= 64)
    MOE_TOPK(1);
  else if (E <= 128)
    MOE_TOPK(2);
  else if (E <= 256)
    MOE_TOPK(4);
  else if (E <= 512)
    MOE_TOPK(8);
  else if (E <= 768)
    MOE_TOPK(12);
  else
    MOE_TOPK(16);
#undef MOE_TOPK
#undef MOE_TOPK_ARGS
  return check_launch();
}

MOE_CHECK_ACCESSOR(check_word_route)

// Split the router's K loop until there are about 1024 (tile, split) work
// items, keeping at least two K-steps per split; the split count divides the
// K-step count.  A function of the shape only, so the workspace size is too.
int router_ksplit(int T, int E, int d_model, int dtype) {
  const int bk = dtype == MOE_BF16 ? 64 : 32;
  const int nK = d_model / bk;
  const long tiles = (long)((T + 15) / 16) * ((E + 127) / 128);
  if ((long)(T / 128) * ((E + 127) / 128) >= 256) return 1;  // 128x128 tiles, enough of them
  int s = 1;
  while (tiles * s * 2 <= 1024 && nK % (s * 2) == 0 && nK / (s * 2) >= 2) s *= 2;
  return s;
}

}  // namespace moe
