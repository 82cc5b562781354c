// Softmax + biased top-k + gates, one wave64 per token.
//
// LongCat-2.0 data sheet (archdb), table "Mixture of experts": the router
// scores FFN and identity experts together and selects the top k by score
// plus e_score_correction_bias; the gates are the unbiased scores times the
// routed scaling factor, not renormalised.
//
// Each lane holds experts lane, lane+64, ... in registers (E <= 1024 -> at
// most 16 per lane).  The softmax max/sum and every selection round are
// butterfly reductions over the wave in a fixed order, so the result is
// deterministic.  Selection compares (key, -id): larger key wins, equal keys
// go to the lower expert id.  The chosen set is emitted in ascending expert
// id with a ballot per register slot.

#include <math.h>

#include "common.h"
#include "internal.h"

namespace moe {

template <int PL, int U>
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ partials, int nsplit, const float* __restrict__ col_bias,
            float* __restrict__ logits_out, const float* __restrict__ bias, int T, int E,
            int k, float scaling, int32_t* __restrict__ idx, float* __restrict__ gate) {
  const int lane = lane_id();
  const int t = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave

  // logits = sum of the K-split partials in split order (+ classifier offset)
  float l[PL];
  float m = -INFINITY;
  if constexpr (U == 1) {
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        float v = partials[(size_t)t * E + e];
        for (int sp = 1; sp < nsplit; ++sp) v += partials[((size_t)sp * T + t) * E + e];
        if (col_bias != nullptr) v += col_bias[e];
        if (logits_out != nullptr) logits_out[(size_t)t * E + e] = v;
        l[i] = v;
      } else {
        l[i] = -INFINITY;
      }
      m = fmaxf(m, l[i]);
    }
  } else {
    // many splits and few tokens: read U splits at a time so the loads overlap
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + 64 * i;
      l[i] = e < E ? partials[(size_t)t * E + e] : 0.f;
    }
    int sp = 1;
    for (; sp + U <= nsplit; sp += U) {
      float v[U][PL];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < PL; ++i) {
          const int e = lane + 64 * i;
          v[u][i] = e < E ? partials[((size_t)(sp + u) * T + t) * E + e] : 0.f;
        }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < PL; ++i) l[i] += v[u][i];
    }
    for (; sp < nsplit; ++sp)
#pragma unroll
      for (int i = 0; i < PL; ++i) {
        const int e = lane + 64 * i;
        if (e < E) l[i] += partials[((size_t)sp * T + t) * E + e];
      }
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + 64 * i;
      if (e < E) {
        if (col_bias != nullptr) l[i] += col_bias[e];
        if (logits_out != nullptr) logits_out[(size_t)t * E + e] = l[i];
      } else {
        l[i] = -INFINITY;
      }
      m = fmaxf(m, l[i]);
    }
  }
  m = wave_max(m);
  float s = 0.f;
  float p[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + 64 * i;
    p[i] = (e < E) ? expf(l[i] - m) : 0.f;
    s += p[i];
  }
  s = wave_sum(s);
  float key[PL];
  bool avail[PL], sel[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int e = lane + 64 * i;
    p[i] = p[i] / s;
    avail[i] = e < E;
    sel[i] = false;
    key[i] = avail[i] ? p[i] + bias[e] : 0.f;
    if (key[i] != key[i]) key[i] = -INFINITY;  // NaN never outranks a number
  }

  for (int r = 0; r < k; ++r) {
    float bk = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int e = lane + 64 * i;
      if (avail[i] && (key[i] > bk || (key[i] == bk && e < bid))) {
        bk = key[i];
        bid = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ok = __shfl_xor(bk, o, kWave);
      const int oid = __shfl_xor(bid, o, kWave);
      if (ok > bk || (ok == bk && oid < bid)) {
        bk = ok;
        bid = oid;
      }
    }
    if ((bid & 63) == lane) {
#pragma unroll
      for (int i = 0; i < PL; ++i)
        if (i == (bid >> 6)) {
          avail[i] = false;
          sel[i] = true;
        }
    }
  }

  int pos = 0;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const uint64_t bal = __ballot(sel[i]);
    if (sel[i]) {
      const int o = t * k + pos + __popcll(bal & lanemask_lt());
      idx[o] = lane + 64 * i;
      gate[o] = scaling * p[i];
    }
    pos += __popcll(bal);
  }
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
  else
    MOE_TOPK(16);
#undef MOE_TOPK
#undef MOE_TOPK_ARGS
  return check_launch();
}

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
