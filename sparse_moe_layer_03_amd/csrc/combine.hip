// Combine with zero-computation experts (LongCat-2.0 Ascend deployment
// article, section "底层定制算子深度优化": Combine supporting
// zero-computation experts; data sheet table "Mixture of experts": identity
// zero experts, routed scaling factor).
//
// One block per token.  Wave 0 reads all of the token's slots at once; the
// FFN slots (idx < n_ffn) are gathered from y_perm through inv_perm (every
// slot's load issued before any is summed) and summed with their gates in
// slot order;
// the identity slots never touch y_perm: their gates are summed first and
// applied to x once, a scaled residual add instead of a GEMM.  fp32
// accumulation, one rounding to the output type, no atomics.

#include "common.h"
#include "internal.h"

namespace moe {

template <typename T, int MAXK>
__global__ void __launch_bounds__(256)
combine_kernel(const T* __restrict__ x, const T* __restrict__ y_perm,
               const int32_t* __restrict__ idx, const float* __restrict__ gate,
               const int32_t* __restrict__ inv_perm, int d, int k, int n_ffn,
               T* __restrict__ y) {
  constexpr int CE = 16 / sizeof(T);
  __shared__ int s_row[MAXK];
  __shared__ float s_g[MAXK];
  __shared__ float s_gz;
  __shared__ int s_nf;
  const int t = blockIdx.x;
  if (threadIdx.x < 64) {
    // wave 0: lane j reads slot j (all slots at once); the FFN slots are
    // compacted in slot order, the identity gates summed in slot order
    const int lane = threadIdx.x;
    int e = n_ffn, row = 0;
    float g = 0.f;
    if (lane < k) {
      const int a = t * k + lane;
      e = idx[a];
      g = gate[a];
      row = inv_perm[a];
      // gridDim.x = T
      const bool row_ok = (unsigned)row < gridDim.x * (unsigned)k;
      if (e < n_ffn && !MOE_GUARD(row_ok, MOE_CHECK_COMBINE_ROW)) row = 0;
    }
    const bool ffn = lane < k && e < n_ffn;
    const uint64_t fb = __ballot(ffn);
    if (ffn) {
      const int pos = __popcll(fb & lanemask_lt());
      s_row[pos] = row;
      s_g[pos] = g;
    }
    const float gid = (lane < k && !ffn) ? g : 0.f;
    float gz = 0.f;
    for (int j = 0; j < k; ++j) {
      const float v = __shfl(gid, j, kWave);
      if (!((fb >> j) & 1)) gz += v;
    }
    if (lane == 0) {
      s_nf = __popcll(fb);
      s_gz = gz;
    }
  }
  __syncthreads();
  const int nf = s_nf;
  const float gz = s_gz;
  const size_t xrow = (size_t)t * d;
  for (int c = threadIdx.x; c < d / CE; c += 256) {
    // issue every slot's load before accumulating (in slot order); y_perm,
    // x and y are touched once here, so they bypass the caches' retention
    // (non-temporal: prefill combine 0.40 -> 0.36 ms)
    u32x4_t raw[MAXK];
#pragma unroll
    for (int f = 0; f < MAXK; ++f)
      if (f < nf)
        raw[f] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4_t*>(y_perm + (size_t)s_row[f] * d + c * CE));
    u32x4_t rx = {0, 0, 0, 0};
    if (gz != 0.f)
      rx = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(x + xrow + c * CE));
    float acc[CE];
#pragma unroll
    for (int i = 0; i < CE; ++i) acc[i] = 0.f;
#pragma unroll
    for (int f = 0; f < MAXK; ++f) {
      if (f < nf) {
        float v[CE];
        unpack16(raw[f], v, (T*)nullptr);
        const float gf = s_g[f];
#pragma unroll
        for (int i = 0; i < CE; ++i) acc[i] += gf * v[i];
      }
    }
    if (gz != 0.f) {
      float v[CE];
      unpack16(rx, v, (T*)nullptr);
#pragma unroll
      for (int i = 0; i < CE; ++i) acc[i] += gz * v[i];
    }
    __builtin_nontemporal_store(pack16(acc, (T*)nullptr),
                                reinterpret_cast<u32x4_t*>(y + xrow + c * CE));
  }
}

MOE_CHECK_ACCESSOR(check_word_combine)

int launch_combine(int dtype, const void* x, const void* y_perm, const int32_t* idx,
                   const float* gate, const int32_t* inv_perm, int T, int d, int k, int n_ffn,
                   void* y, hipStream_t st) {
#define MOE_COMB(TY, MK)                                                                  \
  hipLaunchKernelGGL((combine_kernel<TY, MK>), dim3(T), dim3(256), 0, st, (const TY*)x,   \
                     (const TY*)y_perm, idx, gate, inv_perm, d, k, n_ffn, (TY*)y)
  if (dtype == MOE_BF16) {
    if (k <= 8) MOE_COMB(__bf16, 8);
    else MOE_COMB(__bf16, 16);
  } else {
    if (k <= 8) MOE_COMB(float, 8);
    else MOE_COMB(float, 16);
  }
#undef MOE_COMB
  return check_launch();
}

}  // namespace moe
