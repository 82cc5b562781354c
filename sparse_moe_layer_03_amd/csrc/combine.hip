// Combine with zero-computation experts (LongCat-2.0 Ascend deployment
// article, section "底层定制算子深度优化": Combine supporting
// zero-computation experts; data sheet table "Mixture of experts": identity
// zero experts, routed scaling factor).
//
// One block per token.  The token's FFN slots (idx < n_ffn) are gathered
// from y_perm through inv_perm and summed with their gates in slot order;
// the identity slots never touch y_perm: their gates are summed first and
// applied to x once, a scaled residual add instead of a GEMM.  fp32
// accumulation, one rounding to the output type, no atomics.

#include "common.h"
#include "internal.h"

namespace moe {

template <typename T>
__global__ void __launch_bounds__(256)
combine_kernel(const T* __restrict__ x, const T* __restrict__ y_perm,
               const int32_t* __restrict__ idx, const float* __restrict__ gate,
               const int32_t* __restrict__ inv_perm, int d, int k, int n_ffn,
               T* __restrict__ y) {
  constexpr int CE = 16 / sizeof(T);
  __shared__ int s_row[16];
  __shared__ float s_g[16];
  __shared__ float s_gz;
  __shared__ int s_nf;
  const int t = blockIdx.x;
  if (threadIdx.x == 0) {
    int nf = 0;
    float gz = 0.f;
    for (int j = 0; j < k; ++j) {
      const int a = t * k + j;
      const float g = gate[a];
      if (idx[a] < n_ffn) {
        s_row[nf] = inv_perm[a];
        s_g[nf] = g;
        ++nf;
      } else {
        gz += g;
      }
    }
    s_nf = nf;
    s_gz = gz;
  }
  __syncthreads();
  const int nf = s_nf;
  const float gz = s_gz;
  const size_t xrow = (size_t)t * d;
  for (int c = threadIdx.x; c < d / CE; c += 256) {
    float acc[CE];
#pragma unroll
    for (int i = 0; i < CE; ++i) acc[i] = 0.f;
    for (int f = 0; f < nf; ++f) {
      float v[CE];
      unpack16(ld16(y_perm + (size_t)s_row[f] * d + c * CE), v, (T*)nullptr);
      const float g = s_g[f];
#pragma unroll
      for (int i = 0; i < CE; ++i) acc[i] += g * v[i];
    }
    if (gz != 0.f) {
      float v[CE];
      unpack16(ld16(x + xrow + c * CE), v, (T*)nullptr);
#pragma unroll
      for (int i = 0; i < CE; ++i) acc[i] += gz * v[i];
    }
    st16(y + xrow + c * CE, pack16(acc, (T*)nullptr));
  }
}

int launch_combine(int dtype, const void* x, const void* y_perm, const int32_t* idx,
                   const float* gate, const int32_t* inv_perm, int T, int d, int k, int n_ffn,
                   void* y, hipStream_t st) {
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<__bf16>, dim3(T), dim3(256), 0, st, (const __bf16*)x,
                       (const __bf16*)y_perm, idx, gate, inv_perm, d, k, n_ffn, (__bf16*)y);
  else
    hipLaunchKernelGGL(combine_kernel<float>, dim3(T), dim3(256), 0, st, (const float*)x,
                       (const float*)y_perm, idx, gate, inv_perm, d, k, n_ffn, (float*)y);
  return check_launch();
}

}  // namespace moe
