// Device-side helpers shared by the MoE layer kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// 16-byte global load / store through a plain vector type.
__device__ __forceinline__ u32x4_t ld16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}

// Element <-> float conversion for the two activation types.
template <typename T> struct ElemOps;
template <> struct ElemOps<float> {
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};
template <> struct ElemOps<__bf16> {
  static __device__ __forceinline__ float to_f(__bf16 v) { return (float)v; }
  // float -> bf16 round-to-nearest-even
  static __device__ __forceinline__ __bf16 from_f(float v) { return (__bf16)v; }
};

// Unpack a 16-byte chunk into floats (8 for bf16, 4 for fp32).
__device__ __forceinline__ void unpack16(u32x4_t v, float* f, __bf16*) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t w = v[i];
    f[2 * i] = __uint_as_float(w << 16);
    f[2 * i + 1] = __uint_as_float(w & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack16(u32x4_t v, float* f, float*) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}
__device__ __forceinline__ u32x4_t pack16(const float* f, __bf16*) {
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __bf16 lo = (__bf16)f[2 * i], hi = (__bf16)f[2 * i + 1];
    uint32_t l = __builtin_bit_cast(uint16_t, lo), h = __builtin_bit_cast(uint16_t, hi);
    v[i] = l | (h << 16);
  }
  return v;
}
__device__ __forceinline__ u32x4_t pack16(const float* f, float*) {
  u32x4_t v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
  return v;
}

// Wave-wide reductions in a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ uint64_t lanemask_lt() {
  return (1ull << lane_id()) - 1ull;
}

// Inclusive scan of one int per thread over a block of NT threads (NT a
// multiple of 64, <= 1024).  `s_tmp` holds NT/64 ints.  Contains barriers.
template <int NT>
__device__ __forceinline__ int block_inclusive_scan(int v, int* s_tmp) {
  const int lane = lane_id(), w = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int u = __shfl_up(v, o, kWave);
    if (lane >= o) v += u;
  }
  if (lane == kWave - 1) s_tmp[w] = v;
  __syncthreads();
  int add = 0;
  for (int i = 0; i < w; ++i) add += s_tmp[i];
  __syncthreads();
  return v + add;
}

// Device-side index-range checks of the debug build (-DMOE_DEVICE_CHECKS,
// libmoe_mi355x_checks.so).  A failed check sets its bit (MOE_CHECK_* in
// moe.h) in a word of the translation unit's device memory and the kernel
// carries on with the access guarded as in the release build, so a check
// never faults; moe_debug_checks reads and clears the words.  Release
// builds compile every check out.
#ifdef MOE_DEVICE_CHECKS
static __device__ unsigned moe_check_word;
__device__ __forceinline__ void moe_check_fail(unsigned bit) { atomicOr(&moe_check_word, bit); }
#define MOE_CHECK(cond, bit)              \
  do {                                    \
    if (!(cond)) moe_check_fail(bit);     \
  } while (0)
// a check that also guards an access the release build makes unguarded
__device__ __forceinline__ bool moe_guard(bool ok, unsigned bit) {
  if (!ok) moe_check_fail(bit);
  return ok;
}
#define MOE_GUARD(cond, bit) moe_guard((cond), (bit))
// unsigned fn(bool clear): this translation unit's word (synchronous copy),
// cleared afterwards if `clear`
#define MOE_CHECK_ACCESSOR(fn)                                                            \
  unsigned fn(bool clear) {                                                               \
    unsigned v = 0;                                                                       \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(moe_check_word), sizeof v) != hipSuccess)      \
      return ~0u;                                                                         \
    if (clear) {                                                                          \
      const unsigned z = 0;                                                               \
      if (hipMemcpyToSymbol(HIP_SYMBOL(moe_check_word), &z, sizeof z) != hipSuccess)      \
        return ~0u;                                                                       \
    }                                                                                     \
    return v;                                                                             \
  }
#else
#define MOE_CHECK(cond, bit) \
  do {                       \
  } while (0)
#define MOE_GUARD(cond, bit) true
#define MOE_CHECK_ACCESSOR(fn) \
  unsigned fn(bool) { return 0; }
#endif
