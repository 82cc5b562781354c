// Expert placement balancing over an expert-parallel (EP) domain (LongCat-2.0
// Ascend deployment article, section "MoE专家动态负载均衡": with a very large
// EP domain the tokens each expert receives vary widely, and dynamic load
// balancing narrows the gap between experts' loads).  Routing is untouched:
// the plan decides where the FFN experts' rows are computed, not which
// experts a token picks.
//
// The N FFN experts occupy S >= N expert slots on D devices (S / D each):
//   1. replicas: every expert holds one slot; each redundant slot goes, one
//      at a time, to the expert with the most tokens per replica (largest
//      c_e / r_e, compared exactly as c_a r_b > c_b r_a; ties to the lower
//      id), which minimises the largest per-replica load;
//   2. slots in expert order, replica j of an expert with c rows and r
//      replicas taking rows [j c / r, (j+1) c / r) of its sorted segment;
//   3. placement, longest processing time first: slots by load descending
//      (ties to the lower slot), each to the least-loaded device that still
//      has room (ties to the lower device).
// One workgroup: wave 0 runs the replica rounds (16 experts per lane,
// register-resident) and the placement (one device per lane); all four
// waves run the bitonic sort of the slot keys in LDS.

#include <limits.h>

#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kEplbThreads = 256;
constexpr int kEplbPerLane = 1024 / 64;  // experts per lane (N <= 1024)

// (c_a, r_a, e_a) before (c_b, r_b, e_b): more tokens per replica, then lower id
__device__ __forceinline__ bool eplb_before(int ca, int ra, int ea, int cb, int rb, int eb) {
  const long long l = (long long)ca * rb, rgt = (long long)cb * ra;
  return l > rgt || (l == rgt && ea < eb);
}

__global__ void __launch_bounds__(kEplbThreads)
eplb_kernel(const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets, int N,
            int S, int D, int32_t* __restrict__ replicas, int32_t* __restrict__ slot_expert,
            int32_t* __restrict__ slot_rows, int32_t* __restrict__ slot_device,
            int32_t* __restrict__ device_load) {
  __shared__ unsigned long long s_key[kEplbMaxSlots];  // (load << 32) | ~slot
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int P = 1;  // sort length: a power of two >= S
  while (P < S) P <<= 1;
  for (int i = tid; i < P; i += kEplbThreads) s_key[i] = 0ull;  // padding sorts last
  __syncthreads();

  if (wave == 0) {
    // ---- 1. replicas
    int c[kEplbPerLane], r[kEplbPerLane];
#pragma unroll
    for (int i = 0; i < kEplbPerLane; ++i) {
      const int e = lane + 64 * i;
      c[i] = e < N ? counts[e] : 0;
      r[i] = 1;
    }
    for (int round = 0; round < S - N; ++round) {
      int bc = -1, br = 1, be = INT_MAX;  // below every expert
#pragma unroll
      for (int i = 0; i < kEplbPerLane; ++i) {
        const int e = lane + 64 * i;
        if (e < N && eplb_before(c[i], r[i], e, bc, br, be)) {
          bc = c[i];
          br = r[i];
          be = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const int oc = __shfl_xor(bc, o, kWave), orr = __shfl_xor(br, o, kWave);
        const int oe = __shfl_xor(be, o, kWave);
        if (eplb_before(oc, orr, oe, bc, br, be)) {
          bc = oc;
          br = orr;
          be = oe;
        }
      }
#pragma unroll
      for (int i = 0; i < kEplbPerLane; ++i)
        if (lane + 64 * i == be) ++r[i];
    }
    // ---- 2. slots in expert order (exclusive scan of the replica counts)
    int run = 0;
#pragma unroll
    for (int i = 0; i < kEplbPerLane; ++i) {
      const int e = lane + 64 * i;
      const int v = e < N ? r[i] : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
      }
      const int first = run + incl - v;
      run += __shfl(incl, 63, kWave);
      if (e < N) {
        replicas[e] = v;
        const long long ce = c[i];
        const int base = offsets[e];
        for (int j = 0; j < v; ++j) {
          const int s = first + j;
          const int b = base + (int)((j * ce) / v), en = base + (int)(((j + 1) * ce) / v);
          slot_expert[s] = e;
          slot_rows[2 * s] = b;
          slot_rows[2 * s + 1] = en;
          s_key[s] = ((unsigned long long)(unsigned)(en - b) << 32) | (0xFFFFFFFFu - (unsigned)s);
        }
      }
    }
  }
  __syncthreads();

  // ---- sort the slot keys descending (load descending, then slot ascending)
  for (int k = 2; k <= P; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < P; i += kEplbThreads) {
        const int l = i ^ j;
        if (l > i) {
          const unsigned long long a = s_key[i], b = s_key[l];
          const bool desc = (i & k) == 0;
          if (desc ? (a < b) : (a > b)) {
            s_key[i] = b;
            s_key[l] = a;
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- 3. placement: lane d holds device d.  Loads sum to at most the
  // FFN assignments (< 2^31), so the least load is a 32-bit wave minimum
  // and the lowest device holding it the first set bit of a ballot.
  if (wave == 0) {
    const int cap = S / D;
    int load = 0, used = 0;
    for (int idx = 0; idx < S; ++idx) {
      const unsigned long long key = s_key[idx];
      const int s = (int)(0xFFFFFFFFu - (unsigned)(key & 0xFFFFFFFFull));
      const int w = (int)(key >> 32);
      const bool room = lane < D && used < cap;
      int m = room ? load : INT_MAX;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) m = min(m, __shfl_xor(m, o, kWave));
      const int d = __ffsll((unsigned long long)__ballot(room && load == m)) - 1;
      if (lane == d) {
        load += w;
        ++used;
      }
      if (lane == 0) slot_device[s] = d;
    }
    if (lane < D) device_load[lane] = load;
  }
}

int launch_eplb(const int32_t* counts, const int32_t* offsets, int n_ffn, int n_slots,
                int n_devices, int32_t* replicas, int32_t* slot_expert, int32_t* slot_rows,
                int32_t* slot_device, int32_t* device_load, hipStream_t st) {
  hipLaunchKernelGGL(eplb_kernel, dim3(1), dim3(kEplbThreads), 0, st, counts, offsets, n_ffn,
                     n_slots, n_devices, replicas, slot_expert, slot_rows, slot_device,
                     device_load);
  return check_launch();
}

}  // namespace moe
