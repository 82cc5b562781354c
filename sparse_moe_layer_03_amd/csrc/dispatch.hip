// Dispatch: per-expert histogram, exclusive prefix sum and a stable
// permutation of the T*k assignments (LongCat-2.0 Ascend deployment
// article, section "底层定制算子深度优化": Dispatch with zero-computation
// experts).  Deterministic: LDS atomics only count (integer adds commute);
// every rank is derived from assignment order, never from atomic order.
//
//   hist    nb blocks: block b counts its contiguous chunk of assignments
//           into LDS and writes the expert-major table hist[e * nb + b].
//   rows    one wave per expert: exclusive scan of the expert's row of that
//           table (contiguous, so the reads coalesce) -> the first position
//           of chunk b inside expert e's segment; the row total is counts[e].
//   (up to 4096 assignments the three steps run in one workgroup instead:
//   dispatch_one_kernel below)
//   scatter nb blocks: each block scans counts into the expert offsets (block
//           0 writes them out), so (expert e, chunk b) starts at
//           offsets[e] + row prefix.  Each of the 4 waves of block b owns a
//           quarter of the chunk; wave-level histograms give each wave its
//           starting position per expert, then the wave walks its quarter 64
//           assignments at a time, ranking equal experts among the lanes
//           with a ballot-built peer mask.

#include "common.h"
#include "internal.h"

namespace moe {

constexpr int kDispThreads = 256;

__global__ void __launch_bounds__(kDispThreads)
dispatch_hist_kernel(const int32_t* __restrict__ idx, int Tk, int E, int32_t* __restrict__ hist) {
  extern __shared__ int s_h[];
  const int nb = gridDim.x, b = blockIdx.x;
  const int chunk = (Tk + nb - 1) / nb;
  const int lo = b * chunk, hi = min(Tk, lo + chunk);
  for (int e = threadIdx.x; e < E; e += kDispThreads) s_h[e] = 0;
  __syncthreads();
  for (int a = lo + threadIdx.x; a < hi; a += kDispThreads) {
    const int e = idx[a];
    MOE_CHECK((unsigned)e < (unsigned)E, MOE_CHECK_DISPATCH_ID);
    if ((unsigned)e < (unsigned)E) atomicAdd(&s_h[e], 1);  // ids are in range by contract
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kDispThreads) hist[(size_t)e * nb + b] = s_h[e];
}

// One wave per expert e: exclusive prefix of hist[e * nb + 0 .. nb) over the
// chunks (nb <= 256, 4 per lane), written back in place; counts[e] = total.
__global__ void __launch_bounds__(kDispThreads)
dispatch_rows_kernel(int32_t* __restrict__ hist, int nb, int E, int32_t* __restrict__ counts) {
  const int e = blockIdx.x * (kDispThreads / 64) + (threadIdx.x >> 6);
  if (e >= E) return;  // uniform per wave
  const int lane = lane_id();
  int32_t* row = hist + (size_t)e * nb;
  int v[4];
  int sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // lane holds chunks 4*lane .. 4*lane+3
    const int c = lane * 4 + i;
    v[i] = c < nb ? row[c] : 0;
    sum += v[i];
  }
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  int run = incl - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = lane * 4 + i;
    if (c < nb) row[c] = run;
    run += v[i];
  }
  if (lane == 63) counts[e] = incl;
}

template <int NBITS>
__global__ void __launch_bounds__(kDispThreads)
dispatch_scatter_kernel(const int32_t* __restrict__ idx, int Tk, int E,
                        const int32_t* __restrict__ base, const int32_t* __restrict__ counts,
                        int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                        int32_t* __restrict__ inv_perm) {
  extern __shared__ int s_w[];  // [4][E] wave cursors, then [E] expert offsets
  __shared__ int s_tmp[kDispThreads / 64];
  int* s_off = s_w + 4 * E;
  const int nb = gridDim.x, b = blockIdx.x;
  {
    // expert offsets: exclusive scan of counts (E <= 1024, 4 per thread)
    int c[4];
    int sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x * 4 + i;
      c[i] = e < E ? counts[e] : 0;
      sum += c[i];
    }
    int run = block_inclusive_scan<kDispThreads>(sum, s_tmp) - sum;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = threadIdx.x * 4 + i;
      if (e < E) {
        s_off[e] = run;
        if (b == 0) offsets[e] = run;
      }
      run += c[i];
    }
    if (b == 0 && threadIdx.x == 0) offsets[E] = Tk;
  }
  const int chunk = (Tk + nb - 1) / nb;
  const int lo = b * chunk, hi = min(Tk, lo + chunk);
  const int w = threadIdx.x >> 6, lane = lane_id();
  const int sub = (chunk + 3) / 4;
  const int wlo = min(hi, lo + w * sub), whi = min(hi, wlo + sub);

  for (int i = threadIdx.x; i < 4 * E; i += kDispThreads) s_w[i] = 0;
  __syncthreads();
  for (int a = wlo + lane; a < whi; a += 64) {
    const int e = idx[a];
    if ((unsigned)e < (unsigned)E) atomicAdd(&s_w[w * E + e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kDispThreads) {
    int run = s_off[e] + base[(size_t)e * nb + b];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = s_w[q * E + e];
      s_w[q * E + e] = run;
      run += c;
    }
  }
  __syncthreads();

  int* my = s_w + w * E;
  for (int a0 = wlo; a0 < whi; a0 += 64) {
    const int a = a0 + lane;
    const int e0 = (a < whi) ? idx[a] : -1;
    const bool valid = (unsigned)e0 < (unsigned)E;
    const int e = valid ? e0 : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < NBITS; ++bit) {
      const bool s = (e >> bit) & 1;
      const uint64_t m = __ballot(s);
      peers &= s ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(peers & lanemask_lt());
      const int pos = my[e] + rank;
      if (MOE_GUARD((unsigned)pos < (unsigned)Tk, MOE_CHECK_DISPATCH_POS)) {
        perm[pos] = a;
        inv_perm[a] = pos;
      }
    }
    // the highest lane of each peer group advances that expert's cursor
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers >> lane) == 1ull) my[e] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

// The whole dispatch in one workgroup of 16 waves, for up to 4096
// assignments (one launch instead of three).  Wave w owns the contiguous
// chunk w of the assignments: per-wave LDS histograms, then thread e sums
// expert e over the waves (counts), the counts are scanned into offsets and
// each wave's first position per expert follows in wave order; then every
// wave ranks and scatters its chunk as in dispatch_scatter_kernel.  Same
// stable order (expert, assignment id) as the three-kernel path.
constexpr int kDispOneWaves = 16;
constexpr int kDispOneMax = 4096;

template <int NBITS>
__global__ void __launch_bounds__(64 * kDispOneWaves)
dispatch_one_kernel(const int32_t* __restrict__ idx, int Tk, int E, int32_t* __restrict__ counts,
                    int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                    int32_t* __restrict__ inv_perm) {
  extern __shared__ int s_w[];  // [kDispOneWaves][E]
  __shared__ int s_tmp[kDispOneWaves];
  const int w = threadIdx.x >> 6, lane = lane_id();
  const int chunk = (Tk + kDispOneWaves - 1) / kDispOneWaves;
  const int wlo = min(Tk, w * chunk), whi = min(Tk, wlo + chunk);

  for (int i = threadIdx.x; i < kDispOneWaves * E; i += blockDim.x) s_w[i] = 0;
  __syncthreads();
  for (int a = wlo + lane; a < whi; a += 64) {
    const int e = idx[a];
    MOE_CHECK((unsigned)e < (unsigned)E, MOE_CHECK_DISPATCH_ID);
    if ((unsigned)e < (unsigned)E) atomicAdd(&s_w[w * E + e], 1);  // ids in range by contract
  }
  __syncthreads();
  // thread e: count of expert e, then the exclusive scan over experts
  const int e = threadIdx.x;  // E <= 1024 = blockDim.x
  int c = 0;
  if (e < E)
    for (int q = 0; q < kDispOneWaves; ++q) c += s_w[q * E + e];
  const int start = block_inclusive_scan<64 * kDispOneWaves>(c, s_tmp) - c;
  if (e < E) {
    counts[e] = c;
    offsets[e] = start;
    int run = start;
    for (int q = 0; q < kDispOneWaves; ++q) {
      const int v = s_w[q * E + e];
      s_w[q * E + e] = run;
      run += v;
    }
  }
  if (threadIdx.x == 0) offsets[E] = Tk;
  __syncthreads();

  int* my = s_w + w * E;
  for (int a0 = wlo; a0 < whi; a0 += 64) {
    const int a = a0 + lane;
    const int e0 = (a < whi) ? idx[a] : -1;
    const bool valid = (unsigned)e0 < (unsigned)E;
    const int ex = valid ? e0 : 0;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < NBITS; ++bit) {
      const bool sb = (ex >> bit) & 1;
      const uint64_t m = __ballot(sb);
      peers &= sb ? m : ~m;
    }
    if (valid) {
      const int rank = __popcll(peers & lanemask_lt());
      const int pos = my[ex] + rank;
      if (MOE_GUARD((unsigned)pos < (unsigned)Tk, MOE_CHECK_DISPATCH_POS)) {
        perm[pos] = a;
        inv_perm[a] = pos;
      }
    }
    // the highest lane of each peer group advances that expert's cursor
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers >> lane) == 1ull) my[ex] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

int launch_dispatch(const int32_t* idx, int Tk, int E, int nb, int32_t* block_hist,
                    int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                    hipStream_t st) {
  // 16 E ints of dynamic LDS stay under the 64 KiB default
  if (Tk <= kDispOneMax && E <= 1000) {
    const size_t lds = (size_t)kDispOneWaves * E * sizeof(int);
    if (E <= 256)
      hipLaunchKernelGGL(dispatch_one_kernel<8>, dim3(1), dim3(64 * kDispOneWaves), lds, st,
                         idx, Tk, E, counts, offsets, perm, inv_perm);
    else
      hipLaunchKernelGGL(dispatch_one_kernel<10>, dim3(1), dim3(64 * kDispOneWaves), lds, st,
                         idx, Tk, E, counts, offsets, perm, inv_perm);
    return check_launch();
  }
  hipLaunchKernelGGL(dispatch_hist_kernel, dim3(nb), dim3(kDispThreads), E * sizeof(int), st,
                     idx, Tk, E, block_hist);
  int rc = check_launch();
  if (rc) return rc;
  hipLaunchKernelGGL(dispatch_rows_kernel, dim3((E + 3) / 4), dim3(kDispThreads), 0, st,
                     block_hist, nb, E, counts);
  rc = check_launch();
  if (rc) return rc;
  const size_t lds = 5 * (size_t)E * sizeof(int);
  if (E <= 256)
    hipLaunchKernelGGL(dispatch_scatter_kernel<8>, dim3(nb), dim3(kDispThreads), lds, st, idx, Tk,
                       E, block_hist, counts, offsets, perm, inv_perm);
  else
    hipLaunchKernelGGL(dispatch_scatter_kernel<10>, dim3(nb), dim3(kDispThreads), lds, st, idx,
                       Tk, E, block_hist, counts, offsets, perm, inv_perm);
  return check_launch();
}

// x_perm[p] = x[perm[p] / k] for p < offsets[n_ffn]; one block per row.
template <typename T>
__global__ void __launch_bounds__(256)
gather_rows_kernel(const T* __restrict__ x, const int32_t* __restrict__ perm,
                   const int32_t* __restrict__ offsets, int n_ffn, int k, int d,
                   T* __restrict__ x_perm) {
  const int p = blockIdx.x;
  if (p >= offsets[n_ffn]) return;
  // gridDim.x = T*k
  if (!MOE_GUARD((unsigned)perm[p] < gridDim.x, MOE_CHECK_GEMM_ROW)) return;
  const int tok = perm[p] / k;
  constexpr int CE = 16 / sizeof(T);
  const char* src = (const char*)(x + (size_t)tok * d);
  char* dst = (char*)(x_perm + (size_t)p * d);
  for (int c = threadIdx.x; c < d / CE; c += 256) st16(dst + c * 16, ld16(src + c * 16));
}

MOE_CHECK_ACCESSOR(check_word_dispatch)

int launch_gather(int dtype, const void* x, const int32_t* perm, const int32_t* offsets,
                  int n_ffn, int Tk, int k, int d, void* x_perm, hipStream_t st) {
  if (dtype == MOE_BF16)
    hipLaunchKernelGGL(gather_rows_kernel<__bf16>, dim3(Tk), dim3(256), 0, st,
                       (const __bf16*)x, perm, offsets, n_ffn, k, d, (__bf16*)x_perm);
  else
    hipLaunchKernelGGL(gather_rows_kernel<float>, dim3(Tk), dim3(256), 0, st, (const float*)x,
                       perm, offsets, n_ffn, k, d, (float*)x_perm);
  return check_launch();
}

}  // namespace moe
