// moe_dispatch_noalloc: moe_dispatch for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that
// forbid allocation).  Same kernels and results as moe_dispatch; the one
// scratch buffer those kernels use -- the per-block expert histogram of the
// multi-block path -- is a static device array of this library instead of
// a slice of the caller's workspace.
//
// The array holds E * nb int32 with E <= 1024 experts and nb <= 256 blocks:
// 1 MiB.  Each device the library runs on holds its own copy until the
// process ends.  Nothing in it must start at zero: the histogram kernel
// writes every entry it covers before the scan and scatter read them.
// Every call on a device shares that device's copy, so calls that overlap
// on one device (two streams, two threads) race on it.

#include <mutex>

#include "common.h"
#include "internal.h"

namespace moe {

constexpr size_t kNoallocScratchInts = (size_t)1024 * 256;
static __device__ __align__(256) int32_t scratch[kNoallocScratchInts];

// Device address of `scratch` on the current device, looked up once per
// device with that device current.  In host code `scratch` names a host-side
// stand-in, never the device memory: only this address is passed on.
static int noalloc_scratch(int32_t** ptr) {
  constexpr int kDevs = 64;
  static std::once_flag once[kDevs];
  static int32_t* addr[kDevs];
  static hipError_t err[kDevs];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return MOE_EHIP;
  std::call_once(once[dev], [dev] {
    void* p = nullptr;
    err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = static_cast<int32_t*>(p);
  });
  if (err[dev] != hipSuccess || addr[dev] == nullptr) {
    set_hip_error(err[dev] != hipSuccess ? err[dev] : hipErrorInvalidSymbol);
    return MOE_EHIP;
  }
  *ptr = addr[dev];
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_dispatch_noalloc(const moe_shape* s, const int32_t* topk_idx, const void* x,
                                    int32_t* counts, int32_t* offsets, int32_t* perm,
                                    int32_t* inv_perm, void* x_perm, void* stream) {
  int rc = dispatch_checks(s, topk_idx, x, counts, offsets, perm, inv_perm, x_perm);
  if (rc) return rc;
  const size_t need = (size_t)(s->n_ffn + s->n_zero) * dispatch_blocks((long)s->T * s->top_k);
  if (need > kNoallocScratchInts) return MOE_EUNSUPPORTED;
  int32_t* hist = nullptr;
  rc = noalloc_scratch(&hist);
  if (rc) return rc;
  return dispatch_run(s, topk_idx, x, counts, offsets, perm, inv_perm, x_perm, hist,
                      (hipStream_t)stream);
}
