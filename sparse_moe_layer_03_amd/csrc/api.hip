// C ABI of the MoE layer library: argument checks, workspace layout and the
// launch sequence of each call.  Every check runs on the host before any
// work is enqueued; no call allocates, frees or synchronises.

#include <math.h>
#include <stdint.h>

#include <mutex>

#include <algorithm>

#include "common.h"
#include "internal.h"
#include "plan.h"

namespace moe {

static thread_local hipError_t g_last_hip = hipSuccess;

void set_hip_error(hipError_t e) { g_last_hip = e; }

int check_launch() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_hip = e;
    return MOE_EHIP;
  }
  return MOE_OK;
}

// Multiprocessor count per device, queried once per device (std::call_once;
// a failed query is remembered as MOE_EHIP).
constexpr int kMaxDevices = 64;
int device_cu_count() {
  static std::once_flag once[kMaxDevices];
  static int cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_EHIP;
  std::call_once(once[dev], [dev] {
    int n = 0;
    const bool ok = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) ==
                        hipSuccess && n >= 1;
    cache[dev] = ok ? n : MOE_EHIP;
  });
  return cache[dev];
}

// CUs a stream may use: the set bits of its CU mask (a stream created with
// hipExtStreamCreateWithCUMask), else the device's CU count.  Persistent
// grids are sized by it, so a kernel on a partitioned stream does not queue
// workgroups behind its own.
int stream_cu_count(hipStream_t st) {
  const int dev_cus = device_cu_count();
  if (dev_cus <= 0 || st == nullptr) return dev_cus;
  uint32_t mask[32] = {};  // up to 1024 CUs
  if (hipExtStreamGetCUMask(st, 32, mask) != hipSuccess) {
    (void)hipGetLastError();  // not a launch failure: fall back to the device
    return dev_cus;
  }
  int n = 0;
  for (uint32_t m : mask) n += __builtin_popcount(m);
  return (n >= 1 && n < dev_cus) ? n : dev_cus;
}

static int elem_size(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

static int check_shape(const moe_shape* s) {
  if (s == nullptr) return MOE_EINVAL;
  if (s->T < 1 || s->n_ffn < 1 || s->n_zero < 0 || s->top_k < 1 || s->d_model < 1 || s->d_ff < 1)
    return MOE_EINVAL;
  const long E = (long)s->n_ffn + s->n_zero;
  if (s->top_k > E) return MOE_EINVAL;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_EUNSUPPORTED;
  if (E > 1024 || s->top_k > 16) return MOE_EUNSUPPORTED;
  if (s->d_model % 64 != 0 || s->d_ff % 64 != 0) return MOE_EUNSUPPORTED;
  if ((long)s->T * s->top_k >= (1L << 31)) return MOE_EUNSUPPORTED;
  if (!isfinite(s->routed_scaling)) return MOE_ENONFINITE;
  return MOE_OK;
}

static bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

struct WsLayout {
  size_t logits, hist, h, wrp, total;
};

static size_t up256(size_t v) { return (v + 255) & ~(size_t)255; }
using plan::cdiv;

// Router GEMM plan.  The one-kernel router + top-k takes up to 128 experts.
// Above that, many tokens go through the 256x256 kernel with its K loop
// split so that the (split, tile) items fill about one round of the chip;
// otherwise the general kernel (128x128 tiles, or 16-row tiles with a split
// K loop).  The split count sizes the partial-logit workspace, so it is a
// function of the shape and the device's CU count only.
struct RouterPlan {
  bool big;
  int ksplit;
};
static RouterPlan router_plan(const moe_shape* s) {
  const int E = s->n_ffn + s->n_zero;
  const RouterPlan general{false, router_ksplit(s->T, E, s->d_model, s->dtype)};
  if (router_topk_fused_ok(s->T, E, s->d_model, s->dtype)) return general;
  // token rows are addressed from a 64-bit tile base, router rows by 32-bit
  // offsets ((E * d_model * 2 < 2^32 for E <= 1024 and any int d_model
  // the workspace can hold))
  if (s->dtype != MOE_BF16 || s->d_model % 128 != 0 || s->T < 512 ||
      (size_t)E * s->d_model * 2 >= (1ull << 32))
    return general;
  const long items = cdiv(s->T, kBigTileRows) * cdiv(E, 256);
  const int nK = s->d_model / 64;
  const int G = big_grid(nullptr);  // the device's: it sizes the workspace
  int ks = 1;
  while (ks < 8 && items * ks * 2 <= G && nK % (4 * ks) == 0) ks *= 2;
  if (items * ks * 2 < G) return general;  // too few tiles even when split
  return RouterPlan{true, ks};
}

static WsLayout ws_layout(const moe_shape* s) {
  const size_t E = (size_t)s->n_ffn + s->n_zero;
  const size_t Tk = (size_t)s->T * s->top_k;
  WsLayout w;
  size_t off = 0;
  w.logits = off;  // K-split partial logits, then slack: the top-k kernel
                   // reads whole 64-expert slots of the last row
  off = up256(off + (size_t)router_plan(s).ksplit * s->T * E * sizeof(float) + 4096);
  w.hist = off;
  off = up256(off + E * (size_t)dispatch_blocks((long)Tk) * sizeof(int32_t));
  w.h = off;
  off = up256(off + Tk * (size_t)s->d_ff * elem_size(s->dtype));
  w.wrp = off;  // router matrix repacked for the fused router + top-k kernel
  if (router_topk_fused_ok(s->T, (int)E, s->d_model, s->dtype))
    off = up256(off + router_packed_bytes((int)E, s->d_model));
  w.total = off;
  return w;
}

// 128x128 tiles (else 16x128) for the general kernel.
static int ffn_big_tiles(const moe_shape* s) {
  return plan::ffn_tall_tiles(s->T, s->top_k, s->n_ffn, s->n_zero, s->d_model, s->d_ff);
}

// The many-row expert GEMMs (256x256 and 320x192 direct-to-LDS tiles);
// `gather`: gate/up reads x through perm.
static bool ffn_use_big(const moe_shape* s, bool gather, hipStream_t st) {
  return plan::ffn_use_big(s->T, s->top_k, s->n_ffn, s->n_zero, s->d_model, s->d_ff,
                           s->dtype == MOE_BF16, gather, big_grid(st));
}

// 128x128 router tiles when there are enough of them (prefill), else 16-row
// tiles with a split K loop.
static int router_big_tiles(const moe_shape* s) {
  const int E = s->n_ffn + s->n_zero;
  return router_ksplit(s->T, E, s->d_model, s->dtype) == 1 && (long)(s->T / 128) * ((E + 127) / 128) >= 256;
}

int dispatch_checks(const moe_shape* s, const int32_t* topk_idx, const void* x,
                    int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                    void* x_perm) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!topk_idx || !counts || !offsets || !perm || !inv_perm || (x_perm && !x))
    return MOE_EINVAL;
  if (!al4(topk_idx) || !al4(counts) || !al4(offsets) || !al4(perm) || !al4(inv_perm) ||
      (x_perm && (!al16(x) || !al16(x_perm))))
    return MOE_EALIGN;
  return MOE_OK;
}

int dispatch_run(const moe_shape* s, const int32_t* topk_idx, const void* x,
                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                 void* x_perm, int32_t* hist, hipStream_t st) {
  const int E = s->n_ffn + s->n_zero;
  const int Tk = s->T * s->top_k;
  int rc = launch_dispatch(topk_idx, Tk, E, dispatch_blocks(Tk), hist, counts, offsets, perm,
                           inv_perm, st);
  if (rc) return rc;
  if (x_perm)
    rc = launch_gather(s->dtype, x, perm, offsets, s->n_ffn, Tk, s->top_k, s->d_model, x_perm, st);
  return rc;
}

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK) return 0;
  return ws_layout(s).total;
}

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument (null pointer or size out of range)";
    case MOE_EUNSUPPORTED: return "shape or dtype outside the supported limits";
    case MOE_EHIP: return hipGetErrorString(g_last_hip);
    case MOE_ENONFINITE: return "non-finite parameter";
    case MOE_EALIGN: return "pointer not aligned (16 bytes for bulk arrays, 4 for others)";
    default: return "unknown status";
  }
}

int moe_device_cu_count(void) { return device_cu_count(); }

int moe_route(const moe_shape* s, const void* x, const void* w_router, const float* logit_bias,
              const float* bias, int32_t* topk_idx, float* topk_gate, float* logits_out, void* ws,
              void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!x || !w_router || !bias || !topk_idx || !topk_gate || !ws) return MOE_EINVAL;
  if (!al16(x) || !al16(w_router) || !al16(ws) || !al4(bias) || !al4(topk_idx) ||
      !al4(topk_gate) || (logit_bias && !al4(logit_bias)) || (logits_out && !al4(logits_out)))
    return MOE_EALIGN;
  hipStream_t st = (hipStream_t)stream;
  const int E = s->n_ffn + s->n_zero;
  if (router_topk_fused_ok(s->T, E, s->d_model, s->dtype))
    return launch_router_topk(x, w_router, (char*)ws + ws_layout(s).wrp, logit_bias, logits_out,
                              bias, s->T, E, s->d_model, s->top_k, s->routed_scaling, topk_idx,
                              topk_gate, st);
  const RouterPlan rp = router_plan(s);
  const int nsplit = rp.ksplit;
  float* partials = (float*)((char*)ws + ws_layout(s).logits);
  GemmArgs g{};
  g.a = x;
  g.b0 = w_router;
  g.c = partials;
  g.M = s->T;
  g.N = E;
  g.K = s->d_model;
  g.ngroups = 1;
  g.top_k = s->top_k;
  g.ksplit = nsplit;
  rc = rp.big ? launch_gemm_big(0, g, st) : launch_gemm(s->dtype, 0, router_big_tiles(s), g, st);
  if (rc) return rc;
  return launch_topk(partials, nsplit, logit_bias, logits_out, bias, s->T, E, s->top_k,
                     s->routed_scaling, topk_idx, topk_gate, st);
}

int moe_dispatch(const moe_shape* s, const int32_t* topk_idx, const void* x, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* x_perm, void* ws,
                 void* stream) {
  int rc = dispatch_checks(s, topk_idx, x, counts, offsets, perm, inv_perm, x_perm);
  if (rc) return rc;
  if (!ws) return MOE_EINVAL;
  if (!al16(ws)) return MOE_EALIGN;
  int32_t* hist = (int32_t*)((char*)ws + ws_layout(s).hist);
  return dispatch_run(s, topk_idx, x, counts, offsets, perm, inv_perm, x_perm, hist,
                      (hipStream_t)stream);
}

// Many-row launch settings: the grid multiple that keeps every workgroup
// within its descriptor registers, and the experts of 257..320 rows on the
// 320 x 192 tiles where the shape allows.
static void set_big(const moe_shape* s, GemmArgs& g, hipStream_t st) {
  const int G = big_grid(st);
  g.grid_mult = (int)plan::big_grid_mult(s->T, s->top_k, s->n_ffn, s->d_model, s->d_ff, G);
  if (plan::ffn_use_r320(s->T, s->top_k, s->n_ffn, s->d_model, s->d_ff, G)) {
    g.r320_lo = plan::kR320Lo;
    g.r320_hi = plan::kR320Hi;
  }
}

int moe_ffn_gate_up(const moe_shape* s, const void* x, const void* x_perm, const int32_t* perm,
                    const int32_t* offsets, const void* w_gate, const void* w_up, void* ws,
                    void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!offsets || !w_gate || !w_up || !ws || (!x_perm && (!x || !perm))) return MOE_EINVAL;
  if (!al4(offsets) || !al16(w_gate) || !al16(w_up) || !al16(ws) || (x_perm && !al16(x_perm)) ||
      (!x_perm && (!al16(x) || !al4(perm))))
    return MOE_EALIGN;
  GemmArgs g{};
  g.a = x_perm ? x_perm : x;
  g.perm = x_perm ? nullptr : perm;
  g.offsets = offsets;
  g.b0 = w_gate;
  g.b1 = w_up;
  g.c = (char*)ws + ws_layout(s).h;
  g.N = s->d_ff;
  g.K = s->d_model;
  g.M = s->T;
  g.ngroups = s->n_ffn;
  g.top_k = s->top_k;
  g.ksplit = 1;
  if (ffn_use_big(s, x_perm == nullptr, (hipStream_t)stream)) {
    set_big(s, g, (hipStream_t)stream);
    return launch_gemm_big(1, g, (hipStream_t)stream);
  }
  return launch_gemm(s->dtype, 1, ffn_big_tiles(s), g, (hipStream_t)stream);
}

int moe_ffn_down(const moe_shape* s, const int32_t* offsets, const void* w_down, void* y_perm,
                 void* ws, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!offsets || !w_down || !y_perm || !ws) return MOE_EINVAL;
  if (!al4(offsets) || !al16(w_down) || !al16(y_perm) || !al16(ws)) return MOE_EALIGN;
  GemmArgs g{};
  g.a = (char*)ws + ws_layout(s).h;
  g.offsets = offsets;
  g.b0 = w_down;
  g.c = y_perm;
  g.N = s->d_model;
  g.K = s->d_ff;
  g.ngroups = s->n_ffn;
  g.top_k = s->top_k;
  g.M = s->T;
  g.ksplit = 1;
  if (ffn_use_big(s, false, (hipStream_t)stream)) {
    set_big(s, g, (hipStream_t)stream);
    return launch_gemm_big(2, g, (hipStream_t)stream);
  }
  return launch_gemm(s->dtype, 2, ffn_big_tiles(s), g, (hipStream_t)stream);
}

int moe_expert_ffn(const moe_shape* s, const void* x, const void* x_perm, const int32_t* perm,
                   const int32_t* offsets, const void* w_gate, const void* w_up,
                   const void* w_down, void* y_perm, void* ws, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!w_down || !y_perm) return MOE_EINVAL;
  if (!al16(w_down) || !al16(y_perm)) return MOE_EALIGN;
  rc = moe_ffn_gate_up(s, x, x_perm, perm, offsets, w_gate, w_up, ws, stream);
  if (rc) return rc;
  return moe_ffn_down(s, offsets, w_down, y_perm, ws, stream);
}

int moe_combine(const moe_shape* s, const void* x, const void* y_perm, const int32_t* topk_idx,
                const float* topk_gate, const int32_t* inv_perm, void* y, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!x || !y_perm || !topk_idx || !topk_gate || !inv_perm || !y) return MOE_EINVAL;
  if (!al16(x) || !al16(y_perm) || !al16(y) || !al4(topk_idx) || !al4(topk_gate) ||
      !al4(inv_perm))
    return MOE_EALIGN;
  return launch_combine(s->dtype, x, y_perm, topk_idx, topk_gate, inv_perm, s->T, s->d_model,
                        s->top_k, s->n_ffn, y, (hipStream_t)stream);
}

int moe_pid_update(const moe_shape* s, const moe_pid_params* pp, const int32_t* counts,
                   moe_pid_state* state, float* bias, float* r_log, int32_t r_log_len,
                   void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!pp || !counts || !state || !bias || (r_log && r_log_len < 0)) return MOE_EINVAL;
  if (!isfinite(pp->setpoint) || !isfinite(pp->kp) || !isfinite(pp->ki) || !isfinite(pp->kd))
    return MOE_ENONFINITE;
  if (!al4(counts) || !al4(state) || !al4(bias) || (r_log && !al4(r_log))) return MOE_EALIGN;
  return launch_pid(counts, s->n_ffn, s->T, pp->setpoint, pp->kp, pp->ki, pp->kd, state, bias,
                    r_log, r_log ? r_log_len : 0, (hipStream_t)stream);
}

int moe_balance_update(const moe_shape* s, float gamma, const int32_t* counts, float* bias,
                       void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!counts || !bias) return MOE_EINVAL;
  if (!isfinite(gamma)) return MOE_ENONFINITE;
  if (gamma < 0.f) return MOE_EINVAL;
  if (!al4(counts) || !al4(bias)) return MOE_EALIGN;
  return launch_balance(counts, s->n_ffn, gamma, bias, (hipStream_t)stream);
}

int moe_eplb_plan(const moe_shape* s, int32_t n_slots, int32_t n_devices, const int32_t* counts,
                  const int32_t* offsets, int32_t* replicas, int32_t* slot_expert,
                  int32_t* slot_rows, int32_t* slot_device, int32_t* device_load, void* stream) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (!counts || !offsets || !replicas || !slot_expert || !slot_rows || !slot_device ||
      !device_load)
    return MOE_EINVAL;
  if (n_devices < 1 || n_slots < s->n_ffn || n_slots % n_devices != 0) return MOE_EINVAL;
  if (n_slots > kEplbMaxSlots || n_devices > kEplbMaxDevices) return MOE_EUNSUPPORTED;
  if (!al4(counts) || !al4(offsets) || !al4(replicas) || !al4(slot_expert) || !al4(slot_rows) ||
      !al4(slot_device) || !al4(device_load))
    return MOE_EALIGN;
  return launch_eplb(counts, offsets, s->n_ffn, n_slots, n_devices, replicas, slot_expert,
                     slot_rows, slot_device, device_load, (hipStream_t)stream);
}

int moe_debug_checks(uint32_t* flags, int clear) {
#ifdef MOE_DEVICE_CHECKS
  if (!flags) return MOE_EINVAL;
  const hipError_t e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    set_hip_error(e);
    return MOE_EHIP;
  }
  unsigned (*const words[])(bool) = {check_word_route, check_word_dispatch, check_word_gemm,
                                     check_word_gemm_big, check_word_combine};
  uint32_t v = 0;
  for (auto* fn : words) {
    const unsigned w = fn(clear != 0);
    if (w == ~0u) return MOE_EHIP;
    v |= w;
  }
  *flags = v;
  return MOE_OK;
#else
  (void)flags;
  (void)clear;
  return MOE_EUNSUPPORTED;
#endif
}

}  // extern "C"
