/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse MoE layer library.
 *
 * One LongCat-2.0-style mixture-of-experts layer forward pass:
 *   route -> dispatch -> expert FFN -> combine, and a PID step on the router
 *   bias between batches.
 *
 * Sources (web pages on LongCat-2.0, cited by title and section):
 *   [DS] "LongCat-2.0" model data sheet (archdb), table "Mixture of experts":
 *        one router classifier scores N routed FFN experts plus Z identity
 *        ("zero") experts, an e_score_correction_bias, experts per token,
 *        expert width, routed scaling factor.
 *   [SN] "Meituan lancerer LongCat-2.0: 1,6T MoE-model med million-token
 *        hukommelse" (snilld.dk), section "MoE i praksis og prisen for
 *        fleksibilitet": zero-computation experts and a PID controller on the
 *        router bias that keeps the activation in range.
 *   [AS] Ascend deployment article on LongCat-2.0 (10100.com), section
 *        "底层定制算子深度优化": Dispatch/Combine operators that support
 *        zero-computation experts.
 *   [MD] "2026 Analysis of LongCat-2.0 Technical Principles" (macdate.com),
 *        section 1: soft-max gated top-k routing.
 *
 * Conventions shared by every call
 *   - Expert ids 0..n_ffn-1 are SwiGLU FFN experts; n_ffn..E-1 (E = n_ffn +
 *     n_zero) are identity experts ([DS]: "768 + 128").
 *   - Pointers other than `shape` and `pid_params` are DEVICE pointers owned
 *     by the caller, 16-byte aligned.  The library never allocates, frees or
 *     keeps them after the call returns.  Scratch comes from `ws`, a device
 *     buffer of at least moe_workspace_bytes(shape) bytes.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work; results are valid once the stream has reached them.  No
 *     call synchronises the host.
 *   - Row-major layouts.  x, y: [T, d_model].  W_router: [E, d_model].
 *     W_gate, W_up: [n_ffn, d_ff, d_model].  W_down: [n_ffn, d_model, d_ff]
 *     (the reduction dimension is contiguous in every weight).
 *   - x, weights, x_perm, y_perm and y share one element type (`dtype`):
 *     bf16 or fp32.  Routing scores, biases, gates and the PID are fp32.
 *   - Return value: MOE_OK (0) or a negative moe_status.  Arguments are
 *     checked on the host before anything is enqueued; on error nothing is
 *     enqueued.  Kernels trust the routing arrays produced by these calls.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,        /* null required pointer, or a size out of range */
  MOE_EUNSUPPORTED = -2,  /* valid but outside the library's limits (below) */
  MOE_EHIP = -3,          /* a HIP launch or query failed                  */
  MOE_ENONFINITE = -4,    /* non-finite host-side parameter                */
  MOE_EALIGN = -5         /* a pointer is not 16-byte aligned              */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Layer shape; field names follow the config keys [DS] lists
 * (hidden_size, n_routed_experts, zero_expert_num, expert_ffn_hidden_size,
 * moe_topk, routed_scaling_factor).
 * Limits: T >= 1; n_ffn >= 1; n_zero >= 0; E = n_ffn + n_zero <= 1024;
 * 1 <= top_k <= min(E, 16); d_model and d_ff positive multiples of 64;
 * T * top_k < 2^31; routed_scaling finite. */
typedef struct {
  int32_t T;              /* tokens in the batch                          */
  int32_t d_model;        /* hidden size                                  */
  int32_t n_ffn;          /* routed SwiGLU FFN experts (N)                */
  int32_t n_zero;         /* identity zero-computation experts (Z)        */
  int32_t d_ff;           /* expert intermediate width                    */
  int32_t top_k;          /* experts selected per token (k)               */
  int32_t dtype;          /* moe_dtype of activations and weights         */
  float routed_scaling;   /* multiplies every gate ([DS] routed scaling)  */
} moe_shape;

/* PID gains and set point (host struct, copied into the launch). */
typedef struct {
  float setpoint;  /* target mean number of FFN experts per token */
  float kp, ki, kd;
} moe_pid_params;

/* PID memory; lives in DEVICE memory, caller-owned, zero-initialised before
 * the first update.  flags bit 0 is set by the device when it finds a
 * non-finite integral or previous error; that update is then skipped. */
typedef struct {
  float integral;
  float prev_err;
  int32_t step;
  int32_t flags;
} moe_pid_state;

/* Bytes of device scratch `ws` that the calls below need for `shape` on the
 * current device (the router's K-split count, and with it the size, can
 * depend on the device's multiprocessor count).  Returns 0 if the shape is
 * invalid. */
size_t moe_workspace_bytes(const moe_shape* shape);

/* Text for a status code (static storage). */
const char* moe_strerror(int status);

/* Multiprocessor count of the current device as seen by the library
 * (>0), or a negative moe_status.  Used to size persistent launches. */
int moe_device_cu_count(void);

/* moe_route -- router classifier, softmax, biased top-k and gates.
 * [DS] "Mixture of experts": one classifier scores FFN + zero experts, with
 * e_score_correction_bias and top-k; [MD] section 1: soft-max gating.
 *   logits[t,e] = sum_i x[t,i] W_router[e,i] + logit_bias[e]   (fp32 accum)
 *   p[t,:]      = softmax(logits[t,:]) over all E experts
 *   key[t,e]    = p[t,e] + bias[e]                               (fp32)
 *   topk_idx[t,:]  = the top_k experts by key (ties -> lower id), written in
 *                    ascending expert id                    [T, top_k] int32
 *   topk_gate[t,j] = routed_scaling * p[t, topk_idx[t,j]]  [T, top_k] fp32
 * The bias only steers selection; gates use the unbiased score and are not
 * renormalised.
 *   x [T, d_model] dtype; w_router [E, d_model] dtype;
 *   logit_bias [E] fp32 or NULL (plain classifier offset);
 *   bias [E] fp32 (+-inf allowed: always / never selected);
 *   logits_out [T, E] fp32 or NULL (written when given);
 *   ws: workspace (required; holds the K-split partial logits of the
 *       two-kernel path; with at most 128 experts in bf16 the GEMM and the
 *       selection run in one kernel, and ws holds a copy of w_router
 *       repacked for it, rewritten on every call). */
int moe_route(const moe_shape* shape, const void* x, const void* w_router,
              const float* logit_bias, const float* bias, int32_t* topk_idx,
              float* topk_gate, float* logits_out, void* ws, void* stream);

/* moe_dispatch -- group the T*top_k assignments by expert ([AS] Dispatch
 * operator with zero-computation experts).  Assignment a = t*top_k + j.
 *   counts [E] int32: assignments per expert;
 *   offsets [E+1] int32: exclusive prefix sum, offsets[E] = T*top_k;
 *   perm [T*top_k] int32: perm[p] = assignment at sorted position p, sorted
 *        by (expert, a) -- a stable counting sort, deterministic;
 *   inv_perm [T*top_k] int32: inverse of perm;
 *   x_perm [T*top_k, d_model] dtype or NULL: when given, rows p <
 *        offsets[n_ffn] receive x[perm[p] / top_k] (identity-expert rows are
 *        never gathered).  NULL lets moe_expert_ffn read x through perm. */
int moe_dispatch(const moe_shape* shape, const int32_t* topk_idx,
                 const void* x, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* inv_perm, void* x_perm, void* ws,
                 void* stream);

/* moe_dispatch_noalloc -- moe_dispatch for callers that cannot allocate
 * device memory or hand over a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments
 * (minus ws), kernels and results as moe_dispatch.  Its scratch -- the
 * per-block expert histogram, E * ceil(T*top_k / 1024) int32 (blocks capped
 * at 256), at most 1 MiB -- is a static device array of the library, one
 * per device, held until the process ends; it needs no clearing.  Every
 * call on a device shares that device's array, so calls that overlap on one
 * device (two streams or threads) race on it: serialise them.  A shape whose
 * histogram exceeds 1 MiB returns MOE_EUNSUPPORTED (none within the limits
 * above does).  Allocates nothing: no hipMalloc, no hipFree. */
int moe_dispatch_noalloc(const moe_shape* shape, const int32_t* topk_idx,
                         const void* x, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* inv_perm, void* x_perm,
                         void* stream);

/* moe_expert_ffn -- every FFN expert e < n_ffn on its rows
 * [offsets[e], offsets[e+1]) ([DS] expert width; activation read as SwiGLU):
 *   H = silu(X W_gate[e]^T) * (X W_up[e]^T),  y_perm rows = H W_down[e]^T,
 *   silu(z) = z / (1 + exp(-z)), fp32 accumulation, H rounded to dtype.
 * X rows come from x_perm when it is non-NULL, else from x[perm[p]/top_k].
 *   y_perm [T*top_k, d_model] dtype: rows p < offsets[n_ffn] written.
 * Equals moe_ffn_gate_up followed by moe_ffn_down. */
int moe_expert_ffn(const moe_shape* shape, const void* x, const void* x_perm,
                   const int32_t* perm, const int32_t* offsets,
                   const void* w_gate, const void* w_up, const void* w_down,
                   void* y_perm, void* ws, void* stream);

/* moe_ffn_gate_up -- first half of moe_expert_ffn: writes
 * H = silu(X Wg^T) * (X Wu^T) into the workspace (rows p < offsets[n_ffn]). */
int moe_ffn_gate_up(const moe_shape* shape, const void* x, const void* x_perm,
                    const int32_t* perm, const int32_t* offsets,
                    const void* w_gate, const void* w_up, void* ws,
                    void* stream);

/* moe_ffn_down -- second half of moe_expert_ffn: y_perm rows = H Wd^T, with
 * H read from the workspace written by moe_ffn_gate_up. */
int moe_ffn_down(const moe_shape* shape, const int32_t* offsets,
                 const void* w_down, void* y_perm, void* ws, void* stream);

/* moe_combine -- gate-weighted sum back in token order ([AS] Combine with
 * zero-computation experts; [SN] identity experts as a lightweight path):
 *   y[t] = sum_{j: idx<n_ffn} gate[t,j] * y_perm[inv_perm[t*top_k+j]]
 *        + (sum_{j: idx>=n_ffn} gate[t,j]) * x[t]
 * accumulated in fp32 in slot order, rounded once to dtype.  Identity
 * experts cost a scaled add of x, never a GEMM.  y [T, d_model] dtype. */
int moe_combine(const moe_shape* shape, const void* x, const void* y_perm,
                const int32_t* topk_idx, const float* topk_gate,
                const int32_t* inv_perm, void* y, void* stream);

/* moe_pid_update -- one PID step on the router bias ([SN]: a PID
 * controller adjusts the router bias to keep activation in range):
 *   r = (sum_{e<n_ffn} counts[e]) / T      mean FFN experts per token
 *   err = setpoint - r;  I += err;  D = err - prev_err (0 on step 0)
 *   delta = (kp*err + ki*I) + kd*D         fp32, no fused multiply-add
 *   bias[e] += delta for e < n_ffn;  prev_err = err;  step += 1
 *   r_log[step] = r when r_log != NULL and step < r_log_len.
 *   counts [E] int32 (from moe_dispatch); state: device moe_pid_state;
 *   bias [E] fp32 updated in place.  Non-finite params -> MOE_ENONFINITE. */
int moe_pid_update(const moe_shape* shape, const moe_pid_params* pid_params,
                   const int32_t* counts, moe_pid_state* state, float* bias,
                   float* r_log, int32_t r_log_len, void* stream);

/* moe_balance_update -- per-expert load balancing on the router bias
 * (Ascend deployment article, section "MoE专家动态负载均衡": token loads per
 * expert vary widely and dynamic balancing narrows the gap; the method is
 * not given -- this is a zero-sum sign step):
 *   A = sum_{e<n_ffn} counts[e];  s_e = sign(A - n_ffn * counts[e])
 *   S = sum_{e<n_ffn} s_e;   bias[e] += gamma * ((n_ffn * s_e - S) / n_ffn)
 * for e < n_ffn (fp32, one rounding for the division and one for the
 * product); identity experts untouched.  Over-loaded experts move down,
 * under-loaded ones up, and the mean FFN bias (the PID's lever) is
 * unchanged.  counts [E] int32 (from moe_dispatch); bias [E] fp32 in place.
 * gamma >= 0 and finite (else MOE_EINVAL / MOE_ENONFINITE). */
int moe_balance_update(const moe_shape* shape, float gamma, const int32_t* counts,
                       float* bias, void* stream);

/* moe_eplb_plan -- expert placement balancing over an expert-parallel
 * domain (Ascend deployment article, section "MoE专家动态负载均衡": with a
 * very large EP domain the tokens each expert receives vary widely, and
 * dynamic load balancing narrows the gap between experts' loads).  Routing
 * is untouched: the plan says where FFN experts' rows are computed.
 * The n_ffn experts occupy n_slots expert slots on n_devices devices
 * (n_slots / n_devices each):
 *   replicas[e] >= 1, sum = n_slots: each redundant slot goes, one at a
 *     time, to the expert with the most tokens per replica (largest
 *     counts[e] / replicas[e], exact; ties to the lower id);
 *   slots in expert order: slot_expert[s]; replica j of expert e (c rows,
 *     r replicas) takes sorted positions slot_rows[2s] .. slot_rows[2s+1]
 *     = offsets[e] + j*c/r .. offsets[e] + (j+1)*c/r (integer division);
 *   slot_device[s]: longest first (slot loads descending, ties to the lower
 *     slot), each to the least-loaded device with room (ties to the lower
 *     device); device_load[d] = rows placed on device d.
 *   counts [>= n_ffn] int32, offsets [>= n_ffn + 1] int32 (moe_dispatch);
 *   replicas [n_ffn], slot_expert [n_slots], slot_rows [n_slots, 2],
 *   slot_device [n_slots], device_load [n_devices]: int32 outputs.
 * Limits: n_ffn <= n_slots <= 4096, 1 <= n_devices <= 64, n_devices divides
 * n_slots (else MOE_EINVAL / MOE_EUNSUPPORTED).  One workgroup. */
int moe_eplb_plan(const moe_shape* shape, int32_t n_slots, int32_t n_devices,
                  const int32_t* counts, const int32_t* offsets, int32_t* replicas,
                  int32_t* slot_expert, int32_t* slot_rows, int32_t* slot_device,
                  int32_t* device_load, void* stream);

/* moe_debug_checks -- the device-side index-range checks of the debug build.
 * For callers debugging the library, not part of the layer: the library
 * built with these checks (libmoe_mi355x_checks.so, same entry points) has
 * every kernel test the index ranges it relies on; a failed check sets its
 * bit below on the device that ran the kernel and the kernel continues with
 * the access guarded, as the release build guards it.  This call waits for
 * the current device (hipDeviceSynchronize), stores the OR of the bits set
 * there since the last clearing call in *flags, and clears them if
 * clear != 0.  Release builds: MOE_EUNSUPPORTED, *flags untouched.
 * NULL flags: MOE_EINVAL; a HIP failure: MOE_EHIP. */
#define MOE_CHECK_ROUTE_ID     (1u << 0) /* top-k wrote an expert id outside [0, E) */
#define MOE_CHECK_DISPATCH_ID  (1u << 1) /* topk_idx given to dispatch outside [0, E) */
#define MOE_CHECK_DISPATCH_POS (1u << 2) /* dispatch computed a position outside [0, T*k) */
#define MOE_CHECK_GEMM_ROW     (1u << 3) /* expert GEMM: gathered token outside [0, T) */
#define MOE_CHECK_GEMM_ITEMS   (1u << 4) /* expert GEMM: a workgroup got more work items
                                            than it can track */
#define MOE_CHECK_GEMM_TILE    (1u << 5) /* expert GEMM: a tile outside its expert's rows
                                            or the output columns */
#define MOE_CHECK_COMBINE_ROW  (1u << 6) /* combine: a slot's y_perm row outside [0, T*k) */
int moe_debug_checks(uint32_t* flags, int clear);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
