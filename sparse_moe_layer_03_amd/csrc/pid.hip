// PID step on the router bias, one wave64 (snilld.dk LongCat-2.0 article,
// section "MoE i praksis og prisen for fleksibilitet": a PID controller
// adjusts the router bias so that activation stays in the desired range).
//
// Measured value: r = FFN assignments / T, the mean number of real experts
// per token.  Incremental form: every FFN expert's bias moves by
//   delta = (kp*err + ki*I) + kd*D,   err = setpoint - r,  I += err,
//   D = err - prev_err (0 on the first step).
// Every product and sum is rounded separately (no contraction into FMA), in
// this order.  The count sum is an integer reduction, so r is exact up to
// one division.

#include <math.h>

#include "common.h"
#include "internal.h"

// Device code is compiled with FP contraction on, and HIP's __fmul_rn /
// __fadd_rn are plain operators defined in a header (their operations carry
// the header's contraction setting into any caller): the compiler fused
// kp*err + ki*I into one FMA (one rounding instead of two).  So this file
// turns contraction off and writes every operation as a plain operator.
#pragma clang fp contract(off)

namespace moe {

__global__ void __launch_bounds__(64)
pid_kernel(const int32_t* __restrict__ counts, int n_ffn, int T, float setpoint, float kp,
           float ki, float kd, moe_pid_state* __restrict__ state, float* __restrict__ bias,
           float* __restrict__ r_log, int r_log_len) {
  const int lane = threadIdx.x;
  int a = 0;
  for (int e = lane; e < n_ffn; e += 64) a += counts[e];
  a = wave_sum_i(a);
  const float integral = state->integral, prev = state->prev_err;
  const int step = state->step;
  if (!isfinite(integral) || !isfinite(prev)) {
    if (lane == 0) state->flags |= 1;
    return;
  }
  const float r = (float)a / (float)T;
  const float err = setpoint - r;
  const float I = integral + err;
  const float D = (step == 0) ? 0.f : err - prev;
  const float p_term = kp * err, i_term = ki * I, d_term = kd * D;
  const float delta = (p_term + i_term) + d_term;
  for (int e = lane; e < n_ffn; e += 64) bias[e] = bias[e] + delta;
  if (lane == 0) {
    if (r_log != nullptr && step >= 0 && step < r_log_len) r_log[step] = r;
    state->integral = I;
    state->prev_err = err;
    state->step = step + 1;
  }
}

int launch_pid(const int32_t* counts, int n_ffn, int T, float setpoint, float kp, float ki,
               float kd, moe_pid_state* state, float* bias, float* r_log, int r_log_len,
               hipStream_t st) {
  hipLaunchKernelGGL(pid_kernel, dim3(1), dim3(64), 0, st, counts, n_ffn, T, setpoint, kp, ki,
                     kd, state, bias, r_log, r_log_len);
  return check_launch();
}

}  // namespace moe

namespace moe {

// Per-expert load balancing on the router bias, one wave64 (LongCat-2.0
// Ascend deployment article, section "MoE专家动态负载均衡": dynamic load
// balancing narrows the gap between the tokens experts receive).
// With A = sum_{e<N} counts[e] and s_e = sign(A - N * counts[e]) (+1 for an
// under-loaded expert), every FFN expert's bias moves by
//   delta_e = gamma * ((N * s_e - S) / N),   S = sum_e s_e,
// a zero-sum step: the mean FFN bias, which the PID steers, is unchanged.
// Integer sums are exact; one rounding for the division, one for the product.
__global__ void __launch_bounds__(64)
balance_kernel(const int32_t* __restrict__ counts, int n_ffn, float gamma,
               float* __restrict__ bias) {
  const int lane = threadIdx.x;
  int a = 0;
  for (int e = lane; e < n_ffn; e += 64) a += counts[e];
  a = wave_sum_i(a);
  int ssum = 0;
  for (int e = lane; e < n_ffn; e += 64) {
    const long d = (long)a - (long)n_ffn * counts[e];
    ssum += (d > 0) - (d < 0);
  }
  ssum = wave_sum_i(ssum);
  for (int e = lane; e < n_ffn; e += 64) {
    const long d = (long)a - (long)n_ffn * counts[e];
    const int s = (d > 0) - (d < 0);
    const float frac = (float)(n_ffn * s - ssum) / (float)n_ffn;
    const float step = gamma * frac;
    bias[e] = bias[e] + step;
  }
}

int launch_balance(const int32_t* counts, int n_ffn, float gamma, float* bias, hipStream_t st) {
  hipLaunchKernelGGL(balance_kernel, dim3(1), dim3(64), 0, st, counts, n_ffn, gamma, bias);
  return check_launch();
}

}  // namespace moe
