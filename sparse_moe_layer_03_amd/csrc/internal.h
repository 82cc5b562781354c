// Internal host-side interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

struct GemmArgs {
  const void* a;           // token rows: x (router, gate/up) or H (down)
  const int32_t* perm;     // gate/up: gather rows x[perm[p] / top_k]; else null
  const int32_t* offsets;  // group row offsets [ngroups + 1] (gate/up, down)
  const void* b0;          // W_router | W_gate | W_down
  const void* b1;          // W_up (gate/up only)
  void* c;                 // logits fp32 [M, N] | H [rows, N] | y_perm [rows, N]
  const float* col_bias;   // router: per-column logit offset [N] or null
  int M;                   // router: T (grouped modes use offsets)
  int N;                   // output columns: E | d_ff | d_model
  int K;                   // reduction length: d_model | d_model | d_ff
  int ngroups;             // experts (grouped modes)
  int top_k;
  int ksplit;              // router: K is split into this many partial sums
  int r320_lo, r320_hi;    // many-row expert modes: groups of r320_lo..r320_hi
                           // rows run on 320 x 192 tiles (r320_hi 0: none)
  int grid_mult;           // many-row expert modes: launch big_grid() times this
                           // many workgroups (plan::big_grid_mult; 0 or 1: one
                           // per CU)
};

// mode: 0 router, 1 gate/up + SwiGLU, 2 down.  big: 128x128 tiles, else
// 16-row tiles for few rows per expert.
int launch_gemm(int dtype, int mode, int big, const GemmArgs& g, hipStream_t st);

// bf16 gate/up (mode 1) or down (mode 2) with 256x256 direct-to-LDS tiles,
// and 320x192 tiles for the groups of r320_lo..r320_hi rows (K a multiple of
// 128, at most 1024 groups, at most 256 tiles per workgroup of the
// big_grid() * grid_mult launched: plan::ffn_use_big, plan::big_grid_mult,
// plan::ffn_use_r320); mode 0: the router GEMM.
constexpr int kBigTileRows = 256;
int launch_gemm_big(int mode, const GemmArgs& g, hipStream_t st);
// Workgroups of a many-row launch on stream st (one per CU it may use).
int big_grid(hipStream_t st);

// partials: nsplit slices of [T, E] fp32 summed in slice order, plus
// col_bias (nullable); logits_out (nullable) receives the sum.
int launch_topk(const float* partials, int nsplit, const float* col_bias, float* logits_out,
                const float* bias, int T, int E, int k, float scaling, int32_t* idx, float* gate,
                hipStream_t st);

// Router GEMM + top-k in one launch (bf16, at most 128 experts, d_model a
// multiple of 1024).
bool router_topk_fused_ok(int T, int E, int d_model, int dtype);
// Workspace bytes of the router matrix repacked for that kernel.
size_t router_packed_bytes(int E, int d_model);
int launch_router_topk(const void* x, const void* wr, void* wr_packed, const float* col_bias,
                       float* logits_out,
                       const float* bias, int T, int E, int d, int k, float scaling,
                       int32_t* idx, float* gate, hipStream_t st);

// K split of the router GEMM for a shape (depends on the shape only).
int router_ksplit(int T, int E, int d_model, int dtype);

int launch_dispatch(const int32_t* idx, int Tk, int E, int nb, int32_t* block_hist,
                    int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                    hipStream_t st);

int launch_gather(int dtype, const void* x, const int32_t* perm, const int32_t* offsets,
                  int n_ffn, int Tk, int k, int d, void* x_perm, hipStream_t st);

int launch_combine(int dtype, const void* x, const void* y_perm, const int32_t* idx,
                   const float* gate, const int32_t* inv_perm, int T, int d, int k,
                   int n_ffn, void* y, hipStream_t st);

int launch_pid(const int32_t* counts, int n_ffn, int T, float setpoint, float kp, float ki,
               float kd, moe_pid_state* state, float* bias, float* r_log, int r_log_len,
               hipStream_t st);

int launch_balance(const int32_t* counts, int n_ffn, float gamma, float* bias, hipStream_t st);

// Expert placement over an EP domain: at most 4096 slots on at most 64
// devices (one workgroup; slot keys sorted in 32 KiB of LDS).
constexpr int kEplbMaxSlots = 4096;
constexpr int kEplbMaxDevices = 64;
int launch_eplb(const int32_t* counts, const int32_t* offsets, int n_ffn, int n_slots,
                int n_devices, int32_t* replicas, int32_t* slot_expert, int32_t* slot_rows,
                int32_t* slot_device, int32_t* device_load, hipStream_t st);

int device_cu_count();
int stream_cu_count(hipStream_t st);
int check_launch();
// Records a HIP error for moe_strerror (this thread).
void set_hip_error(hipError_t e);

// Device-check words of the kernels' translation units (debug build; 0 in
// release builds, ~0u on a HIP failure), cleared after reading if `clear`.
unsigned check_word_route(bool clear);
unsigned check_word_dispatch(bool clear);
unsigned check_word_gemm(bool clear);
unsigned check_word_gemm_big(bool clear);
unsigned check_word_combine(bool clear);

// moe_dispatch's argument checks (no workspace) and its launches with the
// per-block histogram `hist` ([E, dispatch_blocks(T*k)] int32).
int dispatch_checks(const moe_shape* s, const int32_t* topk_idx, const void* x, int32_t* counts,
                    int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* x_perm);
int dispatch_run(const moe_shape* s, const int32_t* topk_idx, const void* x, int32_t* counts,
                 int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* x_perm, int32_t* hist,
                 hipStream_t st);

// Number of blocks the dispatch kernels split T*k assignments into.
inline int dispatch_blocks(long Tk) {
  long nb = (Tk + 1023) / 1024;
  if (nb < 1) nb = 1;
  if (nb > 256) nb = 256;
  return (int)nb;
}

}  // namespace moe
