// Host-side interface between the C ABI (gdn_api.cpp) and the kernel
// launchers (*.hip).  Arguments here have already been validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

struct ConvParams {
  const void* x;
  const void* weight;
  const void* bias;
  void* y;
  void* conv_state;
  const int32_t* cu_seqlens;  // nullptr: one sequence
  int64_t total_tokens;
  int32_t n_seqs;
  int32_t channels;
  int32_t width;
  int32_t act;
  int32_t* conv_head;  // [n_seqs] ring heads of conv_state, or null (chronological)
};
hipError_t launch_conv1d(const ConvParams& p, int dtype, hipStream_t stream);

struct DecodeParams {
  const void* x;
  const void* conv_weight;  // nullptr: x already holds q|k|v
  const void* conv_bias;
  void* conv_state;
  const float* g;
  const float* beta;
  void* state;
  void* o;
  int32_t n_seqs;
  int32_t h_qk;
  int32_t h_v;
  int32_t width;
  int32_t act;
  int32_t l2norm;
  float scale;
  int32_t erase;  // 0: erase-off variant, S_t = a_t S_{t-1} + b_t v_t k_t^T
  const int32_t* state_idx;  // [n_seqs] state and conv-state slots, or null (slot n)
  int32_t* conv_head;        // ring heads of the conv-state pool, or null (chronological)
};
hipError_t launch_decode(const DecodeParams& p, int io_dtype, int state_dtype, int d,
                         hipStream_t stream);

struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_stride;
  int64_t k_stride;
  int64_t v_stride;
  const float* g;
  const float* beta;
  const void* initial_state;  // fp32 or bf16 (state_bf16)
  void* final_state;
  void* o;
  const int32_t* cu_seqlens;
  int64_t total_tokens;
  int32_t n_seqs;
  int32_t h_qk;
  int32_t h_v;
  int32_t chunk;
  int32_t l2norm;
  float scale;
  void* workspace;
  size_t workspace_bytes;
  int32_t erase;  // 0: erase-off variant (A = 0, U = diag(beta) V)
  int32_t emit_every;        // > 0: the state after every emit_every-th whole chunk
  void* chunk_states;        // [rows, h_v, d_v, d_k] (rows from the plan)
  const int32_t* state_idx;  // [n_seqs] state slots, or null (slot n)
  int32_t state_bf16;        // initial/final/chunk states stored as bf16 (else fp32)
};
// Workspace of gdn_prefill: chunk offsets plus, per (chunk, V head), the
// chunk operands Tb, P and four per-token scalar rows.
size_t prefill_workspace_bytes(int io_dtype, int64_t total_tokens, int n_seqs, int h_v, int d, int chunk,
                               int emit_every);
bool prefill_supported(int io_dtype, int d, int chunk);
hipError_t launch_prefill(const PrefillParams& p, int io_dtype, int d, hipStream_t stream);
// bf16 io at chunk 32 or 64 with n_seqs <= kNoAllocMaxSeqs: the fused kernel
// with its plan arrays in a static per-device array (p.workspace ignored)
constexpr int kNoAllocMaxSeqs = 8192;
hipError_t launch_prefill_noalloc(const PrefillParams& p, int d, hipStream_t stream);

struct PrefillBwdParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_stride;
  int64_t k_stride;
  int64_t v_stride;
  const float* g;
  const float* beta;
  const float* initial_state;
  const int32_t* cu_seqlens;
  const void* d_o;
  const float* d_final_state;
  void* dq;
  void* dk;
  void* dv;
  int64_t dq_stride;
  int64_t dk_stride;
  int64_t dv_stride;
  float* dg;
  float* dbeta;
  float* d_initial_state;
  int64_t total_tokens;
  int32_t n_seqs;
  int32_t h_qk;
  int32_t h_v;
  int32_t chunk;
  int32_t l2norm;
  int32_t erase;
  float scale;
  void* workspace;
};
// Workspace of gdn_prefill_backward: every chunk's intermediates, or, for one
// sequence past the budget (2 GiB; GDN_BWD_BUDGET_MB), one window's plus the
// window-start states
size_t prefill_backward_workspace_bytes(int io_dtype, int64_t total_tokens, int n_seqs, int h_qk, int h_v, int d,
                                        int chunk);
hipError_t launch_prefill_backward(const PrefillBwdParams& p, int io_dtype, int d, hipStream_t stream);

struct ConvBwdParams {
  const void* x;
  const void* weight;
  const void* bias;
  const void* conv_state;
  const int32_t* cu_seqlens;
  const void* dy;
  const float* d_new_state;
  void* dx;
  float* dweight;
  float* dbias;
  float* d_conv_state;
  int64_t total_tokens;
  int32_t n_seqs;
  int32_t channels;
  int32_t width;
  int32_t act;
  void* workspace;
};
size_t conv1d_backward_workspace_bytes(int64_t total_tokens, int channels);
hipError_t launch_conv1d_backward(const ConvBwdParams& p, int dtype, hipStream_t stream);

}  // namespace gdn
