// Host-side launch interfaces between the C ABI (gdn_api.hip) and the kernel
// files.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdn {

struct DecodeArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  const float* state_in;
  float* state_out;
  void* out;
  int B, H, Dk, Dv;
  bool bf16, out_bf16;
  float scale;
  void* stream;
  bool chgate = false;  // alpha is [B, H, Dk]: channel-wise gate
  bool kgla = false;    // with chgate: key-dependent gate, no erase, write k v^T
};

struct PrefillArgs {
  const void *q, *k, *v;
  const float *alpha, *beta;
  const float* state_in;
  float* state_out;
  void* out;
  int B, T, H, Dk, Dv, chunk;
  bool bf16, out_bf16;
  float scale;
  void* workspace;
  void* stream;
  // Tokens between the starts of consecutive sequences in q, k, v, out,
  // alpha and beta (0 = T: dense [B, T, ...]).  Only the per-head kernels
  // (bf16, Dk = Dv = 128, chunk 64) take another value.
  int seq_stride = 0;
  // Channel-gate kernels only: gated linear attention with a key-dependent
  // gate (no erase, gate alpha o (1 - beta k o k), write k v^T).
  bool kgla = false;
  // Per-head kernels only: q, k, v are the raw projections, and the causal
  // short convolution (4 taps, zero history before token 0) + SiLU, with the
  // L2 normalisation of q and k, runs in the kernels' tile loads.  taps_*
  // [H * Dk][4] f32; all three or none.
  const float *taps_q = nullptr, *taps_k = nullptr, *taps_v = nullptr;
  float conv_eps = 0.f;
};

struct ConvArgs {
  const void* x;
  const float* taps;
  void* y;
  int B, T, Ch, K, group;
  float eps;
  bool bf16, out_bf16;
  void* stream;
};

struct SwaArgs {
  const void* q;
  const void *k_new, *v_new;
  void *k_cache, *v_cache;
  const int* n_tokens;
  int B, H, D, n_sink, window;
  float softmax_scale;
  int accumulate;
  void* out;
  bool bf16, out_bf16;
  void* stream;
};

// Per-chunk workspace layout of the prefill (one record per (b, h, chunk)):
//   Tm    [C][C]  operand type: (I + A)^-1 of the chunk (unit lower)
//   Pm    [C][C]  operand type: scale * exp(g_r - g_i) q_r.k_i for i <= r, else 0
//   gam   [C]     f32: cumulative log gate within the chunk
// Records are padded to 256 bytes.
size_t prefill_record_bytes(int chunk, bool bf16);
// Workspace of the prefill for these sizes: per-chunk records of the
// two-kernel form, or the segment maps of the per-head kernels (0 when they
// run in one pass).
size_t prefill_workspace_bytes(int B, int T, int H, int Dk, int Dv, int chunk, bool bf16);
// Per-head kernels: bf16 inputs, Dk = Dv = 128, chunk 64, T > 0.  Long
// sequences of few heads are split into P segments: segment 0 of L0 chunks,
// the others of L (the last may be shorter); P = 1: one pass, no workspace.
bool prefill_head_supported(const PrefillArgs& p);
// ... and with the fused short convolution (dense sequences only).
bool prefill_head_conv_supported(const PrefillArgs& p);
void prefill_head_segments(int B, int T, int H, int* P, int* L0, int* L);
size_t prefill_head_workspace_bytes(int B, int T, int H);
hipError_t launch_prefill_head(const PrefillArgs& p);

hipError_t launch_decode(const DecodeArgs& p);
hipError_t launch_prefill(const PrefillArgs& p);
hipError_t launch_conv(const ConvArgs& p);
// One decode step (T unused): state [B][K-1][Ch] of the input dtype, in place.
hipError_t launch_conv_step(const ConvArgs& p, void* state);
hipError_t launch_swa(const SwaArgs& p);

// Backward of the scalar-gate recurrence: gradients of q, k, v, alpha, beta
// and the initial state for an output gradient (and optional final-state
// gradient); f32 gradients; Dk, Dv in {16, 32, 64, 128}.
struct BwdArgs {
  const void *q, *k, *v;
  const float *alpha, *beta, *state_in, *dout, *dstate_out;
  float *dq, *dk, *dv, *dalpha, *dbeta, *dstate_in;
  int B, T, H, Dk, Dv;
  bool bf16;
  float scale;
  void* workspace;
  void* stream;
};
size_t backward_workspace_bytes(int B, int T, int H, int Dk, int Dv);
hipError_t launch_backward(const BwdArgs& p);
// Chunked form (Dk = Dv = 128, chunks of 64 tokens, f32 MFMA): the path
// launch_backward takes for those head sizes.
bool backward_chunked_supported(int Dk, int Dv);
size_t backward_chunked_workspace_bytes(int B, int T, int H);
hipError_t launch_backward_chunked(const BwdArgs& p);

// Channel-wise gate prefill (alpha [B, T, H, Dk]); chunks of 32 tokens,
// f32 arithmetic; Dk in {32, 64, 128}, Dv a multiple of 32.  With p.kgla:
// gated linear attention with a key-dependent gate, same workspace.
size_t prefill_chgate_workspace_bytes(int B, int T, int H);
hipError_t launch_prefill_chgate(const PrefillArgs& p);

// Sink + window softmax over a whole sequence: bf16 q, k, v [B, T, H, 128];
// rows t >= acc_from add into out, rows below are written.
struct SwaPrefillArgs {
  const void *q, *k, *v;
  void* out;
  int B, T, H, n_sink, window, acc_from;
  float softmax_scale;
  bool out_bf16;
  void* stream;
};
hipError_t launch_swa_prefill(const SwaPrefillArgs& p);

// Decode-cache fill from a sequence's keys and values.
struct SwaCacheFillArgs {
  const void *k, *v;
  void *k_cache, *v_cache;
  int B, T, H, D, n_sink, window;
  bool bf16;
  void* stream;
};
hipError_t launch_swa_cache_fill(const SwaCacheFillArgs& p);

}  // namespace gdn
