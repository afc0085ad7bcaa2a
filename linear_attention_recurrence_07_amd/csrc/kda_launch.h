// Host-side launchers of the KDA kernels (internal to libkda.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

// The short convolution fused in front of the recurrence (q, k, v in that order): taps
// [H * d, W] fp32, carried inputs [N, W-1, H * d] in the input dtype (or null: zeros) and
// the carried inputs after the call (or null).  W = 0: no convolution.
struct ConvIn {
  const float *w[3];
  const void *init[3];
  void *fin[3];
  int W, silu;
};

// Arguments of one prefill or recurrent call after host validation.
struct Args {
  const void *q, *k, *v;
  const float *g, *beta;
  const float *init;          // prefill: initial state or null
  float *state;               // recurrent: in/out state; prefill: final state
  const int32_t *cu;          // packed offsets or null
  const uint8_t *mask;        // padding mask or null
  void *o;
  const void *gate;
  const float *norm_w;
  void *y;
  int B, T, H, dk, dv, N;
  float scale, eps;
  int use_l2;
  int in_bf16, out_bf16;
  int g_head;                 // g is [B, T, H] (one decay per head), not [B, T, H, dk]
  float *states_out;          // recurrent: the state after every token [B, T, H, dk, dv], or null
  ConvIn conv;                // q, k, v arrive as raw projections when conv.W > 0
};

// Arguments of one short-convolution call after host validation.
struct ConvArgs {
  const void *x;
  const float *w;             // [D, W]
  const void *init;           // [N, W-1, D] or null
  const int32_t *cu;
  const uint8_t *mask;
  void *y;
  void *fin;                  // [N, W-1, D] or null
  int B, T, D, N, W, silu;
  int in_bf16, out_bf16;
};

hipError_t launch_recurrent(const Args &a, hipStream_t s);
hipError_t launch_short_conv(const ConvArgs &a, hipStream_t s);
// The carried inputs after a call for each of q, k and v whose a.conv.fin is set: the
// last W-1 inputs of every sequence (padding skipped), as kda_short_conv leaves them.
// Runs after every kernel of the call that reads a.conv.init (they may be one buffer).
hipError_t launch_conv_carry(const Args &a, hipStream_t s);
// Output projection out[M, N] = x[M, K] W[N, K]^T, bf16 operands, fp32 accumulation.
bool out_proj_supports(int64_t M, int K, int N);
size_t out_proj_workspace_bytes(int64_t M, int K, int N);
hipError_t launch_out_proj(const void *x, const void *w, void *out, int64_t M, int K, int N, int out_bf16,
                           void *ws, hipStream_t s);
// The allocation-free projection's static scratch: 16 MiB per device, enough for the fp32
// partials of up to 64 rows x 16,384 features with K split 4 ways.  *ptr is this
// device's address of it (taken once per device, with that device current).
constexpr size_t kOutProjStaticScratchBytes = size_t(16) << 20;
hipError_t out_proj_static_scratch(void **ptr);
hipError_t launch_prefill_valu(const Args &a, hipStream_t s);
// bf16 chunked prefill, d = 128: the per-chunk preparation (writes one record per
// (slot, head) into ws), then the state scan that reads them.
size_t chunk_prep_workspace_bytes(long long B, long long T, long long H, long long N, bool packed);
uint64_t *chunk_exchange_words(const void *ws, long long B, long long T, long long H, long long N, bool packed);
uint32_t *chunk_status_word(const void *ws, long long B, long long T, long long H, long long N, bool packed);
hipError_t launch_chunk_prep(const Args &a, void *ws, hipStream_t s);
// With a.y set the scan also applies the gated norm (a.gate, a.norm_w, a.eps).  With
// a.states_out set (and no a.y, no convolution) it also stores each chunk's U rows in the
// workspace area after the prefill's own (chunk_states_u_area) and the state after each
// chunk's last position into a.states_out; launch_chunk_states then fills the others.
hipError_t launch_chunk_scan(const Args &a, const void *ws, hipStream_t s);
// The per-token states' workspace area: fp32 U rows, 32 x 128 per (slot, head).
size_t chunk_states_u_bytes(long long B, long long T, long long H, long long N, bool packed);
float *chunk_states_u_area(const void *ws, long long B, long long T, long long H, long long N, bool packed);
hipError_t launch_chunk_states(const Args &a, const void *ws, hipStream_t s);
// With tok_end (a device pointer to the end of the last packed sequence), rows of tokens
// at or past it (row / heads >= *tok_end) are left untouched.
hipError_t launch_gated_rmsnorm(const void *x, const void *gate, const float *w, void *y,
                                int64_t rows, int width, float eps, int x_bf16, int gate_bf16,
                                int out_bf16, hipStream_t s, const int32_t *tok_end = nullptr, int heads = 1);

// Shape support of each kernel family.
bool recurrent_supports(int dk, int dv);
bool prefill_valu_supports(int dk, int dv);
bool prefill_mfma_supports(int dk, int dv, int in_bf16);
bool prefill_mfma_fits(long long T, long long H);

}  // namespace kda
