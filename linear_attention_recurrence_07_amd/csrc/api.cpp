// C ABI of libkda.so: host-side validation and dispatch to the HIP kernels.
// Every check runs before anything is enqueued, so a non-OK status leaves all outputs
// untouched.  See include/kda.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/kda.h"
#include "kda_launch.h"

namespace {

thread_local char g_last_error[512] = "";

kda_status_t fail(kda_status_t s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

// Tensors with a feature axis are read and written in 16-byte vectors; per-token
// scalars (beta, mask, cu_seqlens) only need their element alignment.
kda_status_t check_ptr(const void *p, const char *name, bool required, unsigned align = 16) {
  if (p == nullptr) {
    if (required) return fail(KDA_ERR_NULL, "%s is NULL", name);
    return KDA_OK;
  }
  if ((reinterpret_cast<uintptr_t>(p) & (align - 1u)) != 0)
    return fail(KDA_ERR_ALIGN, "%s is not %u-byte aligned", name, align);
  return KDA_OK;
}

#define KDA_TRY(expr)                      \
  do {                                     \
    const kda_status_t s_ = (expr);        \
    if (s_ != KDA_OK) return s_;           \
  } while (0)

bool valid_dtype(int32_t d) { return d == KDA_F32 || d == KDA_BF16; }

// Shared validation of the problem description.
kda_status_t check_params(const kda_params_t *p, bool prefill) {
  if (p == nullptr) return fail(KDA_ERR_NULL, "params is NULL");
  if (p->B <= 0 || p->T < 0 || p->H <= 0 || p->dk <= 0 || p->dv <= 0)
    return fail(KDA_ERR_SHAPE, "bad sizes B=%d T=%d H=%d dk=%d dv=%d", p->B, p->T, p->H, p->dk, p->dv);
  if (!valid_dtype(p->in_dtype) || !valid_dtype(p->out_dtype))
    return fail(KDA_ERR_DTYPE, "unknown dtype code in=%d out=%d", p->in_dtype, p->out_dtype);
  if (!(p->scale >= 0.f) || !std::isfinite(p->scale)) return fail(KDA_ERR_SHAPE, "scale must be finite and >= 0");
  if (!(p->norm_eps >= 0.f) || !std::isfinite(p->norm_eps)) return fail(KDA_ERR_SHAPE, "norm_eps must be finite and >= 0");
  if (p->use_qk_l2norm != 0 && p->use_qk_l2norm != 1) return fail(KDA_ERR_SHAPE, "use_qk_l2norm must be 0 or 1");
  if (p->decay_per_head != 0 && p->decay_per_head != 1) return fail(KDA_ERR_SHAPE, "decay_per_head must be 0 or 1");
  if (prefill && p->chunk != 0 && p->chunk != 16 && p->chunk != 32 && p->chunk != 64)
    return fail(KDA_ERR_UNSUPPORTED, "chunk %d not supported (0, 16, 32 or 64)", p->chunk);
  // Element counts must stay addressable with 32-bit token indices times heads.
  const double toks = static_cast<double>(p->B) * p->T * p->H;
  if (toks * p->dk > 9.0e18 || static_cast<double>(p->B) * p->T > 2147483647.0)
    return fail(KDA_ERR_SHAPE, "problem too large");
  return KDA_OK;
}

// The bf16 matrix-core prefill runs when the shape and dtype allow it and the caller did
// not ask for the 16-token vector-ALU chunks.  Its blocks are 32 tokens; a 64-token chunk
// (the length the pages name) is carried as its two 32-token halves, the same chunked
// form regrouped, so chunk 64 selects it as well.
bool use_mfma_prefill(const kda_params_t *p) {
  return kda::prefill_mfma_supports(p->dk, p->dv, p->in_dtype == KDA_BF16) &&
         (p->chunk == 0 || p->chunk == 32 || p->chunk == 64) && kda::prefill_mfma_fits(p->T, p->H);
}

size_t prefill_workspace(const kda_params_t *p, bool packed) {
  if (!use_mfma_prefill(p)) return 0;
  return kda::chunk_prep_workspace_bytes(p->B, p->T, p->H, packed ? p->num_seqs : p->B, packed);
}

kda::Args make_args(const kda_params_t *p) {
  kda::Args a{};
  a.B = p->B;
  a.T = p->T;
  a.H = p->H;
  a.dk = p->dk;
  a.dv = p->dv;
  a.N = p->B;
  a.scale = p->scale > 0.f ? p->scale : 1.0f / std::sqrt(static_cast<float>(p->dk));
  a.eps = p->norm_eps;
  a.use_l2 = p->use_qk_l2norm;
  a.in_bf16 = p->in_dtype == KDA_BF16;
  a.out_bf16 = p->out_dtype == KDA_BF16;
  a.g_head = p->decay_per_head;
  return a;
}

kda_status_t check_norm(const void *gate, const float *w, void *y, int dv) {
  const int set = (gate != nullptr) + (w != nullptr) + (y != nullptr);
  if (set != 0 && set != 3) return fail(KDA_ERR_CONFLICT, "gate, norm_weight and y must be all set or all NULL");
  if (set == 3) {
    KDA_TRY(check_ptr(gate, "gate", true));
    KDA_TRY(check_ptr(w, "norm_weight", true));
    KDA_TRY(check_ptr(y, "y", true));
    if (dv < 8 || dv > 512 || (dv & (dv - 1)) != 0)
      return fail(KDA_ERR_UNSUPPORTED, "gated norm width %d must be a power of two in [8, 512]", dv);
  }
  return KDA_OK;
}

kda_status_t hip_status(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(KDA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return KDA_OK;
}

// Packed offsets or a padding mask, and the sequence count that goes with them.
kda_status_t check_layout(const kda_params_t *p, const int32_t *cu, const uint8_t *mask) {
  KDA_TRY(check_ptr(cu, "cu_seqlens", false, 4));
  KDA_TRY(check_ptr(mask, "mask", false, 1));
  if (cu && mask) return fail(KDA_ERR_CONFLICT, "give cu_seqlens or mask, not both");
  if (cu && p->B != 1) return fail(KDA_ERR_CONFLICT, "cu_seqlens needs B == 1 (packed batch)");
  if (cu && p->num_seqs <= 0) return fail(KDA_ERR_SHAPE, "num_seqs must be > 0 with cu_seqlens");
  return KDA_OK;
}

// The two stages exist only for the bf16, d = 128 matrix-core kernel.
kda_status_t check_stage_kernel(const kda_params_t *p) {
  if (!use_mfma_prefill(p))
    return fail(KDA_ERR_UNSUPPORTED, "the two-stage prefill needs bf16 inputs, dk = dv = 128, chunk 0, 32 or 64 "
                                     "and T * H * 128 < 2^31");
  return KDA_OK;
}

// The per-token states also keep each chunk's U rows (16 KB per chunk and head).
size_t prefill_states_workspace(const kda_params_t *p, bool packed) {
  if (!use_mfma_prefill(p)) return 0;
  const int N = packed ? p->num_seqs : p->B;
  return prefill_workspace(p, packed) + kda::chunk_states_u_bytes(p->B, p->T, p->H, N, packed);
}

kda_status_t check_workspace(const kda_params_t *p, const int32_t *cu, const void *ws, size_t bytes,
                             bool states = false) {
  const size_t need = states ? prefill_states_workspace(p, cu != nullptr) : prefill_workspace(p, cu != nullptr);
  if (bytes < need || (need > 0 && ws == nullptr))
    return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, bytes,
                ws == nullptr ? " (NULL)" : "");
  return check_ptr(ws, "workspace", false);
}

// The fused short convolution: filter width and activation, taps of q, k and v, and the
// optional carried inputs before and after the call.
kda_status_t check_conv(const kda_conv_t *c, const kda_params_t *p, int N) {
  if (c == nullptr) return fail(KDA_ERR_NULL, "conv is NULL");
  if (c->activation != 0 && c->activation != 1) return fail(KDA_ERR_SHAPE, "conv activation must be 0 or 1");
  if (c->width < 2 || c->width > 4) return fail(KDA_ERR_UNSUPPORTED, "conv width %d not in 2..4", c->width);
  KDA_TRY(check_ptr(c->weight_q, "conv weight_q", true));
  KDA_TRY(check_ptr(c->weight_k, "conv weight_k", true));
  KDA_TRY(check_ptr(c->weight_v, "conv weight_v", true));
  KDA_TRY(check_ptr(c->initial_q, "conv initial_q", false));
  KDA_TRY(check_ptr(c->initial_k, "conv initial_k", false));
  KDA_TRY(check_ptr(c->initial_v, "conv initial_v", false));
  KDA_TRY(check_ptr(c->final_q, "conv final_q", false));
  KDA_TRY(check_ptr(c->final_k, "conv final_k", false));
  KDA_TRY(check_ptr(c->final_v, "conv final_v", false));
  if (p->dk != p->dv) return fail(KDA_ERR_UNSUPPORTED, "the fused convolution needs dk == dv");
  if (N > 65535) return fail(KDA_ERR_UNSUPPORTED, "the fused convolution takes at most 65535 sequences");
  return KDA_OK;
}

void set_conv(kda::Args &a, const kda_conv_t *c) {
  a.conv.W = c->width;
  a.conv.silu = c->activation;
  a.conv.w[0] = c->weight_q; a.conv.w[1] = c->weight_k; a.conv.w[2] = c->weight_v;
  a.conv.init[0] = c->initial_q; a.conv.init[1] = c->initial_k; a.conv.init[2] = c->initial_v;
  a.conv.fin[0] = c->final_q; a.conv.fin[1] = c->final_k; a.conv.fin[2] = c->final_v;
}

// Shared body of kda_chunk_prefill (conv NULL), kda_chunk_prefill_conv and
// kda_chunk_prefill_states (with_states).
kda_status_t prefill_impl(const kda_params_t *p, const kda_conv_t *conv, bool with_conv, const void *q,
                          const void *k, const void *v, const float *g, const float *beta,
                          const float *initial_state, const int32_t *cu_seqlens, const uint8_t *mask, void *o,
                          float *final_state, const void *gate, const float *norm_weight, void *y,
                          void *workspace, size_t workspace_bytes, void *stream, bool with_states = false,
                          float *states = nullptr) {
  KDA_TRY(check_params(p, true));
  KDA_TRY(check_ptr(q, "q", true));
  KDA_TRY(check_ptr(k, "k", true));
  KDA_TRY(check_ptr(v, "v", true));
  KDA_TRY(check_ptr(g, "g", true, p->decay_per_head ? 4u : 16u));
  KDA_TRY(check_ptr(beta, "beta", true, 4));
  KDA_TRY(check_ptr(o, "o", y == nullptr || with_states));   // optional when y is wanted (not with states)
  if (with_states) KDA_TRY(check_ptr(states, "states", true));
  KDA_TRY(check_ptr(final_state, "final_state", true));
  KDA_TRY(check_ptr(initial_state, "initial_state", false));
  KDA_TRY(check_layout(p, cu_seqlens, mask));
  KDA_TRY(check_norm(gate, norm_weight, y, p->dv));
  kda::Args a = make_args(p);
  a.N = cu_seqlens ? p->num_seqs : p->B;
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.init = initial_state; a.state = final_state;
  a.cu = cu_seqlens; a.mask = mask; a.o = o;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int chunk = p->chunk;
  const bool mfma = use_mfma_prefill(p);
  if (with_conv) {
    KDA_TRY(check_conv(conv, p, a.N));
    if (!mfma)
      return fail(KDA_ERR_UNSUPPORTED, "the fused convolution runs in the bf16, dk = dv = 128 matrix-core prefill "
                                       "(chunk 0, 32 or 64); for other shapes run kda_short_conv first");
    set_conv(a, conv);
  }
  if (with_states && !mfma)
    return fail(KDA_ERR_UNSUPPORTED, "the chunked per-token states need bf16 inputs, dk = dv = 128, chunk 0, 32 or "
                                     "64 and T * H * 128 < 2^31; kda_recurrent_states covers other shapes");
  if (!mfma) {
    if (!kda::prefill_valu_supports(p->dk, p->dv))
      return fail(KDA_ERR_UNSUPPORTED, "no prefill kernel for dk=%d dv=%d", p->dk, p->dv);
    if (chunk == 32 || chunk == 64)
      return fail(KDA_ERR_UNSUPPORTED, "chunk %d needs bf16 inputs with dk = dv = 128 and T * H * 128 < 2^31",
                  chunk);
  }
  if (mfma) {
    // The gated norm runs as its own launch over the head outputs: the scan can apply it
    // itself (kda_chunk_scan with y), but on the scan's 2 work-groups per head that costs
    // more than a separate pass at full HBM bandwidth on every CU, and it needs waits
    // between work-groups.  With y alone, the head outputs are written into y and
    // normalised there, in place.
    KDA_TRY(check_workspace(p, cu_seqlens, workspace, workspace_bytes, with_states));
    KDA_TRY(hip_status(kda::launch_chunk_prep(a, workspace, st), "prefill (chunk preparation)"));
    void *out = o != nullptr ? o : y;
    a.o = out;
    a.states_out = states;
    KDA_TRY(hip_status(kda::launch_chunk_scan(a, workspace, st), "prefill (state scan)"));
    if (with_states) KDA_TRY(hip_status(kda::launch_chunk_states(a, workspace, st), "per-token states"));
    if (y != nullptr) {
      const int64_t rows = static_cast<int64_t>(p->B) * p->T * p->H;
      const int32_t *tok_end = cu_seqlens ? cu_seqlens + a.N : nullptr;   // tokens past it are not written
      KDA_TRY(hip_status(kda::launch_gated_rmsnorm(out, gate, norm_weight, y, rows, p->dv, p->norm_eps,
                                                   a.out_bf16, a.in_bf16, a.out_bf16, st, tok_end, p->H),
                         "gated norm"));
    }
    // the carried inputs after the call, once every kernel that reads the old ones is done
    if (with_conv) KDA_TRY(hip_status(kda::launch_conv_carry(a, st), "carried convolution inputs"));
  } else {
    a.gate = gate; a.norm_w = norm_weight; a.y = y;
    KDA_TRY(hip_status(kda::launch_prefill_valu(a, st), "prefill (VALU)"));
  }
  return KDA_OK;
}

}  // namespace

extern "C" {

kda_status_t kda_chunk_prefill(const kda_params_t *p, const void *q, const void *k, const void *v,
                               const float *g, const float *beta, const float *initial_state,
                               const int32_t *cu_seqlens, const uint8_t *mask, void *o,
                               float *final_state, const void *gate, const float *norm_weight,
                               void *y, void *workspace, size_t workspace_bytes, void *stream) {
  return prefill_impl(p, nullptr, false, q, k, v, g, beta, initial_state, cu_seqlens, mask, o, final_state, gate,
                      norm_weight, y, workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_prefill_conv(const kda_params_t *p, const kda_conv_t *conv, const void *q, const void *k,
                                    const void *v, const float *g, const float *beta, const float *initial_state,
                                    const int32_t *cu_seqlens, const uint8_t *mask, void *o, float *final_state,
                                    const void *gate, const float *norm_weight, void *y, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  return prefill_impl(p, conv, true, q, k, v, g, beta, initial_state, cu_seqlens, mask, o, final_state, gate,
                      norm_weight, y, workspace, workspace_bytes, stream);
}

kda_status_t kda_chunk_prefill_states(const kda_params_t *p, const void *q, const void *k, const void *v,
                                      const float *g, const float *beta, const float *initial_state,
                                      const int32_t *cu_seqlens, const uint8_t *mask, void *o,
                                      float *final_state, const void *gate, const float *norm_weight, void *y,
                                      float *states, void *workspace, size_t workspace_bytes, void *stream) {
  return prefill_impl(p, nullptr, false, q, k, v, g, beta, initial_state, cu_seqlens, mask, o, final_state, gate,
                      norm_weight, y, workspace, workspace_bytes, stream, true, states);
}

size_t kda_chunk_prefill_states_workspace_size(const kda_params_t *p, int32_t packed) {
  if (p == nullptr || check_params(p, true) != KDA_OK) return 0;
  if (packed && p->num_seqs <= 0) return 0;
  return prefill_states_workspace(p, packed != 0);
}

size_t kda_chunk_prefill_workspace_size(const kda_params_t *p, int32_t packed) {
  if (p == nullptr || check_params(p, true) != KDA_OK) return 0;
  if (packed && p->num_seqs <= 0) return 0;
  return prefill_workspace(p, packed != 0);
}

kda_status_t kda_chunk_prefill_status(const kda_params_t *p, int32_t packed, const void *workspace,
                                      size_t workspace_bytes, void *stream) {
  KDA_TRY(check_params(p, true));
  if (packed && p->num_seqs <= 0) return fail(KDA_ERR_SHAPE, "num_seqs must be > 0 with packing");
  KDA_TRY(check_stage_kernel(p));
  const size_t need = prefill_workspace(p, packed != 0);
  if (workspace == nullptr) return fail(KDA_ERR_NULL, "workspace is NULL");
  if (workspace_bytes < need) return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                                          workspace_bytes);
  KDA_TRY(check_ptr(workspace, "workspace", true));
  const uint32_t *word = kda::chunk_status_word(workspace, p->B, p->T, p->H, packed ? p->num_seqs : p->B, packed != 0);
  uint32_t flag = 0;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  KDA_TRY(hip_status(hipMemcpyAsync(&flag, word, sizeof flag, hipMemcpyDeviceToHost, st), "status read"));
  KDA_TRY(hip_status(hipStreamSynchronize(st), "status read"));
  if (flag != 0)
    return fail(KDA_ERR_TIMEOUT, "a wait between the two column tiles of a head ran out: y holds NaN for the "
                                 "tokens after it");
  return KDA_OK;
}

kda_status_t kda_chunk_prepare(const kda_params_t *p, const void *q, const void *k, const float *g,
                               const float *beta, const int32_t *cu_seqlens, const uint8_t *mask,
                               void *workspace, size_t workspace_bytes, void *stream) {
  KDA_TRY(check_params(p, true));
  KDA_TRY(check_ptr(q, "q", true));
  KDA_TRY(check_ptr(k, "k", true));
  KDA_TRY(check_ptr(g, "g", true, p->decay_per_head ? 4u : 16u));
  KDA_TRY(check_ptr(beta, "beta", true, 4));
  KDA_TRY(check_layout(p, cu_seqlens, mask));
  KDA_TRY(check_stage_kernel(p));
  KDA_TRY(check_workspace(p, cu_seqlens, workspace, workspace_bytes));
  kda::Args a = make_args(p);
  a.N = cu_seqlens ? p->num_seqs : p->B;
  a.q = q; a.k = k; a.g = g; a.beta = beta;
  a.cu = cu_seqlens; a.mask = mask;
  KDA_TRY(hip_status(kda::launch_chunk_prep(a, workspace, static_cast<hipStream_t>(stream)),
                     "chunk preparation"));
  return KDA_OK;
}

kda_status_t kda_chunk_scan(const kda_params_t *p, const void *v, const float *initial_state,
                            const int32_t *cu_seqlens, const void *workspace, size_t workspace_bytes,
                            void *o, float *final_state, const void *gate, const float *norm_weight,
                            void *y, void *stream) {
  KDA_TRY(check_params(p, true));
  KDA_TRY(check_ptr(v, "v", true));
  KDA_TRY(check_ptr(o, "o", y == nullptr));   // optional when y is wanted
  KDA_TRY(check_ptr(final_state, "final_state", true));
  KDA_TRY(check_ptr(initial_state, "initial_state", false));
  KDA_TRY(check_layout(p, cu_seqlens, nullptr));
  KDA_TRY(check_norm(gate, norm_weight, y, p->dv));
  KDA_TRY(check_stage_kernel(p));
  KDA_TRY(check_workspace(p, cu_seqlens, workspace, workspace_bytes));
  kda::Args a = make_args(p);
  a.N = cu_seqlens ? p->num_seqs : p->B;
  a.v = v; a.init = initial_state; a.state = final_state;
  a.cu = cu_seqlens; a.o = o;
  a.gate = gate; a.norm_w = norm_weight; a.y = y;
  KDA_TRY(hip_status(kda::launch_chunk_scan(a, workspace, static_cast<hipStream_t>(stream)), "state scan"));
  return KDA_OK;
}

// Shared body of the token-by-token entry points (conv: the fused convolution, or NULL).
static kda_status_t recurrent_impl(const kda_params_t *p, const kda_conv_t *conv, bool with_conv, const void *q,
                                   const void *k, const void *v, const float *g, const float *beta, float *state,
                                   const uint8_t *mask, void *o, const void *gate, const float *norm_weight,
                                   void *y, float *states, void *stream) {
  KDA_TRY(check_params(p, false));
  KDA_TRY(check_ptr(q, "q", true));
  KDA_TRY(check_ptr(k, "k", true));
  KDA_TRY(check_ptr(v, "v", true));
  KDA_TRY(check_ptr(g, "g", true, p->decay_per_head ? 4u : 16u));
  KDA_TRY(check_ptr(beta, "beta", true, 4));
  KDA_TRY(check_ptr(state, "state", true));
  KDA_TRY(check_ptr(o, "o", true));
  KDA_TRY(check_ptr(mask, "mask", false, 1));
  KDA_TRY(check_norm(gate, norm_weight, y, p->dv));
  if (!kda::recurrent_supports(p->dk, p->dv))
    return fail(KDA_ERR_UNSUPPORTED, "no recurrent kernel for dk=%d dv=%d", p->dk, p->dv);
  if (with_conv) KDA_TRY(check_conv(conv, p, p->B));
  kda::Args a = make_args(p);
  a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
  a.state = state; a.mask = mask; a.o = o;
  a.gate = gate; a.norm_w = norm_weight; a.y = y;
  a.states_out = states;
  if (with_conv) set_conv(a, conv);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (p->T == 0) {
    // no token: the carried inputs stay as they were (copied when the buffers differ)
    if (with_conv) KDA_TRY(hip_status(kda::launch_conv_carry(a, st), "carried convolution inputs"));
    return KDA_OK;
  }
  KDA_TRY(hip_status(kda::launch_recurrent(a, st), "recurrent step"));
  return KDA_OK;
}

kda_status_t kda_recurrent_step(const kda_params_t *p, const void *q, const void *k, const void *v,
                                const float *g, const float *beta, float *state,
                                const uint8_t *mask, void *o, const void *gate,
                                const float *norm_weight, void *y, void *stream) {
  return recurrent_impl(p, nullptr, false, q, k, v, g, beta, state, mask, o, gate, norm_weight, y, nullptr, stream);
}

kda_status_t kda_recurrent_step_conv(const kda_params_t *p, const kda_conv_t *conv, const void *q, const void *k,
                                     const void *v, const float *g, const float *beta, float *state,
                                     const uint8_t *mask, void *o, const void *gate, const float *norm_weight,
                                     void *y, void *stream) {
  return recurrent_impl(p, conv, true, q, k, v, g, beta, state, mask, o, gate, norm_weight, y, nullptr, stream);
}

kda_status_t kda_recurrent_states(const kda_params_t *p, const void *q, const void *k, const void *v,
                                  const float *g, const float *beta, float *state,
                                  const uint8_t *mask, void *o, const void *gate,
                                  const float *norm_weight, void *y, float *states, void *stream) {
  KDA_TRY(check_ptr(states, "states", true));
  return recurrent_impl(p, nullptr, false, q, k, v, g, beta, state, mask, o, gate, norm_weight, y, states, stream);
}

kda_status_t kda_gated_rmsnorm(const void *x, const void *gate, const float *weight, void *y,
                               int64_t rows, int32_t width, float eps, int32_t in_dtype,
                               int32_t out_dtype, void *stream) {
  KDA_TRY(check_ptr(x, "x", true));
  KDA_TRY(check_ptr(gate, "gate", true));
  KDA_TRY(check_ptr(weight, "weight", true));
  KDA_TRY(check_ptr(y, "y", true));
  if (rows < 0) return fail(KDA_ERR_SHAPE, "rows must be >= 0");
  if (width < 8 || width > 512 || (width & (width - 1)) != 0)
    return fail(KDA_ERR_UNSUPPORTED, "width %d must be a power of two in [8, 512]", width);
  if (!valid_dtype(in_dtype) || !valid_dtype(out_dtype))
    return fail(KDA_ERR_DTYPE, "unknown dtype code in=%d out=%d", in_dtype, out_dtype);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(KDA_ERR_SHAPE, "eps must be finite and >= 0");
  if (rows / 256 > 2147483647LL) return fail(KDA_ERR_SHAPE, "too many rows");
  const int bf = in_dtype == KDA_BF16;
  KDA_TRY(hip_status(kda::launch_gated_rmsnorm(x, gate, weight, y, rows, width, eps, bf, bf,
                                               out_dtype == KDA_BF16, static_cast<hipStream_t>(stream)),
                     "gated norm"));
  return KDA_OK;
}

kda_status_t kda_short_conv(const kda_conv_params_t *p, const void *x, const float *weight,
                            const void *initial_state, const int32_t *cu_seqlens, const uint8_t *mask,
                            void *y, void *final_state, void *stream) {
  if (p == nullptr) return fail(KDA_ERR_NULL, "params is NULL");
  if (p->B <= 0 || p->T < 0 || p->D <= 0)
    return fail(KDA_ERR_SHAPE, "bad sizes B=%d T=%d D=%d", p->B, p->T, p->D);
  if (!valid_dtype(p->in_dtype) || !valid_dtype(p->out_dtype))
    return fail(KDA_ERR_DTYPE, "unknown dtype code in=%d out=%d", p->in_dtype, p->out_dtype);
  if (p->activation != 0 && p->activation != 1) return fail(KDA_ERR_SHAPE, "activation must be 0 or 1");
  KDA_TRY(check_ptr(x, "x", true));
  KDA_TRY(check_ptr(weight, "weight", true, 4));
  KDA_TRY(check_ptr(y, "y", true));
  KDA_TRY(check_ptr(initial_state, "initial_state", false));
  KDA_TRY(check_ptr(final_state, "final_state", false));
  KDA_TRY(check_ptr(cu_seqlens, "cu_seqlens", false, 4));
  KDA_TRY(check_ptr(mask, "mask", false, 1));
  if (cu_seqlens && mask) return fail(KDA_ERR_CONFLICT, "give cu_seqlens or mask, not both");
  if (cu_seqlens && p->B != 1) return fail(KDA_ERR_CONFLICT, "cu_seqlens needs B == 1 (packed batch)");
  if (cu_seqlens && p->num_seqs <= 0) return fail(KDA_ERR_SHAPE, "num_seqs must be > 0 with cu_seqlens");
  if (p->D % 8 != 0) return fail(KDA_ERR_UNSUPPORTED, "D=%d must be a multiple of 8", p->D);
  if (p->width < 2 || p->width > 4) return fail(KDA_ERR_UNSUPPORTED, "width %d not in 2..4", p->width);
  const int N = cu_seqlens ? p->num_seqs : p->B;
  if (p->B > 65535 || N > 65535 || (p->T + 63) / 64 > 65535)
    return fail(KDA_ERR_UNSUPPORTED, "more than 65535 rows, sequences or 64-token tiles");
  const double elems = static_cast<double>(p->B) * p->T * p->D;
  if (elems * 4 > 9.0e18) return fail(KDA_ERR_SHAPE, "problem too large");
  const uintptr_t xs = reinterpret_cast<uintptr_t>(x), ys = reinterpret_cast<uintptr_t>(y);
  const uintptr_t xb = static_cast<uintptr_t>(elems) * (p->in_dtype == KDA_BF16 ? 2u : 4u);
  const uintptr_t yb = static_cast<uintptr_t>(elems) * (p->out_dtype == KDA_BF16 ? 2u : 4u);
  if (elems > 0 && xs < ys + yb && ys < xs + xb) return fail(KDA_ERR_CONFLICT, "y overlaps x");
  kda::ConvArgs a{};
  a.x = x; a.w = weight; a.init = initial_state; a.cu = cu_seqlens; a.mask = mask;
  a.y = y; a.fin = final_state;
  a.B = p->B; a.T = p->T; a.D = p->D; a.N = N; a.W = p->width; a.silu = p->activation;
  a.in_bf16 = p->in_dtype == KDA_BF16;
  a.out_bf16 = p->out_dtype == KDA_BF16;
  KDA_TRY(hip_status(kda::launch_short_conv(a, static_cast<hipStream_t>(stream)), "short convolution"));
  return KDA_OK;
}

static kda_status_t check_proj_workspace(int64_t rows, int K, int N, const void *ws, size_t bytes) {
  const size_t need = kda::out_proj_workspace_bytes(rows, K, N);
  if (bytes < need || (need > 0 && ws == nullptr))
    return fail(KDA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", need, bytes,
                ws == nullptr ? " (NULL)" : "");
  return check_ptr(ws, "workspace", false);
}

size_t kda_out_proj_workspace_size(int64_t rows, int32_t in_features, int32_t out_features) {
  if (rows < 0 || in_features <= 0 || out_features <= 0 || !kda::out_proj_supports(rows, in_features, out_features))
    return 0;
  return kda::out_proj_workspace_bytes(rows, in_features, out_features);
}

kda_status_t kda_out_proj(const void *x, const void *weight, void *out, int64_t rows, int32_t in_features,
                          int32_t out_features, int32_t out_dtype, void *workspace, size_t workspace_bytes,
                          void *stream) {
  KDA_TRY(check_ptr(x, "x", true));
  KDA_TRY(check_ptr(weight, "weight", true));
  KDA_TRY(check_ptr(out, "out", true));
  if (rows < 0 || in_features <= 0 || out_features <= 0)
    return fail(KDA_ERR_SHAPE, "bad sizes rows=%lld in=%d out=%d", static_cast<long long>(rows), in_features,
                out_features);
  if (!valid_dtype(out_dtype)) return fail(KDA_ERR_DTYPE, "unknown dtype code %d", out_dtype);
  if (!kda::out_proj_supports(rows, in_features, out_features))
    return fail(KDA_ERR_UNSUPPORTED, "in_features %% 256, out_features %% 64 must be 0 and rows <= 65535 * 64");
  KDA_TRY(check_proj_workspace(rows, in_features, out_features, workspace, workspace_bytes));
  KDA_TRY(hip_status(kda::launch_out_proj(x, weight, out, rows, in_features, out_features, out_dtype == KDA_BF16,
                                          workspace, static_cast<hipStream_t>(stream)),
                     "output projection"));
  return KDA_OK;
}

// Shared validation of the layer-exit entry points (everything but the workspace).
static kda_status_t check_norm_proj(const void *o, const void *gate, const float *norm_weight,
                                    const void *proj_weight, void *y, void *out, int64_t rows, int32_t heads,
                                    int32_t head_dim, int32_t out_features, float eps, int32_t out_dtype) {
  KDA_TRY(check_ptr(o, "o", true));
  KDA_TRY(check_ptr(gate, "gate", true));
  KDA_TRY(check_ptr(norm_weight, "norm_weight", true));
  KDA_TRY(check_ptr(proj_weight, "proj_weight", true));
  KDA_TRY(check_ptr(y, "y", true));
  KDA_TRY(check_ptr(out, "out", true));
  if (rows < 0 || heads <= 0 || head_dim <= 0 || out_features <= 0)
    return fail(KDA_ERR_SHAPE, "bad sizes rows=%lld heads=%d head_dim=%d out=%d", static_cast<long long>(rows),
                heads, head_dim, out_features);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(KDA_ERR_SHAPE, "eps must be finite and >= 0");
  if (!valid_dtype(out_dtype)) return fail(KDA_ERR_DTYPE, "unknown dtype code %d", out_dtype);
  if (head_dim < 8 || head_dim > 512 || (head_dim & (head_dim - 1)) != 0)
    return fail(KDA_ERR_UNSUPPORTED, "head_dim %d must be a power of two in [8, 512]", head_dim);
  const int64_t K = static_cast<int64_t>(heads) * head_dim;
  if (K > 0x7fffffff || !kda::out_proj_supports(rows, static_cast<int>(K), out_features))
    return fail(KDA_ERR_UNSUPPORTED, "heads * head_dim %% 256, out_features %% 64 must be 0 and rows <= 65535 * 64");
  if (rows * heads / 256 > 2147483647LL) return fail(KDA_ERR_SHAPE, "too many rows");
  return KDA_OK;
}

kda_status_t kda_gated_norm_proj_noalloc(const void *o, const void *gate, const float *norm_weight,
                                         const void *proj_weight, void *y, void *out, int64_t rows, int32_t heads,
                                         int32_t head_dim, int32_t out_features, float eps, int32_t out_dtype,
                                         void *stream) {
  KDA_TRY(check_norm_proj(o, gate, norm_weight, proj_weight, y, out, rows, heads, head_dim, out_features, eps,
                          out_dtype));
  const int K = heads * head_dim;
  const size_t need = kda::out_proj_workspace_bytes(rows, K, out_features);
  if (need > kda::kOutProjStaticScratchBytes)
    return fail(KDA_ERR_WORKSPACE, "the split-K partial sums need %zu bytes; the static scratch holds %zu "
                                   "(use kda_gated_norm_proj with a workspace)",
                need, kda::kOutProjStaticScratchBytes);
  void *scratch = nullptr;
  if (need > 0) KDA_TRY(hip_status(kda::out_proj_static_scratch(&scratch), "static scratch address"));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  KDA_TRY(hip_status(kda::launch_gated_rmsnorm(o, gate, norm_weight, y, rows * heads, head_dim, eps, 1, 1, 1, st),
                     "gated norm"));
  KDA_TRY(hip_status(kda::launch_out_proj(y, proj_weight, out, rows, K, out_features, out_dtype == KDA_BF16,
                                          scratch, st),
                     "output projection"));
  return KDA_OK;
}

kda_status_t kda_gated_norm_proj(const void *o, const void *gate, const float *norm_weight,
                                 const void *proj_weight, void *y, void *out, int64_t rows, int32_t heads,
                                 int32_t head_dim, int32_t out_features, float eps, int32_t out_dtype,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  KDA_TRY(check_norm_proj(o, gate, norm_weight, proj_weight, y, out, rows, heads, head_dim, out_features, eps,
                          out_dtype));
  const int64_t K = static_cast<int64_t>(heads) * head_dim;
  KDA_TRY(check_proj_workspace(rows, static_cast<int>(K), out_features, workspace, workspace_bytes));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  KDA_TRY(hip_status(kda::launch_gated_rmsnorm(o, gate, norm_weight, y, rows * heads, head_dim, eps, 1, 1, 1, st),
                     "gated norm"));
  KDA_TRY(hip_status(kda::launch_out_proj(y, proj_weight, out, rows, static_cast<int>(K), out_features,
                                          out_dtype == KDA_BF16, workspace, st),
                     "output projection"));
  return KDA_OK;
}

const char *kda_status_string(kda_status_t s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN";
    case KDA_ERR_CONFLICT: return "KDA_ERR_CONFLICT";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE";
    case KDA_ERR_TIMEOUT: return "KDA_ERR_TIMEOUT";
  }
  return "KDA_ERR_UNKNOWN";
}

const char *kda_last_error(void) { return g_last_error; }

const char *kda_version(void) { return "kda-mi355x 0.1.0 gfx950"; }

}  // extern "C"
